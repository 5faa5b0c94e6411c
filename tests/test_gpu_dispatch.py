"""Pull gather and the push-dispatch baseline (the Telegram post on MoK, "Method and
experiments": push through contended per-expert slot counters and scattered writes, pull by
each expert reading its own tokens) against the oracle's plan.

Pull is fully determined: bit-exact rows in plan order. Push is not: the slot a route lands in
follows atomic arrival, so what is unique is compared (each expert's count and its set of
routes) and the rest is checked for validity (every written row is the token row of the route
recorded beside it; nothing is written past the capacity)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _layer import gpu_topk, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = {
    "small_bf16": dict(T=2048, d=256, k=8, E=64, e0=4, E_l=4, tpr=256, dtype=torch.bfloat16),
    "tiny_fp32": dict(T=64, d=128, k=2, E=8, e0=0, E_l=8, tpr=64, dtype=torch.float32),
    "ragged_bf16": dict(T=3000, d=384, k=6, E=40, e0=7, E_l=9, tpr=1000, dtype=torch.bfloat16),
    "ep64_share_bf16": dict(T=262144, d=7168, k=8, E=256, e0=0, E_l=4, tpr=4096,
                            dtype=torch.bfloat16),
}


def _setup(c):
    x = synth.normal_rows(0, 201, c["d"], range(c["T"]), 1.0, c["dtype"], DEV)
    logits = synth.normal_rows(0, 202, c["E"], range(c["T"]), 1.0, torch.float32, DEV)
    idx_g, _ = gpu_topk(logits, c["k"])
    idx, _ = oracle.topk(logits.cpu(), c["k"])
    assert np.array_equal(to_np(idx_g), idx)
    plan = oracle.dispatch_plan(idx, c["e0"], c["E_l"], c["tpr"])
    return x, idx_g, plan


def _gpu_plan(idx_g, c):
    import routing_grouped_expert_gemm_amd as mok
    T, k, E_l = c["T"], c["k"], c["E_l"]
    i32 = dict(dtype=torch.int32, device=DEV)
    counts, offsets = torch.empty(E_l, **i32), torch.empty(E_l + 1, **i32)
    rank_counts = torch.empty((E_l, T // c["tpr"]), **i32)
    route_ids = torch.empty(T * min(k, E_l), **i32)
    ws = torch.empty(mok.mok_dispatch_plan_workspace_bytes(T, k, E_l), dtype=torch.uint8, device=DEV)
    mok.mok_dispatch_plan(idx_g, c["E"], c["e0"], E_l, c["tpr"], counts, offsets, rank_counts,
                          route_ids, ws)
    return route_ids, offsets


@pytest.mark.parametrize("name", list(CASES))
def test_pull_gather_rows_in_plan_order(name):
    import routing_grouped_expert_gemm_amd as mok
    c = CASES[name]
    x, idx_g, plan = _setup(c)
    route_ids, offsets = _gpu_plan(idx_g, c)
    cap = c["T"] * min(c["k"], c["E_l"])
    buf = torch.full((cap, c["d"]), -3.0, dtype=c["dtype"], device=DEV)
    mok.mok_pull_gather(x, c["k"], route_ids, offsets, buf)
    torch.cuda.synchronize()
    n = plan["n"]
    ref = x[torch.from_numpy(plan["route_ids"] // c["k"]).long().to(DEV)]
    assert torch.equal(buf[:n], ref)
    assert bool((buf[n:] == -3.0).all())


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("cap_kind", ["whole", "tight"])
def test_push_dispatch_rows_and_routes(name, cap_kind):
    import routing_grouped_expert_gemm_amd as mok
    c = CASES[name]
    x, idx_g, plan = _setup(c)
    counts = plan["counts"]
    E_l, d, k = c["E_l"], c["d"], c["k"]
    # whole: room for every route; tight: half of the busiest expert's routes (drops)
    cap = int(max(1, counts.max())) if cap_kind == "whole" else int(max(1, counts.max() // 2))
    fill = torch.full((E_l,), 99, dtype=torch.int32, device=DEV)
    buf = torch.full((E_l, cap + 2, d), -3.0, dtype=c["dtype"], device=DEV)   # +2: canary rows
    src = torch.full((E_l, cap + 2), -7, dtype=torch.int32, device=DEV)
    # the capacity argument is cap; the two extra rows per expert must stay untouched
    T = c["T"]
    L = mok._lib
    rc = L.mok_push_dispatch(x.data_ptr(), T, d, k, mok._io(x), idx_g.data_ptr(), c["e0"], E_l,
                             cap, fill.data_ptr(), buf.data_ptr(), src.data_ptr(),
                             torch.cuda.current_stream().cuda_stream)
    assert rc == mok.MOK_OK
    # the library addresses buf / src with row stride cap: view them that way
    torch.cuda.synchronize()
    assert np.array_equal(to_np(fill), counts)
    flat_buf = buf.view(-1, d)
    flat_src = src.view(-1)
    for e in range(E_l):
        n_w = min(int(counts[e]), cap)
        got = to_np(flat_src[e * cap:e * cap + n_w]).astype(np.int64)
        routes = plan["route_ids"][plan["offsets"][e]:plan["offsets"][e + 1]].astype(np.int64)
        if n_w == counts[e]:
            assert np.array_equal(np.sort(got), routes), e
        else:                                   # drops: a subset of distinct routes of e
            assert len(np.unique(got)) == n_w and np.isin(got, routes).all(), e
        rows = flat_buf[e * cap:e * cap + n_w]
        ref = x[torch.from_numpy(got // k).to(DEV)]
        assert torch.equal(rows, ref), e
    # nothing past the capacity: the 2 * E_l canary entries at the end of the arrays
    assert bool((flat_src[E_l * cap:] == -7).all())
    assert bool((flat_buf[E_l * cap:] == -3.0).all())
