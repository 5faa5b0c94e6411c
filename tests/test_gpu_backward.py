"""Backward of the layer through the C ABI (mok_moe_backward) against the oracle's float64
backward (pinned by finite differences of the oracle's forward), on the same seeded inputs and
the same routing. Every gradient tensor must satisfy max|g - ref| / max|ref| <= 1e-2 (bf16
operands, float32 accumulation); reruns are bit-identical."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _layer import TOL, make_inputs, rel_err, to_np
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu
DEV = "cuda"
S_DY = 21      # stream id of the upstream gradients


def _routing(wl, inp):
    cpu = {k: (v.cpu() if v is not None else None) for k, v in inp.items()}
    if wl.routing == "router":
        logits = oracle.router_logits(cpu["x"], cpu["w_router"])
    else:
        logits = cpu["logits"].numpy()
    idx, w = oracle.topk(logits, wl.k)
    return cpu, idx, w


def _run(wl, inp, idx, w, cap=0):
    import routing_grouped_expert_gemm_amd as mok
    full = wl.full_layer
    kw = {}
    if full:
        kw["dy"] = synth.normal_rows(0, S_DY, wl.d, range(wl.T_pool), 1.0, torch.bfloat16, DEV)
    else:
        kw["dy_slots"] = synth.normal_rows(0, S_DY, wl.d, range(wl.T_pool * wl.k), 1.0,
                                           torch.bfloat16, DEV)
        if wl.n_shared:
            kw["dy_shared"] = synth.normal_rows(0, S_DY + 1, wl.d, range(wl.T_own), 1.0,
                                                torch.bfloat16, DEV)
    b = mok.MoeBackward(d=wl.d, E=wl.E, k=wl.k, I=wl.I, e0=wl.e0, E_l=wl.E_l,
                        tokens_per_rank=wl.tokens_per_rank, T_pool=wl.T_pool,
                        own_begin=wl.own_begin, T_own=wl.T_own, n_shared=wl.n_shared,
                        I_shared=wl.I_shared, x=inp["x"],
                        topk_idx=torch.from_numpy(idx).to(DEV),
                        topk_w=torch.from_numpy(w).to(DEV), w_gate=inp["wg"], w_up=inp["wu"],
                        w_down=inp["wd"], ws_gate=inp["sg"], ws_up=inp["su"], ws_down=inp["sd"],
                        route_rows_cap=cap, device=DEV, **kw)
    b.backward()
    torch.cuda.synchronize()
    assert b.device_error() == 0
    return b, kw


def _compare(wl, b, kw, cpu, idx, w, tol=None):
    tol = tol or TOL["bf16"]
    ckw = {k: v.cpu() for k, v in kw.items()}
    ref = oracle.moe_backward(wl, cpu["x"], idx, w, cpu["wg"], cpu["wu"], cpu["wd"], cpu["sg"],
                              cpu["su"], cpu["sd"], **ckw)
    rids = ref["plan"]["route_ids"].astype(np.int64)
    errs = {}
    if len(rids):
        errs["dx_slots"] = rel_err(to_np(b.dx_slots)[rids], ref["dx_slots"])
        errs["dtopk_w"] = rel_err(to_np(b.dtopk_w).reshape(-1)[rids], ref["dtopk_w"])
    for name, r in (("dw_gate", ref["dwg"]), ("dw_up", ref["dwu"]), ("dw_down", ref["dwd"])):
        errs[name] = rel_err(to_np(getattr(b, name)), r)
    if wl.n_shared:
        for name, r in (("dws_gate", ref["dsg"]), ("dws_up", ref["dsu"]), ("dws_down", ref["dsd"])):
            errs[name] = rel_err(to_np(getattr(b, name)), r)
        if wl.T_own:
            errs["dx_shared"] = rel_err(to_np(b.dx_shared), ref["dx_shared"])
    if wl.full_layer:
        errs["dx"] = rel_err(to_np(b.dx), ref["dx"])
    print(f"backward {wl.name}: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad
    return ref


@pytest.mark.parametrize("name", ["full_bf16", "share_bf16"])
def test_backward_small_matches_oracle(name):
    wl = SMALL[name]
    inp = make_inputs(wl, DEV)
    cpu, idx, w = _routing(wl, inp)
    b, kw = _run(wl, inp, idx, w)
    _compare(wl, b, kw, cpu, idx, w)


def test_backward_expert_without_routes_and_route_capacity():
    """A local expert no token picks gets an exactly zero weight gradient; a capacity that is
    just the plan's size works; one row short of it sets the overflow bit."""
    import routing_grouped_expert_gemm_amd as mok
    wl = synth.scaled(SMALL["share_bf16"], name="bwd_edge")
    inp = make_inputs(wl, DEV)
    rng = np.random.default_rng(5)
    allowed = np.array([e for e in range(wl.E) if e != wl.e0 + 1])
    idx = np.stack([rng.choice(allowed, wl.k, replace=False) for _ in range(wl.T_pool)]).astype(np.int32)
    w = rng.random((wl.T_pool, wl.k)).astype(np.float32) + 0.1
    w = (w / w.sum(1, keepdims=True)).astype(np.float32)
    cpu = {k: (v.cpu() if v is not None else None) for k, v in inp.items()}
    n = oracle.dispatch_plan(idx, wl.e0, wl.E_l, wl.tokens_per_rank)["n"]
    b, kw = _run(wl, inp, idx, w, cap=n)
    _compare(wl, b, kw, cpu, idx, w)
    assert float(b.dw_gate[1].abs().max()) == 0.0 and float(b.dw_down[1].abs().max()) == 0.0
    short = mok.MoeBackward(d=wl.d, E=wl.E, k=wl.k, I=wl.I, e0=wl.e0, E_l=wl.E_l,
                            tokens_per_rank=wl.tokens_per_rank, T_pool=wl.T_pool,
                            own_begin=wl.own_begin, T_own=wl.T_own, n_shared=wl.n_shared,
                            I_shared=wl.I_shared, x=inp["x"],
                            topk_idx=torch.from_numpy(idx).to(DEV),
                            topk_w=torch.from_numpy(w).to(DEV), w_gate=inp["wg"], w_up=inp["wu"],
                            w_down=inp["wd"], ws_gate=inp["sg"], ws_up=inp["su"],
                            ws_down=inp["sd"], route_rows_cap=n - 1, device=DEV, **kw)
    short.backward()
    torch.cuda.synchronize()
    assert short.device_error() == mok.MOK_DEVERR_OVERFLOW


def test_backward_reruns_bit_identical():
    wl = SMALL["full_bf16"]
    inp = make_inputs(wl, DEV)
    _, idx, w = _routing(wl, inp)
    b, _ = _run(wl, inp, idx, w)
    outs = lambda: [t.clone() for t in (b.dx, b.dx_shared, b.dtopk_w, b.dw_gate, b.dw_up,
                                        b.dw_down, b.dws_gate, b.dws_up, b.dws_down)]
    first = outs()
    for _ in range(4):
        b.backward()
        torch.cuda.synchronize()
        for a, c in zip(outs(), first):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               c.view(torch.int16) if c.dtype == torch.bfloat16 else c.view(torch.int32))


def test_backward_full_ep1_layer():
    """T=8192, d=2048, 64 experts top-6, I=1408, 2 shared experts: every gradient tensor of the
    whole layer against the oracle."""
    wl = synth.WORKLOADS[synth.EP1]
    inp = make_inputs(wl, DEV)
    cpu, idx, w = _routing(wl, inp)
    b, kw = _run(wl, inp, idx, w)
    _compare(wl, b, kw, cpu, idx, w)


def test_backward_wgrad_tail_split_matches_oracle():
    """A layer whose weight-gradient launch ends in a partial window of shared-expert tiles:
    80 experts x 3 one-tile gradients + 24 shared tiles = 264 tiles, so the last 8 (K = 1,024
    own tokens) are computed as 4 K pieces each and summed. Every gradient against the oracle,
    and reruns bit-identical."""
    wl = synth.scaled(synth.WORKLOADS[synth.EP1], name="bwd_split", T_pool=1024, d=256, E=80,
                      k=2, I=128, E_l=80, tokens_per_rank=1024, T_own=1024, n_shared=2,
                      I_shared=1024)
    cdiv = lambda a, b: -(-a // b)
    sh = (2 * cdiv(wl.n_shared * wl.I_shared, 256) * cdiv(wl.d, 256)
          + wl.n_shared * cdiv(wl.d, 256) * cdiv(wl.I_shared, 256))
    total = 3 * wl.E_l * cdiv(wl.I, 256) * cdiv(wl.d, 256) + sh
    assert (sh, total % 256) == (24, 8)          # the split applies: 8 <= 24 shared tiles
    inp = make_inputs(wl, DEV)
    cpu, idx, w = _routing(wl, inp)
    b, kw = _run(wl, inp, idx, w)
    _compare(wl, b, kw, cpu, idx, w)
    first = [t.clone() for t in (b.dws_gate, b.dws_up, b.dws_down)]
    b.backward()
    torch.cuda.synchronize()
    for a, c in zip((b.dws_gate, b.dws_up, b.dws_down), first):
        assert torch.equal(a.view(torch.int32), c.view(torch.int32))
