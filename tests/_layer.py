"""Shared helpers of the GPU parity tests: seeded inputs of a workload on a device, one
library forward, and the comparison metric."""
from __future__ import annotations

import numpy as np
import torch

import synth


def rel_err(got, ref) -> float:
    """max|got - ref| / max|ref| (float64)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


TOL = {"fp32": 1e-4, "bf16": 1e-2, "mxfp8": 3e-2, "mxfp4": 3e-2}


def make_inputs(wl: synth.Workload, device) -> dict:
    """All inputs of workload wl, generated on `device` by the seeded generator."""
    inp = dict(x=synth.x_rows(wl, range(wl.T_pool), device))
    if wl.routing == "router":
        inp["w_router"] = synth.router_weight(wl, device)
    else:
        inp["logits"] = synth.pool_logits_rows(wl, range(wl.T_pool), device)
    inp["wg"], inp["wu"], inp["wd"] = synth.expert_weights(wl, device)
    if wl.n_shared:
        inp["sg"], inp["su"], inp["sd"] = synth.shared_weights(wl, device)
    else:
        inp["sg"] = inp["su"] = inp["sd"] = None
    return inp


def gpu_layer(wl: synth.Workload, inp: dict, *, topk=None, mb=None, ring=None, flags=0,
              keep=True):
    """A MoeLayer bound to the inputs; routing from the router or from given (idx, w)."""
    import routing_grouped_expert_gemm_amd as mok
    kw = {}
    if wl.routing == "router" and topk is None:
        kw["w_router"] = inp["w_router"]
    else:
        kw["topk_idx"], kw["topk_w"] = topk
    return mok.MoeLayer(
        dtype=wl.dtype, d=wl.d, E=wl.E, k=wl.k, I=wl.I, e0=wl.e0, E_l=wl.E_l,
        tokens_per_rank=wl.tokens_per_rank, T_pool=wl.T_pool, own_begin=wl.own_begin,
        T_own=wl.T_own, n_shared=wl.n_shared, I_shared=wl.I_shared,
        minibatch_rows=mb or wl.minibatch_rows, ring_rows=ring or wl.ring_rows, flags=flags,
        x=inp["x"], w_gate=inp["wg"], w_up=inp["wu"], w_down=inp["wd"], ws_gate=inp["sg"],
        ws_up=inp["su"], ws_down=inp["sd"], keep_intermediates=keep, device=inp["x"].device,
        **kw)


def gpu_topk(logits: torch.Tensor, k: int):
    import routing_grouped_expert_gemm_amd as mok
    T = logits.shape[0]
    idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    mok.mok_topk(logits, k, idx, w)
    return idx, w


def to_np(t):
    return None if t is None else t.detach().float().cpu().numpy() if t.is_floating_point() \
        else t.detach().cpu().numpy()


def kmajor_scales_to_rows(buf, n_rows: int, K: int, R: int) -> np.ndarray:
    """Row-major [n_rows, K/32] E8M0 scales from a K-step-major region (layout stated in
    include/mok.h): matrix g = row // R; (row r, block b) at g*R*(K/32) + ((b//4)*R + r)*4 + b%4."""
    buf = np.asarray(buf)
    rows = np.arange(n_rows, dtype=np.int64)[:, None]
    b = np.arange(K // 32, dtype=np.int64)[None, :]
    g, r = rows // R, rows % R
    return buf[g * R * (K // 32) + ((b // 4) * R + r) * 4 + (b % 4)]


def stage_order_minibatches(counts, offsets, route_ids, k: int, mb: int, own_begin: int,
                            T_own: int, shared: bool):
    """Ring row -> pool row of the gathered A rows of a stage-ordered (MOK_FLAG_NO_RING)
    forward, as include/mok.h states it: minibatch m (routed experts ascending, each region
    cut into mb-row pieces, then the own tokens) keeps ring rows [m*mb, m*mb + rows)."""
    ring_rows, pool_rows = [], []
    m = 0
    for e in range(len(counts)):
        c = int(counts[e])
        for i in range(0, c, mb):
            n = min(mb, c - i)
            ring_rows.append(m * mb + np.arange(n))
            pool_rows.append(np.asarray(route_ids[offsets[e] + i:offsets[e] + i + n]) // k)
            m += 1
    if shared:
        for i in range(0, T_own, mb):
            n = min(mb, T_own - i)
            ring_rows.append(m * mb + np.arange(n))
            pool_rows.append(own_begin + i + np.arange(n))
            m += 1
    if not ring_rows:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    return np.concatenate(ring_rows).astype(np.int64), np.concatenate(pool_rows).astype(np.int64)
