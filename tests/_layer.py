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


TOL = {"fp32": 1e-4, "bf16": 1e-2, "mxfp8": 3e-2}


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
