"""CPU oracle for the MoE-layer forward -- TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import this package.
It shares no code with the HIP library and never imports it.

The integer and bit-level steps (router logits in a fixed float32 FMA order, top-k, the
pull-schedule plan, the MXFP8 codec) are plain C in mok_oracle.c, loaded through ctypes.
The floating-point layer arithmetic is here, in float64 with numpy; a float64 matrix product
serves as the dot-product step of each projection.

Layer (the MoK write-up, "Overlapping compute and communication in MoE"; the layer formula
itself is lost from the extracted page, so the DeepSeek-V3 form the section names is used):
  FFN(a)   = W_down (silu(W_gate a) * (W_up a)),  silu(z) = z / (1 + exp(-z))
  y[t]     = sum_s FFN_s(x[t]) + sum_{j<k} w[t,j] FFN_{idx[t,j]}(x[t])
One rank's share of an expert-parallel layer (same section: 256 experts over 64 ranks gives
each rank 4 routed experts plus the shared expert) computes, for each local route r = t*k+j,
the scaled expert output P[r] = w[t,j] FFN_{idx[t,j]}(x[t]) in a source-indexed slot, and
the shared expert on its own tokens; the sum over j happens at the token's source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mok_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmok_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile mok_oracle.c with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                               "-shared", "-fPIC", "-std=c11", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        L.orc_router_logits.argtypes = [P, P, i64, i32, i32, P]
        L.orc_topk.argtypes = [P, i64, i32, i32, P, P]
        L.orc_dispatch_plan.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, P]
        L.orc_dispatch_plan.restype = i64
        L.orc_e4m3_encode.argtypes = [ctypes.c_float, i32]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_decode.restype = ctypes.c_float
        L.orc_mx_shared_exponent.argtypes = [ctypes.c_float]
        L.orc_mx_shared_exponent.restype = i32
        L.orc_mxfp8_quantize.argtypes = [P, i64, i32, P, P]
        L.orc_mxfp8_dequantize.argtypes = [P, P, i64, i32, P]
        L.orc_e2m1_encode.argtypes = [ctypes.c_float, i32]
        L.orc_e2m1_encode.restype = ctypes.c_uint8
        L.orc_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.orc_e2m1_decode.restype = ctypes.c_float
        L.orc_mx4_shared_exponent.argtypes = [ctypes.c_float]
        L.orc_mx4_shared_exponent.restype = i32
        L.orc_mxfp4_quantize.argtypes = [P, i64, i32, P, P]
        L.orc_mxfp4_dequantize.argtypes = [P, P, i64, i32, P]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(a) -> np.ndarray:
    if hasattr(a, "detach"):  # a torch tensor (bf16 -> fp32 is exact)
        a = a.detach().to("cpu").float().numpy()
    return np.ascontiguousarray(a, dtype=np.float32)


# ------------------------------------------------------------------------ routing

def router_logits(x, w_router) -> np.ndarray:
    """logits[t,e] = float32 FMA chain over i ascending of x[t,i]*W_r[e,i] (C)."""
    x, wr = _f32(x), _f32(w_router)
    T, d = x.shape
    E = wr.shape[0]
    out = np.empty((T, E), np.float32)
    lib().orc_router_logits(_p(x), _p(wr), T, d, E, _p(out))
    return out


def topk(logits, k: int):
    """(idx int32 [T,k], w float32 [T,k]): top-k by logit, ties to the lower index (C)."""
    lg = _f32(logits)
    T, E = lg.shape
    if not (1 <= k <= E <= 1024):
        raise ValueError("need 1 <= k <= E <= 1024")
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    lib().orc_topk(_p(lg), T, E, k, _p(idx), _p(w))
    return idx, w


def dispatch_plan(topk_idx, e0: int, E_l: int, tokens_per_rank: int) -> dict:
    """Pull schedule of the local experts [e0, e0+E_l) (C); see mok_oracle.c."""
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, k = idx.shape
    if T % tokens_per_rank:
        raise ValueError("T must be a multiple of tokens_per_rank")
    R = T // tokens_per_rank
    counts = np.empty(E_l, np.int32)
    offsets = np.empty(E_l + 1, np.int32)
    rank_counts = np.empty((E_l, R), np.int32)
    route_ids = np.empty(max(1, T * min(k, E_l)), np.int32)
    n = lib().orc_dispatch_plan(_p(idx), T, k, e0, E_l, tokens_per_rank, _p(counts),
                                _p(offsets), _p(rank_counts), _p(route_ids))
    return dict(counts=counts, offsets=offsets, rank_counts=rank_counts,
                route_ids=route_ids[:n].copy(), n=int(n))


# ------------------------------------------------------------------------ MXFP8

def mxfp8_quantize(v):
    """OCP MXFP8 along the last axis: (codes uint8 [...,K], scales uint8 [...,K/32]) (C)."""
    a = _f32(v)
    K = a.shape[-1]
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    rows = a.size // K
    codes = np.empty(a.shape, np.uint8)
    scales = np.empty(a.shape[:-1] + (K // 32,), np.uint8)
    lib().orc_mxfp8_quantize(_p(a), rows, K, _p(codes), _p(scales))
    return codes, scales


def mxfp8_dequantize(codes, scales) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    K = codes.shape[-1]
    out = np.empty(codes.shape, np.float32)
    lib().orc_mxfp8_dequantize(_p(codes), _p(scales), codes.size // K, K, _p(out))
    return out


def mx_roundtrip(v) -> np.ndarray:
    """The value an MXFP8 operand carries: dequantize(quantize(v))."""
    return mxfp8_dequantize(*mxfp8_quantize(v))


def mxfp4_quantize(v):
    """OCP MXFP4 along the last axis: (codes uint8 [...,K/2], element 2i in the low nibble of
    byte i; scales uint8 [...,K/32]) (C)."""
    a = _f32(v)
    K = a.shape[-1]
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    rows = a.size // K
    codes = np.empty(a.shape[:-1] + (K // 2,), np.uint8)
    scales = np.empty(a.shape[:-1] + (K // 32,), np.uint8)
    lib().orc_mxfp4_quantize(_p(a), rows, K, _p(codes), _p(scales))
    return codes, scales


def mxfp4_dequantize(codes, scales) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    K = codes.shape[-1] * 2
    out = np.empty(codes.shape[:-1] + (K,), np.float32)
    lib().orc_mxfp4_dequantize(_p(codes), _p(scales), codes.size * 2 // K, K, _p(out))
    return out


def mx4_roundtrip(v) -> np.ndarray:
    """The value an MXFP4 operand carries: dequantize(quantize(v))."""
    return mxfp4_dequantize(*mxfp4_quantize(v))


# ------------------------------------------------------------------------ expert FFN

def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def _mx_fn(mx):
    """The round trip of an MX operand format: MXFP8 (mx True or "mxfp8") or MXFP4."""
    return mx4_roundtrip if mx == "mxfp4" else mx_roundtrip


def swiglu_ffn(a, w_gate, w_up, w_down, mx_hidden=False) -> np.ndarray:
    """FFN(a) = W_down (silu(W_gate a) * (W_up a)) for the rows of a, in float64.

    w_gate, w_up: [I, d]; w_down: [d, I] (nn.Linear [out, in] layout). mx_hidden: the hidden
    activation is an MX operand of the down projection (blocks of 32 along I): True or
    "mxfp8" for MXFP8, "mxfp4" for MXFP4."""
    a = np.asarray(a, np.float64)
    g = a @ np.asarray(w_gate, np.float64).T
    u = a @ np.asarray(w_up, np.float64).T
    h = silu(g) * u
    if mx_hidden:
        h = _mx_fn(mx_hidden)(h.astype(np.float32)).astype(np.float64)
    return h @ np.asarray(w_down, np.float64).T


def shared_ffn(a, s_gate, s_up, s_down, mx_hidden: bool = False) -> np.ndarray:
    """S = sum over shared experts s (ascending) of FFN_s(a)."""
    out = None
    for s in range(len(s_gate)):
        o = swiglu_ffn(a, s_gate[s], s_up[s], s_down[s], mx_hidden)
        out = o if out is None else out + o
    return out


# ------------------------------------------------------------------------ the layer

def _operand(v, mx) -> np.ndarray:
    """Operand values as the GEMMs see them: exact float32 upcast, or the MX round trip (mx True
    or "mxfp8": MXFP8; "mxfp4": MXFP4)."""
    v = _f32(v)
    return _mx_fn(mx)(v) if mx else v


def route_outputs(routes, x_rows, topk_idx, topk_w, e0, wg, wu, wd, mx=False):
    """P[r] = w[t,j] * FFN_{idx[t,j]}(x[t]) for routes r = t*k+j (x_rows[i] = x[t of routes[i]]).

    Returns float64 [len(routes), d]."""
    routes = np.asarray(routes, np.int64)
    k = topk_idx.shape[1]
    a = _operand(x_rows, mx)
    wg, wu, wd = _f32(wg), _f32(wu), _f32(wd)
    out = np.empty((len(routes), wd.shape[1]), np.float64)
    experts = topk_idx.reshape(-1)[routes] - e0
    weights = topk_w.reshape(-1)[routes].astype(np.float64)
    for le in np.unique(experts):
        sel = np.nonzero(experts == le)[0]
        o = swiglu_ffn(a[sel], _operand(wg[le], mx), _operand(wu[le], mx), _operand(wd[le], mx), mx)
        out[sel] = weights[sel, None] * o
    return out


def moe_forward(wl, x, w_router=None, logits=None, wg=None, wu=None, wd=None, sg=None, su=None,
                sd=None, topk_in=None) -> dict:
    """Whole forward (or one rank's share) of the workload wl on a pool x, in the pages' order:

    routing (router projection, top-k, weights) -> pull plan for the local experts -> each
    local route's scaled expert output in its source-indexed slot -> shared experts on the
    own tokens -> (full layer only) y[t] = S[t] + sum_{j ascending} P[t*k+j].

    Returns idx, w, plan, P (float64 [n_local_routes, d], row i for plan route_ids[i]),
    y_shared (float64 [T_own, d]) and y (float64 [T_pool, d] or None)."""
    mx = wl.dtype if wl.dtype in ("mxfp8", "mxfp4") else False
    if topk_in is not None:
        idx, w = topk_in
    else:
        if logits is None:
            logits = router_logits(x, w_router)
        idx, w = topk(logits, wl.k)
    plan = dispatch_plan(idx, wl.e0, wl.E_l, wl.tokens_per_rank)
    rids = plan["route_ids"].astype(np.int64)
    xf = _f32(x)
    P = route_outputs(rids, xf[rids // wl.k], idx, w, wl.e0, wg, wu, wd, mx)
    own = xf[wl.own_begin:wl.own_begin + wl.T_own]
    if wl.n_shared:
        S = shared_ffn(_operand(own, mx), _operand(sg, mx), _operand(su, mx), _operand(sd, mx), mx)
    else:                        # no shared expert: the sum over shared experts is empty
        S = np.zeros((wl.T_own, wl.d), np.float64)
    y = None
    if wl.full_layer:
        assert wl.own_begin == 0 and wl.T_own == wl.T_pool
        slot = np.zeros((wl.T_pool * wl.k, wl.d), np.float64)
        slot[rids] = P
        y = S.copy()
        for j in range(wl.k):
            y += slot[j::wl.k]
    return dict(idx=idx, w=w, plan=plan, P=P, y_shared=S, y=y)


# ------------------------------------------------------------------------ backward

def silu_grad(z: np.ndarray) -> np.ndarray:
    """d silu / dz = sigma(z) (1 + z (1 - sigma(z)))."""
    sg = 1.0 / (1.0 + np.exp(-z))
    return sg * (1.0 + z * (1.0 - sg))


def swiglu_ffn_backward(a, w_gate, w_up, w_down, d_out, scale=1.0):
    """Backward of out = scale * W_down (silu(W_gate a) * (W_up a)) for the rows of a (float64).

    d_out: gradient of out, [rows, d]; scale: a per-row weight ([rows] or a number). Returns
    dict(da, dw_gate, dw_up, dw_down, dscale) where dscale[r] = <d_out[r], FFN(a[r])> (the
    gradient of the per-row weight)."""
    a = np.asarray(a, np.float64)
    wg, wu, wd = (np.asarray(t, np.float64) for t in (w_gate, w_up, w_down))
    dout = np.asarray(d_out, np.float64)
    sc = np.broadcast_to(np.asarray(scale, np.float64), (a.shape[0],))[:, None]
    g = a @ wg.T
    u = a @ wu.T
    h = silu(g) * u
    o = h @ wd.T                                  # unscaled expert output
    dscale = (dout * o).sum(1)
    do = sc * dout                                # gradient of o
    dh = do @ wd
    dg = dh * u * silu_grad(g)
    du = dh * silu(g)
    return dict(da=dg @ wg + du @ wu, dw_gate=dg.T @ a, dw_up=du.T @ a, dw_down=do.T @ h,
                dscale=dscale)


def moe_backward(wl, x, topk_idx, topk_w, wg, wu, wd, sg=None, su=None, sd=None, dy=None,
                 dy_slots=None, dy_shared=None) -> dict:
    """Backward of the layer (or share) of moe_forward with the routing held fixed, in float64.

    Upstream gradient: dy [T_pool, d] for the whole layer (each route slot and the shared
    output then receive dy of their token), or dy_slots [T_pool*k, d] and dy_shared [T_own, d]
    for a share. Returns the gradient of every input the forward multiplies:
      dx_slots  [n_local_routes, d]  d x[t] through local route r (row i for plan route_ids[i])
      dx_shared [T_own, d]           d x through the shared experts (summed over them)
      dx        [T_pool, d] or None  whole layer: dx_shared + sum_j dx through route t*k+j
      dtopk_w   [n_local_routes]     d w[t,j] of local route r = <dP_r, FFN_e(x_t)>
      dwg, dwu [E_l, I, d], dwd [E_l, d, I]; dsg, dsu [n_s, I_s, d], dsd [n_s, d, I_s]."""
    idx = np.asarray(topk_idx)
    w = np.asarray(topk_w, np.float64)
    plan = dispatch_plan(idx, wl.e0, wl.E_l, wl.tokens_per_rank)
    rids = plan["route_ids"].astype(np.int64)
    xf = _f32(x).astype(np.float64)
    k = wl.k
    if dy is not None:
        dyf = _f32(dy).astype(np.float64)
        dP = dyf[rids // k]
        dS = dyf[wl.own_begin:wl.own_begin + wl.T_own]
    else:
        dP = _f32(dy_slots).astype(np.float64)[rids]
        dS = _f32(dy_shared).astype(np.float64) if wl.n_shared else None
    wg, wu, wd = _f32(wg), _f32(wu), _f32(wd)
    dwg, dwu, dwd = np.zeros(wg.shape), np.zeros(wu.shape), np.zeros(wd.shape)
    dx_slots = np.zeros((len(rids), wl.d))
    dtw = np.zeros(len(rids))
    experts = idx.reshape(-1)[rids] - wl.e0
    for le in range(wl.E_l):
        sel = np.nonzero(experts == le)[0]
        if len(sel) == 0:
            continue
        r = swiglu_ffn_backward(xf[rids[sel] // k], wg[le], wu[le], wd[le], dP[sel],
                                w.reshape(-1)[rids[sel]])
        dx_slots[sel] = r["da"]
        dtw[sel] = r["dscale"]
        dwg[le], dwu[le], dwd[le] = r["dw_gate"], r["dw_up"], r["dw_down"]
    out = dict(plan=plan, dx_slots=dx_slots, dtopk_w=dtw, dwg=dwg, dwu=dwu, dwd=dwd)
    own = xf[wl.own_begin:wl.own_begin + wl.T_own]
    dx_shared = np.zeros((wl.T_own, wl.d))
    if wl.n_shared:
        sg, su, sd = _f32(sg), _f32(su), _f32(sd)
        dsg, dsu, dsd = np.zeros(sg.shape), np.zeros(su.shape), np.zeros(sd.shape)
        for s in range(wl.n_shared):
            r = swiglu_ffn_backward(own, sg[s], su[s], sd[s], dS)
            dx_shared += r["da"]
            dsg[s], dsu[s], dsd[s] = r["dw_gate"], r["dw_up"], r["dw_down"]
        out.update(dsg=dsg, dsu=dsu, dsd=dsd)
    out["dx_shared"] = dx_shared
    out["dx"] = None
    if wl.full_layer:
        slot = np.zeros((wl.T_pool * k, wl.d))
        slot[rids] = dx_slots
        dx = dx_shared.copy()
        for j in range(k):
            dx += slot[j::k]
        out["dx"] = dx
    return out
