"""Python binding of libmok (include/mok.h): argument marshalling only.

Every step of the MoE-layer forward runs in the library's HIP kernels; PyTorch supplies
device memory and the current HIP stream. Importing this module loads libmok.so and fails
loudly (ImportError) if it has not been built: there is no fallback of any kind.

Entry points carry the C names: mok_route, mok_topk, mok_dispatch_plan,
mok_dispatch_plan_workspace_bytes, mok_moe_workspace_bytes, mok_moe_forward,
mok_quantize_mxfp8, mok_quantize_mxfp8_f32, mok_quantize_mxfp4_f32, mok_get_device_error,
mok_status_string, mok_version.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmok.so")   # always the in-tree build

MOK_OK, MOK_EINVAL, MOK_EUNSUPPORTED, MOK_EWORKSPACE, MOK_EHIP = range(5)
MOK_FP32, MOK_BF16, MOK_MXFP8, MOK_MXFP4 = 0, 1, 2, 3
MOK_FLAG_NO_RING, MOK_FLAG_STAGE_LOOP = 1, 2
(MOK_STAGE_ROUTE, MOK_STAGE_PLAN, MOK_STAGE_QUANT, MOK_STAGE_UP, MOK_STAGE_DOWN, MOK_STAGE_COMBINE,
 MOK_STAGE_GATHER) = range(7)
MOK_N_STAGES = 7
(MOK_REGION_WORKLIST, MOK_REGION_H, MOK_REGION_H_SCALES, MOK_REGION_A_CODES, MOK_REGION_A_SCALES,
 MOK_REGION_WG_CODES, MOK_REGION_WG_SCALES, MOK_REGION_WU_CODES, MOK_REGION_WU_SCALES,
 MOK_REGION_WD_CODES, MOK_REGION_WD_SCALES, MOK_REGION_SG_CODES, MOK_REGION_SG_SCALES,
 MOK_REGION_SU_CODES, MOK_REGION_SU_SCALES, MOK_REGION_SD_CODES, MOK_REGION_SD_SCALES) = range(17)
MOK_DEVERR_OVERFLOW, MOK_DEVERR_WAIT = 1, 2

EXPORTS = ["mok_status_string", "mok_version", "mok_route", "mok_topk",
           "mok_dispatch_plan_workspace_bytes", "mok_dispatch_plan", "mok_dispatch_plan_noalloc",
           "mok_moe_workspace_bytes",
           "mok_moe_forward", "mok_moe_workspace_region", "mok_moe_backward",
           "mok_moe_backward_workspace_bytes", "mok_moe_backward_error", "mok_pull_gather",
           "mok_push_dispatch", "mok_quantize_mxfp8", "mok_quantize_mxfp4",
           "mok_quantize_mxfp8_f32", "mok_quantize_mxfp4_f32", "mok_get_device_error"]


class MokError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)}")
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(f"libmok.so is not built ({LIB_PATH}); run "
                      "`python routing_grouped_expert_gemm_amd/_build.py` or __graft_entry__.build()")

_lib = ctypes.CDLL(LIB_PATH)
_P, _I64, _I32, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t


class MoeArgs(ctypes.Structure):
    """Mirror of struct mok_moe_args."""
    _fields_ = [
        ("dtype", _I32), ("d", _I32), ("E", _I32), ("k", _I32), ("I", _I32),
        ("e0", _I32), ("E_l", _I32), ("tokens_per_rank", _I32),
        ("T_pool", _I64), ("own_begin", _I64), ("T_own", _I32),
        ("n_shared", _I32), ("I_shared", _I32), ("minibatch_rows", _I32), ("ring_rows", _I32),
        ("flags", ctypes.c_uint32),
        ("x", _P), ("w_router", _P), ("topk_idx_in", _P), ("topk_w_in", _P),
        ("w_gate", _P), ("w_up", _P), ("w_down", _P),
        ("ws_gate", _P), ("ws_up", _P), ("ws_down", _P),
        ("workspace", _P), ("workspace_bytes", _SZ),
        ("y_slots", _P), ("y_shared", _P), ("y", _P),
        ("logits_out", _P), ("topk_idx_out", _P), ("topk_w_out", _P),
        ("counts_out", _P), ("offsets_out", _P), ("rank_counts_out", _P), ("route_ids_out", _P),
        ("stage_events", _P),
    ]


class BwdArgs(ctypes.Structure):
    """Mirror of struct mok_moe_bwd_args."""
    _fields_ = [
        ("dtype", _I32), ("d", _I32), ("E", _I32), ("k", _I32), ("I", _I32), ("e0", _I32),
        ("E_l", _I32), ("tokens_per_rank", _I32), ("T_pool", _I64), ("own_begin", _I64),
        ("T_own", _I32), ("n_shared", _I32), ("I_shared", _I32), ("route_rows_cap", _I64),
        ("x", _P), ("topk_idx", _P), ("topk_w", _P), ("w_gate", _P), ("w_up", _P),
        ("w_down", _P), ("ws_gate", _P), ("ws_up", _P), ("ws_down", _P),
        ("dy", _P), ("dy_slots", _P), ("dy_shared", _P),
        ("workspace", _P), ("workspace_bytes", _SZ),
        ("dx_slots", _P), ("dx_shared", _P), ("dx", _P), ("dtopk_w", _P),
        ("dw_gate", _P), ("dw_up", _P), ("dw_down", _P),
        ("dws_gate", _P), ("dws_up", _P), ("dws_down", _P),
    ]


_lib.mok_status_string.argtypes = [ctypes.c_int]
_lib.mok_status_string.restype = ctypes.c_char_p
_lib.mok_version.argtypes = []
_lib.mok_version.restype = ctypes.c_char_p
_lib.mok_route.argtypes = [_P, _P, _I64, _I32, _I32, _I32, _I32, _P, _P, _P, _P]
_lib.mok_topk.argtypes = [_P, _I64, _I32, _I32, _P, _P, _P]
_lib.mok_dispatch_plan_workspace_bytes.argtypes = [_I64, _I32, _I32, ctypes.POINTER(_SZ)]
_lib.mok_dispatch_plan.argtypes = [_P, _I64, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P,
                                   _SZ, _P]
_lib.mok_dispatch_plan_noalloc.argtypes = [_P, _I64, _I32, _I32, _I32, _I32, _I32, _P, _P, _P,
                                           _P, _P]
_lib.mok_moe_workspace_bytes.argtypes = [ctypes.POINTER(MoeArgs), ctypes.POINTER(_SZ)]
_lib.mok_moe_forward.argtypes = [ctypes.POINTER(MoeArgs), _P]
_lib.mok_moe_workspace_region.argtypes = [ctypes.POINTER(MoeArgs), _I32, ctypes.POINTER(_SZ),
                                          ctypes.POINTER(_SZ), ctypes.POINTER(_I64)]
_lib.mok_moe_backward_workspace_bytes.argtypes = [ctypes.POINTER(BwdArgs), ctypes.POINTER(_SZ)]
_lib.mok_moe_backward.argtypes = [ctypes.POINTER(BwdArgs), _P]
_lib.mok_moe_backward_error.argtypes = [_P, ctypes.POINTER(BwdArgs), ctypes.POINTER(ctypes.c_uint32),
                                        _P]
_lib.mok_quantize_mxfp8.argtypes = [_P, _I64, _I32, _P, _P, _P]
_lib.mok_quantize_mxfp4.argtypes = [_P, _I64, _I32, _P, _P, _P]
_lib.mok_quantize_mxfp8_f32.argtypes = [_P, _I64, _I32, _P, _P, _P]
_lib.mok_quantize_mxfp4_f32.argtypes = [_P, _I64, _I32, _P, _P, _P]
_lib.mok_pull_gather.argtypes = [_P, _I64, _I32, _I32, _I32, _P, _P, _I32, _P, _P]
_lib.mok_push_dispatch.argtypes = [_P, _I64, _I32, _I32, _I32, _P, _I32, _I32, _I64, _P, _P, _P,
                                   _P]
_lib.mok_get_device_error.argtypes = [_P, ctypes.POINTER(ctypes.c_uint32), _P]
for _n in EXPORTS:
    if _n not in ("mok_status_string", "mok_version"):
        getattr(_lib, _n).restype = ctypes.c_int


def status_string(status: int) -> str:
    return _lib.mok_status_string(status).decode()


def version() -> str:
    return _lib.mok_version().decode()


def _check(fn: str, status: int) -> None:
    if status != MOK_OK:
        raise MokError(fn, status)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    if stream is not None:
        return getattr(stream, "cuda_stream", stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


# ------------------------------------------------------------------------ entry points

def mok_route(x, w_router, k: int, logits, topk_idx, topk_w, stream=None) -> None:
    """Router projection + top-k + weights (x [T,d] and w_router [E,d]: float32 or bf16)."""
    import torch
    T, d = x.shape
    E = w_router.shape[0]
    io = MOK_FP32 if x.dtype == torch.float32 else MOK_BF16
    _check("mok_route", _lib.mok_route(_ptr(x), _ptr(w_router), T, d, E, k, io, _ptr(logits),
                                       _ptr(topk_idx), _ptr(topk_w), _stream(stream)))


def mok_topk(logits, k: int, topk_idx, topk_w, stream=None) -> None:
    T, E = logits.shape
    _check("mok_topk", _lib.mok_topk(_ptr(logits), T, E, k, _ptr(topk_idx), _ptr(topk_w),
                                     _stream(stream)))


def mok_dispatch_plan_workspace_bytes(T_pool: int, k: int, E_l: int) -> int:
    out = _SZ(0)
    _check("mok_dispatch_plan_workspace_bytes",
           _lib.mok_dispatch_plan_workspace_bytes(T_pool, k, E_l, ctypes.byref(out)))
    return out.value


def mok_dispatch_plan(topk_idx, E: int, e0: int, E_l: int, tokens_per_rank: int, counts, offsets,
                      rank_counts, route_ids, ws, stream=None) -> None:
    T, k = topk_idx.shape
    _check("mok_dispatch_plan",
           _lib.mok_dispatch_plan(_ptr(topk_idx), T, k, E, e0, E_l, tokens_per_rank, _ptr(counts),
                                  _ptr(offsets), _ptr(rank_counts), _ptr(route_ids), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream)))


def mok_dispatch_plan_noalloc(topk_idx, E: int, e0: int, E_l: int, tokens_per_rank: int, counts,
                              offsets, rank_counts, route_ids, stream=None) -> None:
    """mok_dispatch_plan with the library's fixed device scratch (no workspace argument)."""
    T, k = topk_idx.shape
    _check("mok_dispatch_plan_noalloc",
           _lib.mok_dispatch_plan_noalloc(_ptr(topk_idx), T, k, E, e0, E_l, tokens_per_rank,
                                          _ptr(counts), _ptr(offsets), _ptr(rank_counts),
                                          _ptr(route_ids), _stream(stream)))


def mok_moe_workspace_bytes(args: MoeArgs) -> int:
    out = _SZ(0)
    _check("mok_moe_workspace_bytes", _lib.mok_moe_workspace_bytes(ctypes.byref(args),
                                                                   ctypes.byref(out)))
    return out.value


def mok_moe_forward(args: MoeArgs, stream=None) -> None:
    _check("mok_moe_forward", _lib.mok_moe_forward(ctypes.byref(args), _stream(stream)))


def mok_moe_workspace_region(args: MoeArgs, region: int):
    """(byte offset, bytes, rows R) of an intermediate inside the forward's workspace."""
    off, n, rows = _SZ(0), _SZ(0), _I64(0)
    _check("mok_moe_workspace_region",
           _lib.mok_moe_workspace_region(ctypes.byref(args), region, ctypes.byref(off),
                                         ctypes.byref(n), ctypes.byref(rows)))
    return off.value, n.value, rows.value


def _io(x):
    import torch
    return MOK_FP32 if x.dtype == torch.float32 else MOK_BF16


def mok_pull_gather(x, k: int, route_ids, offsets, buf, stream=None) -> None:
    """buf[i] = x[route_ids[i] // k] for the plan's rows (E_l = offsets.numel() - 1)."""
    T, d = x.shape
    _check("mok_pull_gather", _lib.mok_pull_gather(_ptr(x), T, d, k, _io(x), _ptr(route_ids),
                                                   _ptr(offsets), offsets.numel() - 1,
                                                   _ptr(buf), _stream(stream)))


def mok_push_dispatch(x, topk_idx, e0: int, fill, buf, src_route, stream=None) -> None:
    """Atomic-slot push of every local route's row into buf [E_l, capacity, d]."""
    T, d = x.shape
    k = topk_idx.shape[1]
    E_l, cap = buf.shape[0], buf.shape[1]
    _check("mok_push_dispatch",
           _lib.mok_push_dispatch(_ptr(x), T, d, k, _io(x), _ptr(topk_idx), e0, E_l, cap,
                                  _ptr(fill), _ptr(buf), _ptr(src_route), _stream(stream)))


def mok_quantize_mxfp8(src_bf16, codes, scales, stream=None) -> None:
    rows, K = src_bf16.shape
    _check("mok_quantize_mxfp8", _lib.mok_quantize_mxfp8(_ptr(src_bf16), rows, K, _ptr(codes),
                                                         _ptr(scales), _stream(stream)))


def mok_quantize_mxfp4(src_bf16, codes, scales, stream=None) -> None:
    """MXFP4 along rows: codes [rows, K/2] (two E2M1 codes a byte), scales [rows, K/32]."""
    rows, K = src_bf16.shape
    _check("mok_quantize_mxfp4", _lib.mok_quantize_mxfp4(_ptr(src_bf16), rows, K, _ptr(codes),
                                                         _ptr(scales), _stream(stream)))


def mok_quantize_mxfp8_f32(src_f32, codes, scales, stream=None) -> None:
    """MXFP8 of float32 rows: codes [rows, K], scales [rows, K/32]."""
    rows, K = src_f32.shape
    _check("mok_quantize_mxfp8_f32", _lib.mok_quantize_mxfp8_f32(
        _ptr(src_f32), rows, K, _ptr(codes), _ptr(scales), _stream(stream)))


def mok_quantize_mxfp4_f32(src_f32, codes, scales, stream=None) -> None:
    """MXFP4 of float32 rows: codes [rows, K/2], scales [rows, K/32]."""
    rows, K = src_f32.shape
    _check("mok_quantize_mxfp4_f32", _lib.mok_quantize_mxfp4_f32(
        _ptr(src_f32), rows, K, _ptr(codes), _ptr(scales), _stream(stream)))


def mok_get_device_error(workspace, stream=None) -> int:
    err = ctypes.c_uint32(0)
    _check("mok_get_device_error", _lib.mok_get_device_error(_ptr(workspace), ctypes.byref(err),
                                                             _stream(stream)))
    return err.value


# ------------------------------------------------------------------------ layer helper

_DT = {"fp32": MOK_FP32, "bf16": MOK_BF16, "mxfp8": MOK_MXFP8, "mxfp4": MOK_MXFP4}


class MoeLayer:
    """Holds the argument struct, the workspace and the outputs of one layer configuration.

    Shapes follow mok_moe_args. `forward()` enqueues one mok_moe_forward on the current stream.
    """

    def __init__(self, *, dtype: str, d: int, E: int, k: int, I: int, e0: int, E_l: int,
                 tokens_per_rank: int, T_pool: int, own_begin: int, T_own: int, n_shared: int,
                 I_shared: int, minibatch_rows: int, ring_rows: int, x, w_gate, w_up, w_down,
                 ws_gate=None, ws_up=None, ws_down=None, w_router=None, topk_idx=None,
                 topk_w=None, flags: int = 0, keep_intermediates: bool = False, device="cuda"):
        import torch
        self._keep = [x, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, w_router, topk_idx, topk_w]
        odt = torch.float32 if dtype == "fp32" else torch.bfloat16
        a = MoeArgs()
        a.dtype, a.d, a.E, a.k, a.I = _DT[dtype], d, E, k, I
        a.e0, a.E_l, a.tokens_per_rank = e0, E_l, tokens_per_rank
        a.T_pool, a.own_begin, a.T_own = T_pool, own_begin, T_own
        a.n_shared, a.I_shared = n_shared, I_shared
        a.minibatch_rows, a.ring_rows, a.flags = minibatch_rows, ring_rows, flags
        a.x, a.w_router = _ptr(x), _ptr(w_router)
        a.topk_idx_in, a.topk_w_in = _ptr(topk_idx), _ptr(topk_w)
        a.w_gate, a.w_up, a.w_down = _ptr(w_gate), _ptr(w_up), _ptr(w_down)
        a.ws_gate, a.ws_up, a.ws_down = _ptr(ws_gate), _ptr(ws_up), _ptr(ws_down)
        self.y_slots = torch.empty((T_pool * k, d), dtype=odt, device=device)
        # at least one row, so that a share with no own tokens still passes a valid pointer
        ysh = torch.empty((max(1, T_own), d), dtype=odt, device=device) if n_shared else None
        self.y_shared = ysh[:T_own] if n_shared else None
        self.y = torch.empty((T_pool, d), dtype=odt, device=device) if E_l == E else None
        a.y_slots, a.y_shared, a.y = _ptr(self.y_slots), _ptr(ysh), _ptr(self.y)
        self._keep.append(ysh)
        self.inter = {}
        if keep_intermediates:
            i32 = dict(dtype=torch.int32, device=device)
            if w_router is not None:
                self.inter["logits"] = torch.empty((T_pool, E), dtype=torch.float32, device=device)
                self.inter["topk_idx"] = torch.empty((T_pool, k), **i32)
                self.inter["topk_w"] = torch.empty((T_pool, k), dtype=torch.float32, device=device)
                a.logits_out = _ptr(self.inter["logits"])
                a.topk_idx_out = _ptr(self.inter["topk_idx"])
                a.topk_w_out = _ptr(self.inter["topk_w"])
            self.inter["counts"] = torch.empty(E_l, **i32)
            self.inter["offsets"] = torch.empty(E_l + 1, **i32)
            self.inter["rank_counts"] = torch.empty((E_l, T_pool // tokens_per_rank), **i32)
            self.inter["route_ids"] = torch.empty(max(1, T_pool * min(k, E_l)), **i32)
            a.counts_out = _ptr(self.inter["counts"])
            a.offsets_out = _ptr(self.inter["offsets"])
            a.rank_counts_out = _ptr(self.inter["rank_counts"])
            a.route_ids_out = _ptr(self.inter["route_ids"])
        nbytes = mok_moe_workspace_bytes(a)
        self.workspace = torch.empty(max(1, nbytes), dtype=torch.uint8, device=device)
        a.workspace, a.workspace_bytes = _ptr(self.workspace), nbytes
        self.args = a

    def forward(self, stream=None) -> None:
        mok_moe_forward(self.args, stream)

    def device_error(self, stream=None) -> int:
        return mok_get_device_error(self.workspace, stream)

    def region(self, region: int):
        """(uint8 view of the workspace bytes of an intermediate, rows R); see
        mok_moe_workspace_region. Read it after the forward has finished."""
        off, n, rows = mok_moe_workspace_region(self.args, region)
        return self.workspace[off:off + n], rows


class MoeBackward:
    """Argument struct, workspace and outputs of one backward configuration (mok_moe_backward).

    Whole layer: pass dy [T_pool, d]. Share: dy_slots [T_pool*k, d] and dy_shared [T_own, d].
    Outputs: dx_slots, dx_shared, dx (whole layer), dtopk_w, dw_* and dws_* (float32)."""

    def __init__(self, *, d: int, E: int, k: int, I: int, e0: int, E_l: int,
                 tokens_per_rank: int, T_pool: int, own_begin: int, T_own: int, n_shared: int,
                 I_shared: int, x, topk_idx, topk_w, w_gate, w_up, w_down, ws_gate=None,
                 ws_up=None, ws_down=None, dy=None, dy_slots=None, dy_shared=None,
                 route_rows_cap: int = 0, device="cuda"):
        import torch
        self._keep = [x, topk_idx, topk_w, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, dy,
                      dy_slots, dy_shared]
        a = BwdArgs()
        a.dtype, a.d, a.E, a.k, a.I, a.e0, a.E_l = MOK_BF16, d, E, k, I, e0, E_l
        a.tokens_per_rank, a.T_pool, a.own_begin, a.T_own = tokens_per_rank, T_pool, own_begin, T_own
        a.n_shared, a.I_shared, a.route_rows_cap = n_shared, I_shared, route_rows_cap
        a.x, a.topk_idx, a.topk_w = _ptr(x), _ptr(topk_idx), _ptr(topk_w)
        a.w_gate, a.w_up, a.w_down = _ptr(w_gate), _ptr(w_up), _ptr(w_down)
        a.ws_gate, a.ws_up, a.ws_down = _ptr(ws_gate), _ptr(ws_up), _ptr(ws_down)
        a.dy, a.dy_slots, a.dy_shared = _ptr(dy), _ptr(dy_slots), _ptr(dy_shared)
        bf, f32 = dict(dtype=torch.bfloat16, device=device), dict(dtype=torch.float32, device=device)
        self.dx_slots = torch.empty((T_pool * k, d), **bf)
        sh = n_shared > 0 and T_own > 0
        self.dx_shared = torch.empty((T_own, d), **bf) if sh else None
        self.dx = torch.empty((T_pool, d), **bf) if E_l == E else None
        self.dtopk_w = torch.empty((T_pool, k), **f32)
        self.dw_gate = torch.empty((E_l, I, d), **f32)
        self.dw_up = torch.empty((E_l, I, d), **f32)
        self.dw_down = torch.empty((E_l, d, I), **f32)
        if n_shared:
            self.dws_gate = torch.empty((n_shared, I_shared, d), **f32)
            self.dws_up = torch.empty((n_shared, I_shared, d), **f32)
            self.dws_down = torch.empty((n_shared, d, I_shared), **f32)
        else:
            self.dws_gate = self.dws_up = self.dws_down = None
        a.dx_slots, a.dx_shared, a.dx = _ptr(self.dx_slots), _ptr(self.dx_shared), _ptr(self.dx)
        a.dtopk_w = _ptr(self.dtopk_w)
        a.dw_gate, a.dw_up, a.dw_down = _ptr(self.dw_gate), _ptr(self.dw_up), _ptr(self.dw_down)
        a.dws_gate, a.dws_up, a.dws_down = (_ptr(self.dws_gate), _ptr(self.dws_up),
                                            _ptr(self.dws_down))
        n = _SZ(0)
        _check("mok_moe_backward_workspace_bytes",
               _lib.mok_moe_backward_workspace_bytes(ctypes.byref(a), ctypes.byref(n)))
        self.workspace = torch.empty(max(1, n.value), dtype=torch.uint8, device=device)
        a.workspace, a.workspace_bytes = _ptr(self.workspace), n.value
        self.args = a

    def backward(self, stream=None) -> None:
        _check("mok_moe_backward", _lib.mok_moe_backward(ctypes.byref(self.args), _stream(stream)))

    def device_error(self, stream=None) -> int:
        err = ctypes.c_uint32(0)
        _check("mok_moe_backward_error",
               _lib.mok_moe_backward_error(_ptr(self.workspace), ctypes.byref(self.args),
                                           ctypes.byref(err), _stream(stream)))
        return err.value
