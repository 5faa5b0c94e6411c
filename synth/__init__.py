"""Seeded synthetic inputs for the MoE-layer forward.

Both sides of every parity check draw their inputs from here: the CPU oracle and the HIP
path. The module holds none of the layer's arithmetic (no routing, no top-k, no FFN); it
only turns (seed, stream, flat index) into numbers.

Generator (counter-based):
  u32(seed, stream, j, i) = fmix32(fmix32(i XOR key_j) XOR rotl(key_j))  (MurmurHash3's
  32-bit finaliser, used as a hash of the counter i), key_j derived from (seed, stream, j).
  normal(i) = sqrt(-2 ln u_0) cos(2 pi u_1), u_j = (u32(.., j, i) + 1/2) / 2^32 in (0, 1):
  the Box-Muller transform (its cosine branch), one standard normal per counter, in float64,
  scaled by sigma and rounded to float32 (then to bf16 for bf16 tensors). The 32-bit draws
  bound |normal| by sqrt(2 ln 2^33) = 6.8.
  The hashes are integer-exact on every device; the float64 log and cosine may differ in the
  last bit between the CPU and the GPU, which moves a float32 result only when it lies within
  about 2^-29 of a rounding boundary. Parity tests therefore generate each input once and hand
  the same tensor (copied) to both sides.

Every element is a pure function of its flat index, so any rows of any tensor can be
regenerated without producing the rest.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

MASK32 = 0xFFFFFFFF
SEED = 0

# stream ids, one per tensor
S_X, S_WR, S_WG, S_WU, S_WD, S_SG, S_SU, S_SD, S_LOGITS, S_PERM = 1, 2, 3, 4, 5, 6, 7, 8, 9, 10


def _fmix32_int(h: int) -> int:
    h &= MASK32
    h ^= h >> 16
    h = (h * 0x85EBCA6B) & MASK32
    h ^= h >> 13
    h = (h * 0xC2B2AE35) & MASK32
    h ^= h >> 16
    return h


def _key(seed: int, stream: int, j: int) -> int:
    return _fmix32_int((seed * 0x9E3779B9 + stream * 0x85EBCA77 + j * 0xC2B2AE3D + 0x27D4EB2F) & MASK32)


def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    """(x * c) mod 2^32 for int64 x in [0, 2^32), without int64 overflow."""
    lo, hi = c & 0xFFFF, c >> 16
    return (x * lo + ((x * hi) & 0xFFFF) * 65536) & MASK32


def _fmix32(h: torch.Tensor) -> torch.Tensor:
    h = h ^ (h >> 16)
    h = _mul32(h, 0x85EBCA6B)
    h = h ^ (h >> 13)
    h = _mul32(h, 0xC2B2AE35)
    return h ^ (h >> 16)


def u32(seed: int, stream: int, j: int, idx: torch.Tensor) -> torch.Tensor:
    """32-bit hash of the counter idx (int64 tensor, values < 2^32); returns int64 in [0, 2^32)."""
    k = _key(seed, stream, j)
    k2 = ((k << 13) | (k >> 19)) & MASK32
    return _fmix32(_fmix32(idx ^ k) ^ k2)


_INV_2_32 = 1.0 / 4294967296.0


def _normal_of(seed: int, stream: int, idx: torch.Tensor, sigma: float) -> torch.Tensor:
    """Box-Muller normal of counters idx (int64 tensor): float32, standard deviation sigma."""
    u0 = (u32(seed, stream, 0, idx).to(torch.float64) + 0.5) * _INV_2_32
    u1 = (u32(seed, stream, 1, idx).to(torch.float64) + 0.5) * _INV_2_32
    z = torch.sqrt(-2.0 * torch.log(u0)) * torch.cos((2.0 * math.pi) * u1)
    return (z * sigma).to(torch.float32)


def normal_flat(seed: int, stream: int, start: int, count: int, sigma: float,
                device="cpu") -> torch.Tensor:
    """float32 values number start .. start+count-1 of stream `stream` (std sigma)."""
    if start < 0 or start + count > (1 << 32):
        raise ValueError("counter range exceeds 2^32")
    idx = torch.arange(start, start + count, dtype=torch.int64, device=device)
    return _normal_of(seed, stream, idx, sigma)


def normal_rows(seed: int, stream: int, n_cols: int, rows, sigma: float, dtype=torch.float32,
                device="cpu", chunk_elems: int = 1 << 25) -> torch.Tensor:
    """Rows `rows` (a range or an int64 tensor of row ids) of a [R, n_cols] tensor."""
    if isinstance(rows, range):
        assert rows.step == 1
        r0, r1 = rows.start, rows.stop
        out = torch.empty((r1 - r0, n_cols), dtype=dtype, device=device)
        step = max(1, chunk_elems // max(1, n_cols))
        for a in range(r0, r1, step):
            b = min(r1, a + step)
            v = normal_flat(seed, stream, a * n_cols, (b - a) * n_cols, sigma, device)
            out[a - r0:b - r0] = v.view(b - a, n_cols).to(dtype)
        return out
    rows = torch.as_tensor(rows, dtype=torch.int64)
    out = torch.empty((rows.numel(), n_cols), dtype=dtype, device=device)
    cols = torch.arange(n_cols, dtype=torch.int64, device=device)
    for i, r in enumerate(rows.tolist()):
        out[i] = _normal_of(seed, stream, r * n_cols + cols, sigma).to(dtype)
    return out


def normal_tensor(shape, seed: int, stream: int, sigma: float, dtype=torch.float32,
                  device="cpu") -> torch.Tensor:
    n_cols = shape[-1]
    n_rows = 1
    for s in shape[:-1]:
        n_rows *= s
    return normal_rows(seed, stream, n_cols, range(n_rows), sigma, dtype, device).view(*shape)


def seeded_permutation(seed: int, stream: int, n: int) -> torch.Tensor:
    """A permutation of range(n): ascending order of (hash, index)."""
    keys = u32(seed, stream, 0, torch.arange(n, dtype=torch.int64))
    order = sorted(range(n), key=lambda i: (int(keys[i]), i))
    return torch.tensor(order, dtype=torch.int64)


# --------------------------------------------------------------------------- workloads

@dataclass
class Workload:
    """Shapes of one MoE-layer forward (or one rank's share of it)."""
    name: str
    dtype: str                 # "fp32" | "bf16" | "mxfp8" | "mxfp4"
    T_pool: int                # rows in the token pool held in HBM
    d: int                     # model dim
    E: int                     # routed experts in the whole layer
    k: int                     # top-k
    I: int                     # routed expert intermediate
    e0: int                    # first local expert
    E_l: int                   # local experts
    tokens_per_rank: int       # pool rows per simulated source rank
    own_begin: int             # first row of this rank's own tokens
    T_own: int                 # own tokens (shared-expert rows)
    n_shared: int
    I_shared: int
    routing: str               # "router" (x . W_r computed here) | "logits" (given pool logits)
    zipf_beta: float = 0.0     # Zipf(s=1.1) logit-bias strength ("logits" routing only)
    ring_rows: int = 16384
    minibatch_rows: int = 256
    notes: str = ""

    @property
    def full_layer(self) -> bool:
        return self.E_l == self.E

    @property
    def n_ranks(self) -> int:
        return self.T_pool // self.tokens_per_rank


ZIPF_S = 1.1
# Bias strength for the skewed 384-expert workload, found by bisection on the oracle's own
# top-k counts (oracle/calibrate_zipf.py) so that local expert 0 receives 4.0x the mean load.
ZIPF_BETA_EP96 = 0.1245574951171875

WORKLOADS = {
    "tiny_fp32_t64_d128_e8_top2": Workload(
        name="tiny_fp32_t64_d128_e8_top2", dtype="fp32", T_pool=64, d=128, E=8, k=2, I=256,
        e0=0, E_l=8, tokens_per_rank=64, own_begin=0, T_own=64, n_shared=1, I_shared=256,
        routing="router", ring_rows=1024, minibatch_rows=128),
    "ep1_bf16_t8192_d2048_e64_top6": Workload(
        name="ep1_bf16_t8192_d2048_e64_top6", dtype="bf16", T_pool=8192, d=2048, E=64, k=6,
        I=1408, e0=0, E_l=64, tokens_per_rank=8192, own_begin=0, T_own=8192, n_shared=2,
        I_shared=1408, routing="router", ring_rows=16384, minibatch_rows=256),
    "ep64_share_bf16_pool262144_d7168_e256_top8": Workload(
        name="ep64_share_bf16_pool262144_d7168_e256_top8", dtype="bf16", T_pool=262144,
        d=7168, E=256, k=8, I=2048, e0=0, E_l=4, tokens_per_rank=4096, own_begin=0,
        T_own=4096, n_shared=1, I_shared=2048, routing="logits", ring_rows=16384,
        minibatch_rows=512),
    "ep64_share_mxfp8_pool262144_d7168_e256_top8": Workload(
        name="ep64_share_mxfp8_pool262144_d7168_e256_top8", dtype="mxfp8", T_pool=262144,
        d=7168, E=256, k=8, I=2048, e0=0, E_l=4, tokens_per_rank=4096, own_begin=0,
        T_own=4096, n_shared=1, I_shared=2048, routing="logits", ring_rows=16384,
        minibatch_rows=512),
    "ep96_zipf_bf16_pool196608_d7168_e384_top8_ring16384": Workload(
        name="ep96_zipf_bf16_pool196608_d7168_e384_top8_ring16384", dtype="bf16",
        T_pool=196608, d=7168, E=384, k=8, I=2048, e0=0, E_l=4, tokens_per_rank=2048,
        own_begin=0, T_own=2048, n_shared=1, I_shared=2048, routing="logits",
        zipf_beta=ZIPF_BETA_EP96, ring_rows=16384, minibatch_rows=512),
    # the MXFP8 share's shapes with MXFP4 operands (the MX sibling of the MXFP8 path)
    "ep64_share_mxfp4_pool262144_d7168_e256_top8": Workload(
        name="ep64_share_mxfp4_pool262144_d7168_e256_top8", dtype="mxfp4", T_pool=262144,
        d=7168, E=256, k=8, I=2048, e0=0, E_l=4, tokens_per_rank=4096, own_begin=0,
        T_own=4096, n_shared=1, I_shared=2048, routing="logits", ring_rows=16384,
        minibatch_rows=512),
}

TINY, EP1, EP64, EP64_MX, EP96, EP64_MX4 = list(WORKLOADS)


def scaled(w: Workload, **kw) -> Workload:
    """A copy of w with some fields replaced (smaller parity cases of the same structure)."""
    import dataclasses
    return dataclasses.replace(w, **kw)


# ------------------------------------------------------------------ tensors of a workload

def _torch_dtype(w: Workload):
    return torch.float32 if w.dtype == "fp32" else torch.bfloat16


def x_rows(w: Workload, rows, device="cpu") -> torch.Tensor:
    """Pool rows, x ~ N(0,1), in the workload's storage type (fp32, or bf16 for bf16/mxfp8)."""
    return normal_rows(SEED, S_X, w.d, rows, 1.0, _torch_dtype(w), device)


def router_weight(w: Workload, device="cpu") -> torch.Tensor:
    """W_r [E, d] ~ N(0, 1/d)."""
    return normal_tensor((w.E, w.d), SEED, S_WR, 1.0 / math.sqrt(w.d), _torch_dtype(w), device)


def expert_weights(w: Workload, device="cpu"):
    """Local routed experts: W_gate, W_up [E_l, I, d] ~ N(0,1/d); W_down [E_l, d, I] ~ N(0,1/I).

    Expert e0+l's weights are rows l of the global [E, ...] streams, so the same expert has the
    same weights in every share of the layer."""
    dt = _torch_dtype(w)
    wg = normal_rows(SEED, S_WG, w.d, range(w.e0 * w.I, (w.e0 + w.E_l) * w.I),
                     1.0 / math.sqrt(w.d), dt, device).view(w.E_l, w.I, w.d)
    wu = normal_rows(SEED, S_WU, w.d, range(w.e0 * w.I, (w.e0 + w.E_l) * w.I),
                     1.0 / math.sqrt(w.d), dt, device).view(w.E_l, w.I, w.d)
    wd = normal_rows(SEED, S_WD, w.I, range(w.e0 * w.d, (w.e0 + w.E_l) * w.d),
                     1.0 / math.sqrt(w.I), dt, device).view(w.E_l, w.d, w.I)
    return wg, wu, wd


def shared_weights(w: Workload, device="cpu"):
    """Shared experts: [n_s, I_s, d] gate/up ~ N(0,1/d); [n_s, d, I_s] down ~ N(0,1/I_s)."""
    dt = _torch_dtype(w)
    sg = normal_tensor((w.n_shared, w.I_shared, w.d), SEED, S_SG, 1.0 / math.sqrt(w.d), dt, device)
    su = normal_tensor((w.n_shared, w.I_shared, w.d), SEED, S_SU, 1.0 / math.sqrt(w.d), dt, device)
    sd = normal_tensor((w.n_shared, w.d, w.I_shared), SEED, S_SD, 1.0 / math.sqrt(w.I_shared),
                       dt, device)
    return sg, su, sd


def zipf_bias(w: Workload) -> torch.Tensor:
    """Per-expert logit bias beta * (-s * ln rank_e), float32 [E]; zero when beta == 0.

    Experts 0..3 (the local experts of rank 0) take Zipf ranks 1, E/24, E/3 and E (1, 16, 128
    and 384 for E = 384); the other experts take the remaining ranks in a seeded order."""
    if w.zipf_beta == 0.0:
        return torch.zeros(w.E, dtype=torch.float32)
    fixed = []
    for r in (1, max(2, w.E // 24), max(3, w.E // 3), w.E):
        if r <= w.E and r not in fixed:
            fixed.append(r)
    fixed = fixed[:min(4, w.E)]
    rest = [r for r in range(1, w.E + 1) if r not in fixed]
    perm = seeded_permutation(SEED, S_PERM, len(rest)).tolist()
    ranks = fixed + [rest[p] for p in perm]
    b = [w.zipf_beta * (-ZIPF_S * math.log(r)) for r in ranks]
    return torch.tensor(b, dtype=torch.float64).to(torch.float32)


def pool_logits_rows(w: Workload, rows, device="cpu") -> torch.Tensor:
    """Given router logits of pool rows: N(0,1) float32 plus the Zipf bias (float32 add)."""
    z = normal_rows(SEED, S_LOGITS, w.E, rows, 1.0, torch.float32, device)
    if w.zipf_beta != 0.0:
        z = z + zipf_bias(w).to(device)
    return z
