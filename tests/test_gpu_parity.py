"""GPU parity: the HIP library through its C ABI against the CPU oracle on the same seeded
inputs. Integer results (logits-decided routing, plan, MXFP8 codes) must be bit-exact;
floating-point outputs within max|y-ref|/max|ref| <= 1e-4 (fp32), 1e-2 (bf16), 3e-2 (MXFP8);
reruns bit-identical."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _layer import TOL, gpu_layer, gpu_topk, make_inputs, rel_err, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _sync():
    torch.cuda.synchronize()


# --------------------------------------------------------------------- generator parity

def test_seeded_generator_on_gpu_and_cpu():
    """The counter hashes are bit-identical on both devices; the Box-Muller normals (float64
    log and cosine, whose last bit may differ between devices) agree to one float32 ulp and are
    nearly all identical. Parity tests never rely on this: they copy one tensor to both sides."""
    idx = torch.arange(0, 1 << 20, dtype=torch.int64)
    for j in (0, 1):
        assert torch.equal(synth.u32(0, 1, j, idx.to(DEV)).cpu(), synth.u32(0, 1, j, idx))
    g = synth.normal_flat(0, 1, 0, 1 << 20, 1.0, DEV).cpu()
    c = synth.normal_flat(0, 1, 0, 1 << 20, 1.0)
    diff = (g.view(torch.int32).long() - c.view(torch.int32).long()).abs()
    assert int(diff.max()) <= 1
    assert float((diff == 0).double().mean()) > 0.9999
    wz = synth.WORKLOADS[synth.EP96]
    a = synth.pool_logits_rows(wz, range(100, 110), DEV).cpu()
    b = synth.pool_logits_rows(wz, range(100, 110))
    assert float((a - b).abs().max()) <= 1e-6


# --------------------------------------------------------------------- routing

# E of 16, 32 or 64 with d a multiple of 16 take the fused router + top-k kernel (32 tokens a
# workgroup: T = 1, 45, 300, 1000 leave ragged last workgroups), the rest the two-launch path
@pytest.mark.parametrize("dtype,T,d,E,k", [("fp32", 64, 128, 8, 2), ("bf16", 300, 192, 64, 6),
                                           ("bf16", 97, 64, 130, 8), ("fp32", 33, 100, 5, 5),
                                           ("bf16", 1000, 2048, 64, 6), ("fp32", 130, 272, 20, 4),
                                           ("fp32", 45, 144, 16, 16), ("bf16", 70, 96, 32, 3),
                                           ("fp32", 257, 64, 64, 64), ("bf16", 1, 16, 16, 1),
                                           ("bf16", 96, 48, 32, 32)])
def test_route_bit_exact(dtype, T, d, E, k):
    import routing_grouped_expert_gemm_amd as mok
    tdt = torch.float32 if dtype == "fp32" else torch.bfloat16
    x = synth.normal_rows(0, 101, d, range(T), 1.0, tdt)
    wr = synth.normal_rows(0, 102, d, range(E), d ** -0.5, tdt)
    lg = torch.empty((T, E), device=DEV)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), device=DEV)
    mok.mok_route(x.to(DEV), wr.to(DEV), k, lg, idx, w)
    _sync()
    ref_lg = oracle.router_logits(x, wr)
    assert np.array_equal(to_np(lg), ref_lg)
    ref_idx, ref_w = oracle.topk(ref_lg, k)
    assert np.array_equal(to_np(idx), ref_idx)
    np.testing.assert_allclose(to_np(w), ref_w, rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("E,k", [(8, 1), (8, 2), (64, 6), (256, 8), (384, 8), (1000, 16), (40, 40)])
def test_topk_bit_exact_with_ties(E, k):
    rng = np.random.default_rng(E * 100 + k)
    T = 777
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[::3] = np.round(lg[::3] * 2) / 2                       # many exact ties
    lg[1, :] = 0.0
    lg[1, ::2] = -0.0                                         # +0 == -0
    lg[2, :] = -1.0
    idx, w = gpu_topk(torch.from_numpy(lg).to(DEV), k)
    _sync()
    ref_idx, ref_w = oracle.topk(lg, k)
    assert np.array_equal(to_np(idx), ref_idx)
    np.testing.assert_allclose(to_np(w), ref_w, rtol=2e-6, atol=1e-7)


# --------------------------------------------------------------------- plan

def _gpu_plan(idx_np, E, e0, E_l, tpr):
    import routing_grouped_expert_gemm_amd as mok
    T, k = idx_np.shape
    R = T // tpr
    i32 = dict(dtype=torch.int32, device=DEV)
    counts = torch.full((E_l,), -7, **i32)
    offsets = torch.full((E_l + 1,), -7, **i32)
    rank_counts = torch.full((E_l, R), -7, **i32)
    route_ids = torch.full((max(1, T * min(k, E_l)),), -7, **i32)
    ws = torch.empty(mok.mok_dispatch_plan_workspace_bytes(T, k, E_l), dtype=torch.uint8, device=DEV)
    mok.mok_dispatch_plan(torch.from_numpy(idx_np).to(DEV), E, e0, E_l, tpr, counts, offsets,
                          rank_counts, route_ids, ws)
    _sync()
    n = int(offsets[-1])
    return dict(counts=to_np(counts), offsets=to_np(offsets), rank_counts=to_np(rank_counts),
                route_ids=to_np(route_ids)[:n], untouched=to_np(route_ids)[n:])


def _check_plan(idx_np, E, e0, E_l, tpr):
    g = _gpu_plan(idx_np, E, e0, E_l, tpr)
    r = oracle.dispatch_plan(idx_np, e0, E_l, tpr)
    for key in ("counts", "offsets", "rank_counts", "route_ids"):
        assert np.array_equal(g[key], r[key]), key
    assert (g["untouched"] == -7).all()


def test_plan_worked_example():
    idx = np.zeros((16, 1), np.int32)
    for e, toks in {2: [0, 2, 9, 15], 5: [3, 8], 7: [1, 4, 5, 6]}.items():
        idx[toks, 0] = e
    g = _gpu_plan(idx, 8, 0, 8, 16)
    assert g["route_ids"][g["offsets"][2]:g["offsets"][3]].tolist() == [0, 2, 9, 15]
    assert g["route_ids"][g["offsets"][5]:g["offsets"][6]].tolist() == [3, 8]
    assert g["route_ids"][g["offsets"][7]:g["offsets"][8]].tolist() == [1, 4, 5, 6]
    _check_plan(idx, 8, 0, 8, 16)
    _check_plan(idx, 8, 5, 3, 4)


# (8192, 8, 256, ...), (16384, 4, ...) and (8192, 8, 64, ...) cut into whole chunks per source
# rank (the rank counts are then sums of chunk histograms), the rest straddle ranks
@pytest.mark.parametrize("T,k,E,e0,E_l,tpr", [(4096, 6, 64, 0, 64, 4096), (8192, 8, 256, 12, 4, 256),
                                               (3000, 2, 8, 3, 1, 1000), (64, 2, 8, 0, 8, 64),
                                               (20000, 8, 384, 380, 4, 2000), (1, 1, 1, 0, 1, 1),
                                               (4096, 2, 8, 0, 8, 16), (16384, 4, 32, 0, 32, 512),
                                               (8192, 8, 64, 0, 64, 8192)])
def test_plan_bit_exact_random(T, k, E, e0, E_l, tpr):
    rng = np.random.default_rng(T + E)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    _check_plan(idx, E, e0, E_l, tpr)


def test_plan_all_routes_on_one_expert_and_none_local():
    idx = np.zeros((5000, 2), np.int32)
    idx[:, 1] = 3
    _check_plan(idx, 8, 0, 4, 1000)       # experts 0 and 3 take everything, 1 and 2 nothing
    _check_plan(idx, 8, 4, 4, 1000)       # no local route at all


# --------------------------------------------------------------------- MXFP8 quantiser

def test_quantize_mxfp8_exhaustive_bf16_patterns():
    import routing_grouped_expert_gemm_amd as mok
    bits = np.arange(1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    f = f[np.isfinite(f)]
    rng = np.random.default_rng(9)
    # rows of 256: the raw patterns, and the patterns shuffled with per-row amplitude changes
    f = np.concatenate([f, rng.permutation(f)])
    f = f[: (len(f) // 256) * 256].reshape(-1, 256)
    f[::7, 5] = 0.0
    f[3] = 0.0                                              # all-zero blocks: scale 2^-127
    src = torch.from_numpy(f).to(torch.bfloat16)
    assert torch.equal(src.float(), torch.from_numpy(f))    # every value is a bf16 value
    codes = torch.empty(src.shape, dtype=torch.uint8, device=DEV)
    scales = torch.empty((src.shape[0], 8), dtype=torch.uint8, device=DEV)
    mok.mok_quantize_mxfp8(src.to(DEV), codes, scales)
    _sync()
    rc, rs = oracle.mxfp8_quantize(src)
    assert np.array_equal(to_np(scales), rs)
    assert np.array_equal(to_np(codes), rc)


def test_quantize_mxfp4_exhaustive_bf16_patterns():
    """Every finite bf16 pattern through mok_quantize_mxfp4, bit-exact against the oracle's
    MXFP4 codes (two a byte) and scales."""
    import routing_grouped_expert_gemm_amd as mok
    bits = np.arange(1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    f = f[np.isfinite(f)]
    rng = np.random.default_rng(19)
    f = np.concatenate([f, rng.permutation(f)])
    f = f[: (len(f) // 256) * 256].reshape(-1, 256)
    f[::7, 5] = 0.0
    f[3] = 0.0
    src = torch.from_numpy(f).to(torch.bfloat16)
    codes = torch.empty((src.shape[0], 128), dtype=torch.uint8, device=DEV)
    scales = torch.empty((src.shape[0], 8), dtype=torch.uint8, device=DEV)
    mok.mok_quantize_mxfp4(src.to(DEV), codes, scales)
    _sync()
    rc, rs = oracle.mxfp4_quantize(src)
    assert np.array_equal(to_np(scales), rs)
    assert np.array_equal(to_np(codes), rc)


def _f32_rounding_sweep(fp4, rows=1024, K=256, seed=23):
    """float32 blocks whose elements sit on, and a few ulps either side of, the midpoints of the
    E2M1 (fp4) or E4M3 grid after scaling, plus saturating values, zeros, signs and denormals.
    Each 32-element block gets its own shared exponent (its largest magnitude is fixed first)."""
    rng = np.random.default_rng(seed)
    if fp4:
        grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
        top, emax = 7.0, 2                           # |v| 2^-s < 8 = 2^(emax + 1)
    else:
        grid = np.unique(np.concatenate([np.arange(8) * 2.0 ** -9] +
                                        [np.arange(8, 16) * 2.0 ** (e - 3) for e in range(-6, 9)]))
        grid = grid[grid <= 448]
        top, emax = 500.0, 8
    mids = (grid[1:] + grid[:-1]) / 2
    out = np.empty((rows, K), np.float32)
    for r in range(rows):
        for b in range(K // 32):
            s = int(rng.integers(-60, 60))
            y = rng.choice(np.concatenate([mids, grid, [top, 6.5 if fp4 else 460.0]]), 32)
            y = y.astype(np.float32)
            ulps = rng.integers(-3, 4, 32).astype(np.int32)
            y = (y.view(np.int32) + np.where(y > 0, ulps, 0)).view(np.float32)
            y[0] = np.float32(top)                   # fixes the block's shared exponent
            v = np.ldexp(y.astype(np.float64), s).astype(np.float32)
            v *= np.where(rng.random(32) < 0.5, -1, 1).astype(np.float32)
            out[r, 32 * b:32 * b + 32] = v
    out[::9, 7] = 0.0
    out[::11, 9] = -0.0
    out[5, :32] = np.float32(1e-42)                  # denormal block
    out[6, :32] = rng.standard_normal(32).astype(np.float32)
    return out


@pytest.mark.parametrize("fp4", [False, True])
def test_quantize_mx_f32_rounding_boundaries(fp4):
    """mok_quantize_mxfp{8,4}_f32 (the H epilogue's encoders) on float32 values at and next to
    every rounding midpoint of the element grid, bit-exact against the oracle's codes and
    scales."""
    import routing_grouped_expert_gemm_amd as mok
    f = _f32_rounding_sweep(fp4)
    src = torch.from_numpy(f).to(DEV)
    rows, K = f.shape
    codes = torch.empty((rows, K // 2 if fp4 else K), dtype=torch.uint8, device=DEV)
    scales = torch.empty((rows, K // 32), dtype=torch.uint8, device=DEV)
    (mok.mok_quantize_mxfp4_f32 if fp4 else mok.mok_quantize_mxfp8_f32)(src, codes, scales)
    _sync()
    rc, rs = (oracle.mxfp4_quantize if fp4 else oracle.mxfp8_quantize)(f)
    assert np.array_equal(to_np(scales), rs)
    assert np.array_equal(to_np(codes), rc)


# --------------------------------------------------------------------- layer, small sizes

SMALL = {
    "tiny_fp32": synth.WORKLOADS[synth.TINY],
    "full_bf16": synth.scaled(synth.WORKLOADS[synth.EP1], name="full_bf16", T_pool=640, d=256,
                              E=16, k=4, I=192, E_l=16, tokens_per_rank=640, T_own=640,
                              n_shared=2, I_shared=128, minibatch_rows=128, ring_rows=4096),
    "share_bf16": synth.scaled(synth.WORKLOADS[synth.EP64], name="share_bf16", T_pool=2048, d=384,
                               E=64, k=8, I=192, e0=8, E_l=4, tokens_per_rank=256,
                               own_begin=512, T_own=256, I_shared=256, minibatch_rows=128,
                               ring_rows=1024),
    "share_mxfp8": synth.scaled(synth.WORKLOADS[synth.EP64_MX], name="share_mxfp8", T_pool=2048,
                                d=256, E=64, k=8, I=256, e0=4, E_l=4, tokens_per_rank=256,
                                own_begin=256, T_own=256, I_shared=128, minibatch_rows=128,
                                ring_rows=1024),
    "share_mxfp4": synth.scaled(synth.WORKLOADS[synth.EP64_MX4], name="share_mxfp4", T_pool=2048,
                                d=512, E=64, k=8, I=256, e0=4, E_l=4, tokens_per_rank=256,
                                own_begin=256, T_own=256, I_shared=256, minibatch_rows=128,
                                ring_rows=1024),
    # the fused router on a partial layer (local experts 8..15 of 32, four source ranks of 250
    # tokens, which straddle the plan's chunks)
    "part_router_bf16": synth.scaled(synth.WORKLOADS[synth.EP1], name="part_router_bf16",
                                     T_pool=1000, d=256, E=32, k=4, I=192, e0=8, E_l=8,
                                     tokens_per_rank=250, own_begin=250, T_own=250, n_shared=1,
                                     I_shared=128, minibatch_rows=128, ring_rows=1024),
    "zipf_bf16": synth.scaled(synth.WORKLOADS[synth.EP96], name="zipf_bf16", T_pool=4096,
                              d=256, E=96, k=8, I=128, e0=0, E_l=4, tokens_per_rank=256,
                              own_begin=0, T_own=256, I_shared=128, minibatch_rows=128,
                              ring_rows=512, zipf_beta=0.5),
}


def _run_and_compare(wl, flags, mb=None):
    import routing_grouped_expert_gemm_amd as mok
    inp = make_inputs(wl, DEV)
    topk = None
    if wl.routing == "logits":
        topk = gpu_topk(inp["logits"], wl.k)
    layer = gpu_layer(wl, inp, topk=topk, flags=flags, mb=mb)
    layer.forward()
    _sync()
    cpu = {k: (v.cpu() if v is not None else None) for k, v in inp.items()}
    if wl.routing == "router":
        ref = oracle.moe_forward(wl, cpu["x"], w_router=cpu["w_router"], wg=cpu["wg"],
                                 wu=cpu["wu"], wd=cpu["wd"], sg=cpu["sg"], su=cpu["su"],
                                 sd=cpu["sd"])
        assert np.array_equal(to_np(layer.inter["logits"]),
                              oracle.router_logits(cpu["x"], cpu["w_router"]))
        assert np.array_equal(to_np(layer.inter["topk_idx"]), ref["idx"])
        np.testing.assert_allclose(to_np(layer.inter["topk_w"]), ref["w"], rtol=2e-6, atol=1e-7)
    else:
        ridx, rw = oracle.topk(cpu["logits"], wl.k)
        assert np.array_equal(to_np(topk[0]), ridx)
        np.testing.assert_allclose(to_np(topk[1]), rw, rtol=2e-6, atol=1e-7)
        ref = oracle.moe_forward(wl, cpu["x"], wg=cpu["wg"], wu=cpu["wu"], wd=cpu["wd"],
                                 sg=cpu["sg"], su=cpu["su"], sd=cpu["sd"], topk_in=(ridx, rw))
    plan = ref["plan"]
    assert np.array_equal(to_np(layer.inter["counts"]), plan["counts"])
    assert np.array_equal(to_np(layer.inter["offsets"]), plan["offsets"])
    assert np.array_equal(to_np(layer.inter["rank_counts"]), plan["rank_counts"])
    assert np.array_equal(to_np(layer.inter["route_ids"])[:plan["n"]], plan["route_ids"])
    tol = TOL[wl.dtype]
    slots = to_np(layer.y_slots)[plan["route_ids"]]
    assert rel_err(slots, ref["P"]) <= tol
    if wl.n_shared:
        assert rel_err(to_np(layer.y_shared), ref["y_shared"]) <= tol
    if wl.full_layer:
        assert rel_err(to_np(layer.y), ref["y"]) <= tol
    assert layer.device_error() == 0
    return layer, ref


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_small_matches_oracle(name):
    import routing_grouped_expert_gemm_amd as mok
    _run_and_compare(SMALL[name], mok.MOK_FLAG_NO_RING)


@pytest.mark.parametrize("name", ["full_bf16", "share_mxfp8", "share_mxfp4"])
def test_layer_reruns_bit_identical_and_minibatch_invariant(name):
    import routing_grouped_expert_gemm_amd as mok
    wl = SMALL[name]
    inp = make_inputs(wl, DEV)
    topk = gpu_topk(inp["logits"], wl.k) if wl.routing == "logits" else None
    outs = []
    for mb in (128, 128, 256, 512, 1024, 128):
        layer = gpu_layer(wl, inp, topk=topk, mb=mb, ring=4096, flags=mok.MOK_FLAG_NO_RING)
        layer.forward()
        _sync()
        outs.append([t.clone() for t in (layer.y_slots, layer.y_shared, layer.y) if t is not None])
    # the slot rows of non-local routes are never written: compare the written rows only
    rid = layer.inter["route_ids"][: int(layer.inter["offsets"][-1])].long()
    for o in outs[1:]:
        assert torch.equal(o[0][rid].view(torch.int16), outs[0][0][rid].view(torch.int16))
        for a, b in zip(o[1:], outs[0][1:]):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
