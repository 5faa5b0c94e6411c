"""Pins of the CPU oracle to facts outside itself (no GPU).

Each test fixes a part of the oracle against the pages' worked example, a closed form, an
invariant, a textbook special case or brute force on tiny inputs, so that a plausible slip
(a dropped term, a wrong sign or index, a transposed operand, a wrong tie rule) fails.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- worked example (pages)

def _read_worked_example():
    push, pull = {}, {}
    with open(os.path.join(GOLDEN, "worked_example_pull_dispatch.txt")) as f:
        for line in f:
            line = line.split("#")[0].split()
            if not line:
                continue
            if line[0] == "push":
                push[int(line[1][1:])] = int(line[2])
            elif line[0] == "pull":
                pull[int(line[1][1:])] = [int(v) for v in line[2:]]
    return push, pull


def _worked_example_routing():
    push, pull = _read_worked_example()
    idx = np.zeros((16, 1), np.int32)         # unassigned tokens go to expert 0
    for e, toks in pull.items():
        for t in toks:
            idx[t, 0] = e
    for t, e in push.items():                 # the page's two views agree
        assert idx[t, 0] == e
    return idx, pull


def test_worked_example_plan_reproduces_pull_lists():
    idx, pull = _worked_example_routing()
    plan = oracle.dispatch_plan(idx, e0=0, E_l=8, tokens_per_rank=16)
    for e, toks in pull.items():
        a, b = plan["offsets"][e], plan["offsets"][e + 1]
        assert plan["route_ids"][a:b].tolist() == toks   # k=1: route id == token id
        assert plan["counts"][e] == len(toks)
    assert plan["n"] == 16


def test_worked_example_through_topk_with_one_hot_logits():
    idx, pull = _worked_example_routing()
    logits = np.full((16, 8), -1.0, np.float32)
    logits[np.arange(16), idx[:, 0]] = 1.0
    tidx, tw = oracle.topk(logits, 1)
    assert (tidx == idx).all()
    assert (tw == 1.0).all()
    plan = oracle.dispatch_plan(tidx, 0, 8, 16)
    for e, toks in pull.items():
        assert plan["route_ids"][plan["offsets"][e]:plan["offsets"][e + 1]].tolist() == toks


def test_worked_example_local_share_of_experts_5_to_7():
    """One rank holding experts [5, 8) sees only E5's and E7's lists, in page order."""
    idx, pull = _worked_example_routing()
    plan = oracle.dispatch_plan(idx, e0=5, E_l=3, tokens_per_rank=4)
    assert plan["route_ids"][plan["offsets"][0]:plan["offsets"][1]].tolist() == pull[5]
    assert plan["route_ids"][plan["offsets"][2]:plan["offsets"][3]].tolist() == pull[7]
    assert plan["counts"].tolist() == [2, 0, 4]
    # source ranks of 4 tokens each: E5 takes tokens 3 (rank 0) and 8 (rank 2)
    assert plan["rank_counts"][0].tolist() == [1, 0, 1, 0]
    assert plan["rank_counts"][2].tolist() == [1, 3, 0, 0]     # E7: token 1; tokens 4, 5, 6


# ----------------------------------------------------------------- plan vs a sort

@pytest.mark.parametrize("seed", range(6))
def test_plan_equals_stable_sort_and_invariants(seed):
    rng = np.random.default_rng(seed)
    T, k, E = int(rng.integers(1, 40)) * 4, int(rng.integers(1, 5)), int(rng.integers(5, 12))
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    e0, E_l = int(rng.integers(0, E - 1)), 0
    E_l = int(rng.integers(1, E - e0 + 1))
    tpr = 4
    plan = oracle.dispatch_plan(idx, e0, E_l, tpr)
    flat = idx.reshape(-1)
    local = np.nonzero((flat >= e0) & (flat < e0 + E_l))[0]
    order = local[np.argsort(flat[local], kind="stable")]           # library stable sort
    assert plan["route_ids"].tolist() == order.tolist()
    assert plan["counts"].sum() == len(local)
    assert (np.diff(plan["offsets"]) == plan["counts"]).all() and plan["offsets"][0] == 0
    for e in range(E_l):
        reg = plan["route_ids"][plan["offsets"][e]:plan["offsets"][e + 1]]
        assert (flat[reg] == e0 + e).all() and (np.diff(reg) > 0).all()
        ranks = (reg // k) // tpr
        assert np.bincount(ranks, minlength=T // tpr).tolist() == plan["rank_counts"][e].tolist()


def test_plan_empty_and_all_on_one_expert():
    idx = np.zeros((8, 2), np.int32)
    idx[:, 1] = 1
    plan = oracle.dispatch_plan(idx, 2, 3, 8)       # no local route at all
    assert plan["n"] == 0 and plan["counts"].tolist() == [0, 0, 0]
    assert plan["offsets"].tolist() == [0, 0, 0, 0]
    plan = oracle.dispatch_plan(idx, 0, 1, 4)       # every slot-0 route on expert 0
    assert plan["route_ids"].tolist() == [0, 2, 4, 6, 8, 10, 12, 14]
    assert plan["rank_counts"].tolist() == [[4, 4]]


# ----------------------------------------------------------------- top-k and weights

def test_topk_matches_full_sort_with_ties():
    rng = np.random.default_rng(1)
    logits = rng.integers(-3, 4, size=(200, 9)).astype(np.float32)   # many exact ties
    logits[0, :] = 0.0
    logits[1, :] = 0.0
    logits[1, ::2] = -0.0                                            # +0 and -0 are equal
    k = 4
    idx, _ = oracle.topk(logits, k)
    for t in range(200):
        order = np.lexsort((np.arange(9), -logits[t].astype(np.float64)))
        assert idx[t].tolist() == order[:k].tolist()
    assert idx[0].tolist() == [0, 1, 2, 3] and idx[1].tolist() == [0, 1, 2, 3]


def test_topk_weights_are_renormalised_full_softmax():
    rng = np.random.default_rng(2)
    logits = (rng.standard_normal((300, 16)) * 3).astype(np.float32)
    for k in (1, 2, 6, 16):
        idx, w = oracle.topk(logits, k)
        full = np.exp(logits.astype(np.float64) - logits.max(1, keepdims=True))
        full /= full.sum(1, keepdims=True)
        sel = np.take_along_axis(full, idx.astype(np.int64), 1)
        np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-6, atol=1e-7)
        assert (np.diff(w, axis=1) <= 0).all()          # slots in descending weight
    _, w1 = oracle.topk(logits, 1)
    assert (w1 == 1.0).all()


# ----------------------------------------------------------------- router logits

def test_router_logits_bf16_chain_equals_sequential_exact_products():
    """bf16 x bf16 products are exact in float32, so an FMA chain is a plain float32 chain of
    adds; an independent numpy loop in that order must give the same bits."""
    g = torch.Generator().manual_seed(3)
    x = torch.randn(37, 96, generator=g).bfloat16()
    wr = (torch.randn(11, 96, generator=g) / 10).bfloat16()
    got = oracle.router_logits(x, wr)
    xf, wf = x.float().numpy(), wr.float().numpy()
    acc = np.zeros((37, 11), np.float32)
    for i in range(96):
        acc = (acc + np.outer(xf[:, i], wf[:, i]).astype(np.float32)).astype(np.float32)
    assert np.array_equal(got, acc)


def test_router_logits_fp32_within_summation_bound():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((20, 128)).astype(np.float32)
    wr = rng.standard_normal((8, 128)).astype(np.float32)
    got = oracle.router_logits(x, wr).astype(np.float64)
    exact = x.astype(np.float64) @ wr.astype(np.float64).T
    bound = 128 * 2.0 ** -24 * (np.abs(x).astype(np.float64) @ np.abs(wr).astype(np.float64).T)
    assert (np.abs(got - exact) <= bound).all()


# ----------------------------------------------------------------- MXFP8 codec

def _e4m3_table():
    """The 127 finite non-negative E4M3 values from the format's definition (bias 7)."""
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(vals)


def test_e4m3_known_codes():
    L = oracle.lib()
    for code, v in [(0x00, 0.0), (0x01, 2 ** -9), (0x07, 7 * 2 ** -9), (0x08, 2 ** -6), (0x38, 1.0),
                    (0x40, 2.0), (0x7E, 448.0), (0xB8, -1.0), (0xFE, -448.0), (0x80, -0.0)]:
        assert L.orc_e4m3_decode(code) == v
        assert math.copysign(1, L.orc_e4m3_decode(code)) == math.copysign(1, v)
    assert L.orc_e4m3_encode(-0.0, 0) == 0x80 and L.orc_e4m3_encode(0.0, 0) == 0x00
    assert L.orc_e4m3_encode(1e30, 0) == 0x7E                      # saturates, never NaN
    assert L.orc_mx_shared_exponent(1.0) == -8 and L.orc_mx_shared_exponent(448.0) == 0
    assert L.orc_mx_shared_exponent(0.0) == -127


def _bf16_all_finite():
    bits = np.arange(1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    return f[np.isfinite(f)]


def test_e4m3_encode_exhaustive_vs_nearest_search():
    """Every finite bf16 value times 2^-s for s in [-20, 20] against a brute-force nearest
    search over the E4M3 grid (ties to the even code), then saturation at 448."""
    table = _e4m3_table()
    L = oracle.lib()
    vals = _bf16_all_finite()
    rng = np.random.default_rng(5)
    sub = np.concatenate([vals[::37], rng.choice(vals, 3000, replace=False)])
    for s in range(-20, 21):
        a = np.abs(sub.astype(np.float64)) * 2.0 ** -s
        dist = np.abs(a[:, None] - table[None, :])
        best = dist.min(1, keepdims=True)
        cand = dist == best
        # among equidistant candidates pick the even code (even mantissa)
        codes = np.where(cand.sum(1) > 1, np.argmax(cand & (np.arange(127)[None, :] % 2 == 0), 1),
                         np.argmin(dist, 1))
        codes = np.where(a >= 448.0, 0x7E, codes)
        for v, c in zip(sub, codes):
            got = L.orc_e4m3_encode(float(v), s)
            assert got & 0x7F == c, (float(v), s, got, c)
            assert (got >> 7) == (1 if math.copysign(1, v) < 0 else 0)


def test_mxfp8_scale_is_exponent_field_and_grid_round_trips():
    vals = _bf16_all_finite()
    vals = vals[(vals != 0) & (np.abs(vals) >= 2 ** -126)]        # bf16 normals
    exp_field = ((vals.view(np.uint32) >> 23) & 0xFF).astype(np.int64) - 127
    L = oracle.lib()
    for v, e in zip(vals[::97], exp_field[::97]):
        assert L.orc_mx_shared_exponent(abs(float(v))) == max(-127, min(127, e - 8))
    table = _e4m3_table()
    rng = np.random.default_rng(6)
    for s in (-30, -8, 0, 5):
        blk = rng.choice(table, (64, 32)) * rng.choice([-1, 1], (64, 32))
        blk[:, 0] = 448.0                                       # amax fixes the scale at s
        v = (blk * 2.0 ** s).astype(np.float32)
        codes, scales = oracle.mxfp8_quantize(v)
        assert (scales == s + 127).all()
        assert np.array_equal(oracle.mxfp8_dequantize(codes, scales), v)


def test_mxfp8_quantize_error_bound():
    rng = np.random.default_rng(7)
    v = rng.standard_normal((50, 256)).astype(np.float32)
    q = oracle.mx_roundtrip(v)
    blk_max = np.abs(v.reshape(50, 8, 32)).max(2, keepdims=True)
    err = np.abs(q - v).reshape(50, 8, 32)
    # relative step of E4M3 is 2^-3, so RNE error <= 2^-4 of the value's binade; the
    # saturation region [448, 512) * 2^s adds at most 64 * 2^s < blk_max / 4.
    assert (err <= np.maximum(np.abs(v).reshape(50, 8, 32) * 2 ** -4 + blk_max * 2 ** -9 * 2,
                              blk_max / 4)).all()


# ----------------------------------------------------------------- SwiGLU closed form

def test_swiglu_ffn_permutation_matrices_closed_form():
    """W_gate, W_up, W_down permutation matrices (d = I): y[m] = silu(x[pg(pd(m))]) *
    x[pu(pd(m))]. A transposed operand, swapped gate/up or a wrong silu sign all fail."""
    rng = np.random.default_rng(8)
    n = 16
    pg, pu, pd = rng.permutation(n), rng.permutation(n), rng.permutation(n)
    Wg = np.zeros((n, n)); Wg[np.arange(n), pg] = 1
    Wu = np.zeros((n, n)); Wu[np.arange(n), pu] = 1
    Wd = np.zeros((n, n)); Wd[np.arange(n), pd] = 1
    x = rng.standard_normal((5, n))
    y = oracle.swiglu_ffn(x, Wg, Wu, Wd)
    sig = lambda z: 1 / (1 + np.exp(-z))
    ref = np.empty_like(x)
    for m in range(n):
        a, b = x[:, pg[pd[m]]], x[:, pu[pd[m]]]
        ref[:, m] = a * sig(a) * b
    np.testing.assert_allclose(y, ref, rtol=1e-14, atol=1e-14)
    # identity weights: the textbook SwiGLU silu(x) * x
    I = np.eye(n)
    np.testing.assert_allclose(oracle.swiglu_ffn(x, I, I, I), x * x * sig(x), rtol=1e-14)


# ----------------------------------------------------------------- whole layer

def _tiny_layer(seed=0, T=24, d=32, E=5, k=2, I=48, n_s=2, I_s=32, dtype="fp32"):
    wl = synth.scaled(synth.WORKLOADS[synth.TINY], T_pool=T, d=d, E=E, k=k, I=I, E_l=E,
                      tokens_per_rank=T, T_own=T, n_shared=n_s, I_shared=I_s, dtype=dtype)
    x = synth.x_rows(wl, range(T))
    wr = synth.router_weight(wl)
    wg, wu, wd = synth.expert_weights(wl)
    sg, su, sd = synth.shared_weights(wl)
    return wl, x, wr, wg, wu, wd, sg, su, sd


def _f64(t):
    return t.float().double().numpy()


def test_layer_brute_force_per_token():
    """The plan/gather/slot/combine path equals a per-token loop over the picks."""
    wl, x, wr, wg, wu, wd, sg, su, sd = _tiny_layer()
    out = oracle.moe_forward(wl, x, w_router=wr, wg=wg, wu=wu, wd=wd, sg=sg, su=su, sd=sd)
    logits = oracle.router_logits(x, wr)
    idx, w = oracle.topk(logits, wl.k)
    for t in range(wl.T_pool):
        xt = _f64(x[t:t + 1])
        ref = np.zeros((1, wl.d))
        for s in range(wl.n_shared):
            ref += oracle.swiglu_ffn(xt, _f64(sg[s]), _f64(su[s]), _f64(sd[s]))
        for j in range(wl.k):
            e = idx[t, j]
            ref += float(w[t, j]) * oracle.swiglu_ffn(xt, _f64(wg[e]), _f64(wu[e]), _f64(wd[e]))
        np.testing.assert_allclose(out["y"][t], ref[0], rtol=1e-12, atol=1e-12)


def test_layer_k_equals_E_unit_weights_is_dense_mixture():
    wl, x, wr, wg, wu, wd, sg, su, sd = _tiny_layer(k=5)
    T, E = wl.T_pool, wl.E
    idx = np.tile(np.arange(E, dtype=np.int32)[::-1], (T, 1)).copy()   # any order of all E
    w = np.ones((T, E), np.float32)
    out = oracle.moe_forward(wl, x, wg=wg, wu=wu, wd=wd, sg=sg, su=su, sd=sd, topk_in=(idx, w))
    xf = _f64(x)
    dense = oracle.shared_ffn(xf, [_f64(t) for t in sg], [_f64(t) for t in su], [_f64(t) for t in sd])
    for e in range(E):
        dense += oracle.swiglu_ffn(xf, _f64(wg[e]), _f64(wu[e]), _f64(wd[e]))
    np.testing.assert_allclose(out["y"], dense, rtol=1e-11, atol=1e-11)


def test_layer_k_equals_E_softmax_is_full_softmax_mixture():
    wl, x, wr, wg, wu, wd, sg, su, sd = _tiny_layer(k=5)
    out = oracle.moe_forward(wl, x, w_router=wr, wg=wg, wu=wu, wd=wd, sg=sg, su=su, sd=sd)
    xf = _f64(x)
    lg = xf @ _f64(wr).T
    p = np.exp(lg - lg.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    ref = oracle.shared_ffn(xf, [_f64(t) for t in sg], [_f64(t) for t in su], [_f64(t) for t in sd])
    for e in range(wl.E):
        ref += p[:, e:e + 1] * oracle.swiglu_ffn(xf, _f64(wg[e]), _f64(wu[e]), _f64(wd[e]))
    np.testing.assert_allclose(out["y"], ref, rtol=2e-6, atol=2e-6)


def test_layer_invariant_to_permuting_expert_ids():
    wl, x, wr, wg, wu, wd, sg, su, sd = _tiny_layer(seed=1, E=6, k=3)
    out = oracle.moe_forward(wl, x, w_router=wr, wg=wg, wu=wu, wd=wd, sg=sg, su=su, sd=sd)
    perm = torch.tensor([3, 0, 5, 1, 4, 2])
    out2 = oracle.moe_forward(wl, x, w_router=wr[perm], wg=wg[perm], wu=wu[perm], wd=wd[perm],
                              sg=sg, su=su, sd=sd)
    logits = oracle.router_logits(x, wr)
    srt = np.sort(logits, axis=1)
    assert (np.diff(srt, axis=1) != 0).all()           # no exact ties in the seeded data
    np.testing.assert_allclose(out2["y"], out["y"], rtol=1e-12, atol=1e-12)
    assert (perm.numpy()[out2["idx"]] == out["idx"]).all()   # new expert i is old perm[i]


def test_share_slots_match_full_layer_routes():
    """A rank's share (experts [2,4)) produces, at its local routes, the same scaled expert
    outputs the full layer uses; shared output on its own rows."""
    wl, x, wr, wg, wu, wd, sg, su, sd = _tiny_layer(E=6, k=2)
    full = oracle.moe_forward(wl, x, w_router=wr, wg=wg, wu=wu, wd=wd, sg=sg, su=su, sd=sd)
    share = synth.scaled(wl, e0=2, E_l=2, tokens_per_rank=8, own_begin=8, T_own=8)
    part = oracle.moe_forward(share, x, w_router=wr, wg=wg[2:4], wu=wu[2:4], wd=wd[2:4],
                              sg=sg, su=su, sd=sd)
    rid_full = full["plan"]["route_ids"]
    pos = {int(r): i for i, r in enumerate(rid_full)}
    for i, r in enumerate(part["plan"]["route_ids"]):
        np.testing.assert_allclose(part["P"][i], full["P"][pos[int(r)]], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(part["y_shared"], full["y_shared"][8:16], rtol=1e-12, atol=1e-14)
    assert part["y"] is None


def test_mx_layer_uses_dequantised_operands():
    """MXFP8 share == float64 layer run on the MXFP8 round-tripped operands, with the hidden
    activation also round-tripped along I."""
    wl, x, wr, wg, wu, wd, sg, su, sd = _tiny_layer(d=64, I=64, I_s=64, dtype="mxfp8")
    out = oracle.moe_forward(wl, x, w_router=wr, wg=wg, wu=wu, wd=wd, sg=sg, su=su, sd=sd)
    rt = lambda t: oracle.mx_roundtrip(t.float().numpy()).astype(np.float64)
    r = int(out["plan"]["route_ids"][0])
    t, e = r // wl.k, int(out["idx"].reshape(-1)[r])
    h = oracle.silu(rt(x[t:t + 1]) @ rt(wg[e]).T) * (rt(x[t:t + 1]) @ rt(wu[e]).T)
    h = oracle.mx_roundtrip(h.astype(np.float32)).astype(np.float64)
    ref = float(out["w"].reshape(-1)[r]) * (h @ rt(wd[e]).T)
    np.testing.assert_allclose(out["P"][0], ref[0], rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------- MXFP4 (OCP MX v1.0, E2M1)

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def test_e2m1_known_codes():
    """Values worked out by hand from the E2M1 grid (0, 0.5, 1, 1.5, 2, 3, 4, 6): midpoints go
    to the code with the even mantissa bit, everything past 6 saturates, the sign is bit 3."""
    L = oracle.lib()
    cases = [(0.0, 0), (0.24, 0), (0.25, 0), (0.26, 1), (0.5, 1), (0.74, 1), (0.75, 2),
             (1.0, 2), (1.25, 2), (1.26, 3), (1.5, 3), (1.75, 4), (2.5, 4), (2.51, 5), (3.0, 5),
             (3.5, 6), (4.0, 6), (5.0, 6), (5.01, 7), (6.0, 7), (7.99, 7), (1e9, 7)]
    for v, c in cases:
        assert L.orc_e2m1_encode(v, 0) == c, (v, L.orc_e2m1_encode(v, 0), c)
        assert L.orc_e2m1_encode(-v, 0) == (c | 8), v
        assert L.orc_e2m1_encode(v * 2.0 ** 5, 5) == c, v        # the scale is exact
    for c in range(16):
        assert L.orc_e2m1_decode(c) == (-1 if c & 8 else 1) * E2M1[c & 7]


def test_e2m1_encode_exhaustive_vs_nearest_search():
    """Every finite bf16 value (sampled) times 2^-s for s in [-20, 20] against a numpy nearest
    search over the 8 magnitudes, ties to the even code, saturation at 6."""
    L = oracle.lib()
    vals = _bf16_all_finite()
    rng = np.random.default_rng(15)
    sub = np.concatenate([vals[::53], rng.choice(vals, 2000, replace=False)])
    for s in range(-20, 21):
        a = np.abs(sub.astype(np.float64)) * 2.0 ** -s
        dist = np.abs(a[:, None] - E2M1[None, :])
        cand = dist == dist.min(1, keepdims=True)
        codes = np.where(cand.sum(1) > 1, np.argmax(cand & (np.arange(8)[None, :] % 2 == 0), 1),
                         np.argmin(dist, 1))
        codes = np.where(a >= 6.0, 7, codes)
        for v, c in zip(sub, codes):
            got = L.orc_e2m1_encode(float(v), s)
            assert got & 7 == c and (got >> 3) == (1 if math.copysign(1, v) < 0 else 0), (v, s)


def test_mxfp4_scale_packing_and_grid_round_trip():
    """Shared exponent = floor(log2 amax) - 2 from the float's exponent field; element 2i in the
    low nibble of byte i; E2M1 grid values times 2^s round-trip exactly."""
    L = oracle.lib()
    vals = _bf16_all_finite()
    vals = vals[(vals != 0) & (np.abs(vals) >= 2 ** -126)]
    exp_field = ((vals.view(np.uint32) >> 23) & 0xFF).astype(np.int64) - 127
    for v, e in zip(vals[::97], exp_field[::97]):
        assert L.orc_mx4_shared_exponent(abs(float(v))) == max(-127, min(127, e - 2))
    v = np.zeros((1, 32), np.float32)
    v[0, 0], v[0, 1], v[0, 2], v[0, 31] = 1.0, -6.0, 0.5, 3.0      # amax 6 -> s = 0
    codes, scales = oracle.mxfp4_quantize(v)
    assert scales[0, 0] == 127 and codes.shape == (1, 16)
    assert codes[0, 0] == (0x2 | (0xF << 4)) and codes[0, 1] == 0x1 and codes[0, 15] == (0x5 << 4)
    rng = np.random.default_rng(16)
    for s in (-30, -4, 0, 7):
        blk = rng.choice(E2M1, (64, 32)) * rng.choice([-1, 1], (64, 32))
        blk[:, 0] = 6.0
        x = (blk * 2.0 ** s).astype(np.float32)
        c, sc = oracle.mxfp4_quantize(x)
        assert (sc == s + 127).all()
        assert np.array_equal(oracle.mxfp4_dequantize(c, sc), x)


def test_mxfp4_quantize_error_bound():
    """|q - v| <= max(|v| / 3, amax / 16) per block: half a step (a quarter of the binade) for
    normals, a quarter of 2^s for the subnormal step, and saturation [6, 8) * 2^s."""
    rng = np.random.default_rng(17)
    v = rng.standard_normal((50, 256)).astype(np.float32)
    q = oracle.mx4_roundtrip(v)
    blk_max = np.abs(v.reshape(50, 8, 32)).max(2, keepdims=True)
    err = np.abs(q - v).reshape(50, 8, 32)
    assert (err <= np.maximum(np.abs(v).reshape(50, 8, 32) / 3, blk_max / 16) + 1e-12).all()


def test_mxfp4_layer_uses_dequantised_operands():
    wl, x, wr, wg, wu, wd, sg, su, sd = _tiny_layer(d=64, I=64, I_s=64, dtype="mxfp4")
    out = oracle.moe_forward(wl, x, w_router=wr, wg=wg, wu=wu, wd=wd, sg=sg, su=su, sd=sd)
    rt = lambda t: oracle.mx4_roundtrip(t.float().numpy()).astype(np.float64)
    r = int(out["plan"]["route_ids"][0])
    t, e = r // wl.k, int(out["idx"].reshape(-1)[r])
    h = oracle.silu(rt(x[t:t + 1]) @ rt(wg[e]).T) * (rt(x[t:t + 1]) @ rt(wu[e]).T)
    h = oracle.mx4_roundtrip(h.astype(np.float32)).astype(np.float64)
    ref = float(out["w"].reshape(-1)[r]) * (h @ rt(wd[e]).T)
    np.testing.assert_allclose(out["P"][0], ref[0], rtol=1e-12, atol=1e-12)
    # MXFP4 differs from MXFP8 (a coarser grid): the two layers do not coincide
    out8 = oracle.moe_forward(synth.scaled(wl, dtype="mxfp8"), x, w_router=wr, wg=wg, wu=wu,
                              wd=wd, sg=sg, su=su, sd=sd)
    assert np.abs(out["y"] - out8["y"]).max() > 1e-3


# ----------------------------------------------------------------- backward

def _fd_layer(seed=3, T=6, d=8, E=4, k=2, I=6, n_s=2, I_s=4):
    """A tiny layer in float64 with fixed routing, its loss sum(dy * y) and the pieces."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    wg, wu = rng.standard_normal((E, I, d)) / 3, rng.standard_normal((E, I, d)) / 3
    wd = rng.standard_normal((E, d, I)) / 3
    sg, su = rng.standard_normal((n_s, I_s, d)) / 3, rng.standard_normal((n_s, I_s, d)) / 3
    sd = rng.standard_normal((n_s, d, I_s)) / 3
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)) + 0.2
    dy = rng.standard_normal((T, d))

    def loss(x, wg, wu, wd, sg, su, sd, w):
        y = np.zeros((T, d))
        for t in range(T):
            for j in range(k):
                e = idx[t, j]
                y[t] += w[t, j] * oracle.swiglu_ffn(x[t:t + 1], wg[e], wu[e], wd[e])[0]
            for s in range(n_s):
                y[t] += oracle.swiglu_ffn(x[t:t + 1], sg[s], su[s], sd[s])[0]
        return float((dy * y).sum())

    wl = synth.scaled(synth.WORKLOADS[synth.TINY], T_pool=T, d=d, E=E, k=k, I=I, E_l=E,
                      tokens_per_rank=T, T_own=T, n_shared=n_s, I_shared=I_s, dtype="fp32")
    return wl, dict(x=x, wg=wg, wu=wu, wd=wd, sg=sg, su=su, sd=sd, w=w), idx, dy, loss


def test_backward_matches_finite_differences_of_the_forward():
    """Every gradient of the oracle's backward equals the central difference of the oracle's
    forward loss sum(dy * y) (float64, step 1e-6): x, all routed and shared weights and the
    routing weights. A dropped term, a wrong sign or a transposed operand fails here."""
    wl, P, idx, dy, loss = _fd_layer()
    g = oracle.moe_backward(wl, P["x"], idx, P["w"], P["wg"], P["wu"], P["wd"], P["sg"],
                            P["su"], P["sd"], dy=dy)
    # dtopk_w is per local route in plan order; put it back at [t, j]
    dw = np.zeros(idx.size)
    dw[g["plan"]["route_ids"]] = g["dtopk_w"]
    grads = dict(x=g["dx"], wg=g["dwg"], wu=g["dwu"], wd=g["dwd"], sg=g["dsg"], su=g["dsu"],
                 sd=g["dsd"], w=dw.reshape(idx.shape))
    rng = np.random.default_rng(4)
    h = 1e-6
    for name, grad in grads.items():
        for _ in range(6):
            pos = tuple(rng.integers(0, n) for n in P[name].shape)
            Pp = {kk: v.copy() for kk, v in P.items()}
            Pm = {kk: v.copy() for kk, v in P.items()}
            Pp[name][pos] += h
            Pm[name][pos] -= h
            fd = (loss(**Pp) - loss(**Pm)) / (2 * h)
            assert abs(fd - grad[pos]) <= 1e-6 * max(1.0, abs(fd)), (name, pos, fd, grad[pos])


def test_backward_share_equals_full_layer_routes():
    """A share's slot gradients and weight gradients are the full layer's at the share's
    experts when its slots receive the same upstream gradient."""
    wl, P, idx, dy, _ = _fd_layer(T=8)
    full = oracle.moe_backward(wl, P["x"], idx, P["w"], P["wg"], P["wu"], P["wd"], P["sg"],
                               P["su"], P["sd"], dy=dy)
    share = synth.scaled(wl, e0=1, E_l=2, tokens_per_rank=4, own_begin=4, T_own=4)
    slots = np.repeat(dy, wl.k, axis=0)
    part = oracle.moe_backward(share, P["x"], idx, P["w"], P["wg"][1:3], P["wu"][1:3],
                               P["wd"][1:3], P["sg"], P["su"], P["sd"], dy_slots=slots,
                               dy_shared=dy[4:8])
    fr = full["plan"]["route_ids"]
    loc = (idx.reshape(-1)[fr] >= 1) & (idx.reshape(-1)[fr] < 3)
    np.testing.assert_allclose(part["dx_slots"], full["dx_slots"][loc], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(part["dtopk_w"], full["dtopk_w"][loc], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(part["dwg"], full["dwg"][1:3], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(part["dx_shared"], full["dx_shared"][4:8], rtol=1e-12, atol=1e-12)
