"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times.

Routing, plan and per-(expert, rank) counts are compared in full and bit-exactly; the layer's
floating-point outputs on sampled rows that the oracle computes one by one (float64). Inputs
are generated on the GPU by the seeded generator; the oracle gets the same tensors (the
generator gives the same bits on every device, checked in test_gpu_parity)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _layer import TOL, gpu_layer, gpu_topk, make_inputs, rel_err, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
# local expert loads of the 384-expert Zipf share (oracle top-k of the seeded pool logits)
EP96_COUNTS = [16380, 7782, 4021, 2738]


def _cpu(inp):
    return {k: (v.cpu() if v is not None else None) for k, v in inp.items()}


def _sample(rng, n, size):
    return np.sort(rng.choice(n, size=min(n, size), replace=False))


def _check_plan(layer, ref_plan):
    for key in ("counts", "offsets", "rank_counts"):
        assert np.array_equal(to_np(layer.inter[key]).reshape(ref_plan[key].shape), ref_plan[key]), key
    n = ref_plan["n"]
    assert np.array_equal(to_np(layer.inter["route_ids"])[:n], ref_plan["route_ids"])


def _check_sampled_outputs(wl, layer, cpu, idx, w, plan, rng, n_routes=1024, n_own=None):
    """Sampled route slots (default 1024) and the own tokens' shared output (default: all of
    them) against the oracle, float64; idx and w are the oracle's own routing."""
    mx = wl.dtype if wl.dtype in ("mxfp8", "mxfp4") else False
    tol = TOL[wl.dtype]
    rids = plan["route_ids"].astype(np.int64)
    pick = rids[_sample(rng, len(rids), n_routes)]
    ref = oracle.route_outputs(pick, cpu["x"][torch.from_numpy(pick // wl.k)], idx, w, wl.e0,
                               cpu["wg"], cpu["wu"], cpu["wd"], mx)
    got = to_np(layer.y_slots[torch.from_numpy(pick).to(DEV)])
    err_p = rel_err(got, ref)
    assert err_p <= tol, err_p
    own = np.arange(wl.T_own) if n_own is None else _sample(rng, wl.T_own, n_own)
    a = oracle._operand(cpu["x"][torch.from_numpy(wl.own_begin + own)], mx)
    S = oracle.shared_ffn(a, oracle._operand(cpu["sg"], mx), oracle._operand(cpu["su"], mx),
                          oracle._operand(cpu["sd"], mx), mx)
    err_s = rel_err(to_np(layer.y_shared[torch.from_numpy(own).to(DEV)]), S)
    assert err_s <= tol, err_s
    print(f"{wl.name}: {len(pick)} routes rel err {err_p:.2e}, {len(own)} own rows {err_s:.2e}",
          flush=True)
    return err_p, err_s


def _written(layer, plan):
    """The forward's written outputs as raw bits: local route slots, S, y."""
    rid = torch.from_numpy(plan["route_ids"].astype(np.int64)).to(DEV)
    outs = [layer.y_slots[rid]] + [t for t in (layer.y_shared, layer.y) if t is not None]
    return [o.clone().view(torch.int32 if o.dtype == torch.float32 else torch.int16) for o in outs]


def _reruns_bit_identical(layer, plan, n=10):
    first = _written(layer, plan)
    for _ in range(n - 1):
        layer.forward()
        torch.cuda.synchronize()
        assert layer.device_error() == 0
        for a, b in zip(_written(layer, plan), first):
            assert torch.equal(a, b)


@pytest.mark.parametrize("ring", [False, True])
def test_ep1_full_layer_bf16(ring):
    """T=8192, d=2048, 64 experts top-6, I=1408, 2 shared experts: the whole layer, every
    output element against the oracle's whole forward, in both work-loop modes; 10 runs
    bit-identical."""
    import routing_grouped_expert_gemm_amd as mok
    wl = synth.WORKLOADS[synth.EP1]
    inp = make_inputs(wl, DEV)
    layer = gpu_layer(wl, inp, flags=0 if ring else mok.MOK_FLAG_NO_RING)
    layer.forward()
    torch.cuda.synchronize()
    assert layer.device_error() == 0
    cpu = _cpu(inp)
    ref = oracle.moe_forward(wl, cpu["x"], w_router=cpu["w_router"], wg=cpu["wg"], wu=cpu["wu"],
                             wd=cpu["wd"], sg=cpu["sg"], su=cpu["su"], sd=cpu["sd"])
    logits = oracle.router_logits(cpu["x"], cpu["w_router"])
    assert np.array_equal(to_np(layer.inter["logits"]), logits)
    assert np.array_equal(to_np(layer.inter["topk_idx"]), ref["idx"])
    np.testing.assert_allclose(to_np(layer.inter["topk_w"]), ref["w"], rtol=2e-6, atol=1e-7)
    plan = ref["plan"]
    _check_plan(layer, plan)
    mean = wl.T_pool * wl.k / wl.E
    assert plan["counts"].min() >= 0.8 * mean and plan["counts"].max() <= 1.2 * mean
    tol = TOL["bf16"]
    err_p = rel_err(to_np(layer.y_slots)[plan["route_ids"]], ref["P"])
    err_s = rel_err(to_np(layer.y_shared), ref["y_shared"])
    err_y = rel_err(to_np(layer.y), ref["y"])
    print(f"ep1 ring={ring}: all {plan['n']} slots {err_p:.2e}, S {err_s:.2e}, y {err_y:.2e}",
          flush=True)
    assert err_p <= tol and err_s <= tol and err_y <= tol
    _reruns_bit_identical(layer, plan, 10)


@pytest.mark.parametrize("name,ring", [(synth.EP64, False), (synth.EP64, True),
                                       (synth.EP64_MX, False), (synth.EP96, False),
                                       (synth.EP64_MX4, False)])
def test_share_workloads(name, ring):
    """One rank's share: pool of 64 x 4096 (or 96 x 2048) tokens, d=7168, 4 local experts.
    Routing and plan bit-exact over the whole pool; 1024 sampled route slots and every own
    token's shared output against the oracle; reruns bit-identical (10 for MXFP8)."""
    import routing_grouped_expert_gemm_amd as mok
    wl = synth.WORKLOADS[name]
    inp = make_inputs(wl, DEV)
    idx_g, w_g = gpu_topk(inp["logits"], wl.k)
    cpu = _cpu(inp)
    idx, w = oracle.topk(cpu["logits"], wl.k)
    assert np.array_equal(to_np(idx_g), idx)
    np.testing.assert_allclose(to_np(w_g), w, rtol=2e-6, atol=1e-7)
    del cpu["logits"]
    layer = gpu_layer(wl, inp, topk=(idx_g, w_g), flags=0 if ring else mok.MOK_FLAG_NO_RING)
    layer.forward()
    torch.cuda.synchronize()
    assert layer.device_error() == 0
    plan = oracle.dispatch_plan(idx, wl.e0, wl.E_l, wl.tokens_per_rank)
    _check_plan(layer, plan)
    if name == synth.EP96:
        assert plan["counts"].tolist() == EP96_COUNTS   # calibrated Zipf load
    rng = np.random.default_rng(12)
    _check_sampled_outputs(wl, layer, cpu, idx, w, plan, rng)
    _reruns_bit_identical(layer, plan, 10 if wl.dtype.startswith("mx") else 2)


def test_zipf_share_minibatch_sweep_bit_identical():
    """The skewed share at minibatch sizes 128..1024 gives the same bits."""
    import routing_grouped_expert_gemm_amd as mok
    wl = synth.WORKLOADS[synth.EP96]
    inp = make_inputs(wl, DEV)
    topk = gpu_topk(inp["logits"], wl.k)
    ref = None
    for mb in (128, 256, 512, 1024):
        layer = gpu_layer(wl, inp, topk=topk, mb=mb, flags=mok.MOK_FLAG_NO_RING)
        layer.forward()
        torch.cuda.synchronize()
        n = int(layer.inter["offsets"][-1])
        rid = layer.inter["route_ids"][:n].long()
        out = (layer.y_slots[rid].clone(), layer.y_shared.clone())
        if ref is None:
            ref = out
        else:
            assert torch.equal(out[0].view(torch.int16), ref[0].view(torch.int16))
            assert torch.equal(out[1].view(torch.int16), ref[1].view(torch.int16))
        del layer


class _Events:
    """2 * MOK_N_STAGES timing events through the HIP runtime."""

    def __init__(self, n):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.ev = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(h)) == 0
            self.ev[i] = h

    def elapsed_ms(self, a, b):
        out = self.ct.c_float(0)
        rc = self.hip.hipEventElapsedTime(self.ct.byref(out), self.ev[a], self.ev[b])
        return rc, out.value


@pytest.mark.parametrize("dtype,ring", [("fp32", False), ("fp32", True), ("mxfp8", False)])
def test_stage_events_time_every_stage(dtype, ring):
    """Every stage's event pair is recorded (on its kernels, or as markers for a stage that
    launches nothing), the stages that run kernels take positive time, and a timed forward
    gives the same bits as an untimed one."""
    import ctypes
    import dataclasses
    import routing_grouped_expert_gemm_amd as mok
    wl = dataclasses.replace(synth.WORKLOADS[synth.TINY], dtype=dtype,
                             name=f"tiny_{dtype}_t64_d128_e8_top2")
    inp = make_inputs(wl, DEV)
    layer = gpu_layer(wl, inp, flags=0 if ring else mok.MOK_FLAG_NO_RING)
    layer.forward()
    torch.cuda.synchronize()
    y0 = layer.y.clone()
    n2 = 2 * mok.MOK_N_STAGES
    ev = _Events(n2)
    layer.args.stage_events = ctypes.cast(ev.ev, ctypes.c_void_p).value
    layer.forward()
    torch.cuda.synchronize()
    layer.args.stage_events = None
    assert torch.equal(layer.y.view(torch.int32 if dtype == "fp32" else torch.int16),
                       y0.view(torch.int32 if dtype == "fp32" else torch.int16))
    ms = {}
    for s in range(mok.MOK_N_STAGES):
        rc, t = ev.elapsed_ms(2 * s, 2 * s + 1)
        assert rc == 0, (s, rc)
        assert 0.0 <= t < 1000.0, (s, t)
        ms[s] = t
    running = [mok.MOK_STAGE_ROUTE, mok.MOK_STAGE_PLAN, mok.MOK_STAGE_UP, mok.MOK_STAGE_COMBINE,
               mok.MOK_STAGE_GATHER]
    if not ring:
        running.append(mok.MOK_STAGE_DOWN)
    if dtype == "mxfp8":
        running.append(mok.MOK_STAGE_QUANT)
    for s in running:
        assert ms[s] > 0.0, (s, ms)
