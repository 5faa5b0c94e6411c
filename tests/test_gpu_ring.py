"""The persistent ring work loop (the default of mok_moe_forward).

Minibatches walk a ring of ring_rows / minibatch_rows slots: the gate/up tiles of minibatch m
write ring slot m % slots and wait until the down tiles of the minibatch that last used the
slot are done; the down tiles of m wait for all up tiles of m (MXFP8: the gather + quantise
items of m also wait for the up tiles of the slot's previous minibatch). No route is dropped
however small the ring. The ring changes the schedule only: outputs must match the oracle
and be bit-identical to the stage-ordered launches (MOK_FLAG_NO_RING), across ring sizes,
minibatch sizes and reruns, with the device error word left at 0."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _layer import TOL, gpu_layer, gpu_topk, make_inputs, rel_err, to_np
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _outputs(layer):
    """Written outputs: the local routes' slot rows, S and y (as int16 bit patterns)."""
    n = int(layer.inter["offsets"][-1])
    rid = layer.inter["route_ids"][:n].long()
    outs = [layer.y_slots[rid]]
    outs += [t for t in (layer.y_shared, layer.y) if t is not None]
    return [o.clone().view(torch.int32 if o.dtype == torch.float32 else torch.int16) for o in outs]


def _run(wl, inp, topk, flags, mb=None, ring=None):
    layer = gpu_layer(wl, inp, topk=topk, flags=flags, mb=mb, ring=ring)
    layer.forward()
    torch.cuda.synchronize()
    assert layer.device_error() == 0
    return layer


@pytest.mark.parametrize("name", list(SMALL))
def test_ring_small_layers_match_oracle(name):
    import routing_grouped_expert_gemm_amd as mok
    wl = SMALL[name]
    inp = make_inputs(wl, DEV)
    topk = gpu_topk(inp["logits"], wl.k) if wl.routing == "logits" else None
    print(f"ring small layer {name}: ring_rows={wl.ring_rows} mb={wl.minibatch_rows}", flush=True)
    layer = _run(wl, inp, topk, 0)
    cpu = {k: (v.cpu() if v is not None else None) for k, v in inp.items()}
    if wl.routing == "router":
        ref = oracle.moe_forward(wl, cpu["x"], w_router=cpu["w_router"], wg=cpu["wg"],
                                 wu=cpu["wu"], wd=cpu["wd"], sg=cpu["sg"], su=cpu["su"],
                                 sd=cpu["sd"])
    else:
        ridx, rw = oracle.topk(cpu["logits"], wl.k)
        assert np.array_equal(to_np(topk[0]), ridx)
        ref = oracle.moe_forward(wl, cpu["x"], wg=cpu["wg"], wu=cpu["wu"], wd=cpu["wd"],
                                 sg=cpu["sg"], su=cpu["su"], sd=cpu["sd"], topk_in=(ridx, rw))
    plan = ref["plan"]
    tol = TOL[wl.dtype]
    assert rel_err(to_np(layer.y_slots)[plan["route_ids"]], ref["P"]) <= tol
    if wl.n_shared:
        assert rel_err(to_np(layer.y_shared), ref["y_shared"]) <= tol
    if wl.full_layer:
        assert rel_err(to_np(layer.y), ref["y"]) <= tol


@pytest.mark.parametrize("name", ["full_bf16", "share_mxfp8", "share_mxfp4", "zipf_bf16",
                                  "tiny_fp32"])
def test_ring_bit_identical_to_stage_order_any_ring_and_minibatch(name):
    """Ring capacities down to a single slot (every minibatch waits for the previous one's
    down tiles) and minibatch sizes 128..1024 all give the stage-ordered bits."""
    import routing_grouped_expert_gemm_amd as mok
    wl = SMALL[name]
    inp = make_inputs(wl, DEV)
    topk = gpu_topk(inp["logits"], wl.k) if wl.routing == "logits" else None
    ref = _outputs(_run(wl, inp, topk, mok.MOK_FLAG_NO_RING))
    cases = [(128, 128), (128, 256), (128, 512), (256, 256), (256, 1024), (512, 2048),
             (1024, 1024), (128, 4096)]
    for mb, ring in cases:
        print(f"ring {name}: mb={mb} ring_rows={ring}", flush=True)
        got = _outputs(_run(wl, inp, topk, 0, mb=mb, ring=ring))
        for a, b in zip(got, ref):
            assert torch.equal(a, b), (mb, ring)


def test_ring_reruns_bit_identical():
    wl = SMALL["share_bf16"]
    inp = make_inputs(wl, DEV)
    topk = gpu_topk(inp["logits"], wl.k)
    layer = _run(wl, inp, topk, 0, mb=128, ring=256)
    first = _outputs(layer)
    for _ in range(9):
        layer.forward()
        torch.cuda.synchronize()
        assert layer.device_error() == 0
        for a, b in zip(_outputs(layer), first):
            assert torch.equal(a, b)


@pytest.mark.parametrize("name", [synth.EP96, synth.EP64_MX, synth.EP64_MX4])
def test_ring_full_share_workloads(name):
    """The skewed 384-expert share with its 16384-row ring at minibatch sizes 128..1024, and
    the MXFP8 share (gather + quantise items in the ring): bit-identical to the stage-ordered
    launches, and sampled rows within tolerance of the oracle."""
    import routing_grouped_expert_gemm_amd as mok
    wl = synth.WORKLOADS[name]
    inp = make_inputs(wl, DEV)
    topk = gpu_topk(inp["logits"], wl.k)
    mbs = (128, 256, 512, 1024) if name == synth.EP96 else (wl.minibatch_rows,)
    ref = None
    for mb in mbs:
        print(f"ring {name}: mb={mb} ring_rows={wl.ring_rows}", flush=True)
        base = _outputs(_run(wl, inp, topk, mok.MOK_FLAG_NO_RING, mb=mb))
        layer = _run(wl, inp, topk, 0, mb=mb)
        got = _outputs(layer)
        for a, b in zip(got, base):
            assert torch.equal(a, b), mb
        if ref is None:
            ref = got
        else:
            for a, b in zip(got, ref):
                assert torch.equal(a, b), mb
        del layer
    # sampled rows against the oracle (the last ring layer)
    layer = _run(wl, inp, topk, 0)
    cpu = {k: (v.cpu() if v is not None else None) for k, v in inp.items()}
    idx, w = oracle.topk(cpu["logits"], wl.k)
    assert np.array_equal(to_np(topk[0]), idx)
    rids = oracle.dispatch_plan(idx, wl.e0, wl.E_l, wl.tokens_per_rank)["route_ids"].astype(np.int64)
    n = len(rids)
    rng = np.random.default_rng(7)
    pick = np.sort(rng.choice(rids, size=min(1024, n), replace=False))
    mx = wl.dtype if wl.dtype in ("mxfp8", "mxfp4") else False
    refp = oracle.route_outputs(pick, cpu["x"][torch.from_numpy(pick // wl.k)], idx, w, wl.e0,
                                cpu["wg"], cpu["wu"], cpu["wd"], mx)
    assert rel_err(to_np(layer.y_slots[torch.from_numpy(pick).to(DEV)]), refp) <= TOL[wl.dtype]
