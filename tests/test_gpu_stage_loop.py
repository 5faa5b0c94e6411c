"""The stage order run by one persistent launch (MOK_FLAG_STAGE_LOOP).

The two stage launches' tile tables are cut into per-XCD queues (a contiguous range of
minibatches each, up tiles then down tiles) that the persistent loop walks; a down tile waits
only for the up tiles of its own minibatch. It changes the schedule only: every tile runs the
same arithmetic on the same operands, so the outputs must be bit-identical to the two stage
launches (MOK_FLAG_NO_RING), whose agreement with the oracle the parity tests establish, with
the device error word left at 0. One layer is also compared with the oracle directly."""
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
    """Written outputs: the local routes' slot rows, S and y (as integer bit patterns)."""
    n = int(layer.inter["offsets"][-1])
    rid = layer.inter["route_ids"][:n].long()
    outs = [layer.y_slots[rid]]
    outs += [t for t in (layer.y_shared, layer.y) if t is not None]
    return [o.clone().view(torch.int32 if o.dtype == torch.float32 else torch.int16) for o in outs]


def _run(wl, inp, topk, flags, mb=None):
    layer = gpu_layer(wl, inp, topk=topk, flags=flags, mb=mb)
    layer.forward()
    torch.cuda.synchronize()
    assert layer.device_error() == 0
    return layer


@pytest.mark.parametrize("name", list(SMALL))
def test_stage_loop_bit_identical_to_stage_launches(name):
    import routing_grouped_expert_gemm_amd as mok
    wl = SMALL[name]
    inp = make_inputs(wl, DEV)
    topk = gpu_topk(inp["logits"], wl.k) if wl.routing == "logits" else None
    for mb in (None, 128, 512):
        print(f"stage loop {name}: mb={mb}", flush=True)
        ref = _outputs(_run(wl, inp, topk, mok.MOK_FLAG_NO_RING, mb))
        got = _outputs(_run(wl, inp, topk, mok.MOK_FLAG_STAGE_LOOP, mb))
        for a, b in zip(got, ref):
            assert torch.equal(a, b), (name, mb)


def test_stage_loop_small_layer_matches_oracle():
    import routing_grouped_expert_gemm_amd as mok
    wl = SMALL["full_bf16"]
    inp = make_inputs(wl, DEV)
    print("stage loop full_bf16 against the oracle", flush=True)
    layer = _run(wl, inp, None, mok.MOK_FLAG_STAGE_LOOP)
    cpu = {k: (v.cpu() if v is not None else None) for k, v in inp.items()}
    ref = oracle.moe_forward(wl, cpu["x"], w_router=cpu["w_router"], wg=cpu["wg"], wu=cpu["wu"],
                             wd=cpu["wd"], sg=cpu["sg"], su=cpu["su"], sd=cpu["sd"])
    plan = ref["plan"]
    tol = TOL[wl.dtype]
    assert rel_err(to_np(layer.y_slots)[plan["route_ids"]], ref["P"]) <= tol
    assert rel_err(to_np(layer.y_shared), ref["y_shared"]) <= tol
    assert rel_err(to_np(layer.y), ref["y"]) <= tol


@pytest.mark.parametrize("name", [synth.EP1, synth.EP64_MX])
def test_stage_loop_full_size_bit_identical_and_reruns(name):
    """Full-size layers (the EP=1 layer: 224 minibatches over 8 XCD queues; the MXFP8 share):
    bit-identical to the stage launches, and over five reruns."""
    import routing_grouped_expert_gemm_amd as mok
    wl = synth.WORKLOADS[name]
    inp = make_inputs(wl, DEV)
    topk = gpu_topk(inp["logits"], wl.k) if wl.routing == "logits" else None
    print(f"stage loop {name}: stage launches", flush=True)
    ref = _outputs(_run(wl, inp, topk, mok.MOK_FLAG_NO_RING))
    layer = gpu_layer(wl, inp, topk=topk, flags=mok.MOK_FLAG_STAGE_LOOP)
    for i in range(5):
        print(f"stage loop {name}: run {i}", flush=True)
        layer.forward()
        torch.cuda.synchronize()
        assert layer.device_error() == 0
        for a, b in zip(_outputs(layer), ref):
            assert torch.equal(a, b), (name, i)
