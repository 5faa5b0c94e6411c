"""The forward's OWN MX operands (MXFP8, and MXFP4), read back from its workspace
(mok_moe_workspace_region), are bit-exact against the oracle's quantiser (OCP MX v1.0 rules;
the news summary names MXFP8 as a supported operand format).

The forward quantises every weight on the device with K-step-major scales and fuses the pull
gather into the quantisation of the A rows -- device code that mok_quantize_mxfp8 does not
run. Here each of those bytes is compared with oracle.mxfp8_quantize of the same bf16 source:
all routed and shared weight codes and scales, and every gathered A row of a stage-ordered
forward (where every minibatch keeps its own ring slot)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _layer import (gpu_layer, gpu_topk, kmajor_scales_to_rows, make_inputs,
                    stage_order_minibatches, to_np)
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _quantize(wl, src):
    return oracle.mxfp4_quantize(src) if wl.dtype == "mxfp4" else oracle.mxfp8_quantize(src)


def _weights_bit_exact(mok, layer, inp, wl):
    R = mok
    cases = [(R.MOK_REGION_WG_CODES, R.MOK_REGION_WG_SCALES, inp["wg"]),
             (R.MOK_REGION_WU_CODES, R.MOK_REGION_WU_SCALES, inp["wu"]),
             (R.MOK_REGION_WD_CODES, R.MOK_REGION_WD_SCALES, inp["wd"])]
    if wl.n_shared:
        cases += [(R.MOK_REGION_SG_CODES, R.MOK_REGION_SG_SCALES, inp["sg"]),
                  (R.MOK_REGION_SU_CODES, R.MOK_REGION_SU_SCALES, inp["su"]),
                  (R.MOK_REGION_SD_CODES, R.MOK_REGION_SD_SCALES, inp["sd"])]
    n_bytes = 0
    for rc, rs, w in cases:
        K = w.shape[-1]
        src = w.reshape(-1, K)
        codes, _ = layer.region(rc)
        scales, R_rows = layer.region(rs)
        ref_c, ref_s = _quantize(wl, src.cpu())
        got_c = to_np(codes).reshape(ref_c.shape)
        got_s = kmajor_scales_to_rows(to_np(scales), src.shape[0], K, R_rows)
        assert np.array_equal(got_s, ref_s), (rc, int((got_s != ref_s).sum()))
        assert np.array_equal(got_c, ref_c), (rc, int((got_c != ref_c).sum()))
        n_bytes += got_c.size
    return n_bytes


def _gathered_rows_bit_exact(layer, inp, wl, mb):
    import routing_grouped_expert_gemm_amd as mok
    counts = to_np(layer.inter["counts"])
    offsets = to_np(layer.inter["offsets"])
    rids = to_np(layer.inter["route_ids"])
    ring_rows, pool_rows = stage_order_minibatches(counts, offsets, rids, wl.k, mb, wl.own_begin,
                                                   wl.T_own, wl.n_shared > 0)
    codes, R_rows = layer.region(mok.MOK_REGION_A_CODES)
    scales, _ = layer.region(mok.MOK_REGION_A_SCALES)
    d = wl.d
    row_bytes = d // 2 if wl.dtype == "mxfp4" else d
    codes = codes.view(-1, row_bytes)[torch.from_numpy(ring_rows).to(DEV)]
    src = inp["x"][torch.from_numpy(pool_rows).to(DEV)]
    ref_c, ref_s = _quantize(wl, src.cpu())
    # scales of the selected ring rows (one matrix of R_rows rows)
    all_s = kmajor_scales_to_rows(to_np(scales), R_rows, d, R_rows)
    got_s = all_s[ring_rows]
    assert np.array_equal(got_s, ref_s), int((got_s != ref_s).sum())
    got_c = to_np(codes)
    assert np.array_equal(got_c, ref_c), int((got_c != ref_c).sum())
    return len(ring_rows)


@pytest.mark.parametrize("name", ["share_mxfp8", "share_mxfp4"])
@pytest.mark.parametrize("ring", [False, True])
def test_small_share_mx_operands_bit_exact(name, ring):
    import routing_grouped_expert_gemm_amd as mok
    wl = SMALL[name]
    inp = make_inputs(wl, DEV)
    topk = gpu_topk(inp["logits"], wl.k)
    layer = gpu_layer(wl, inp, topk=topk, flags=0 if ring else mok.MOK_FLAG_NO_RING)
    layer.forward()
    torch.cuda.synchronize()
    assert layer.device_error() == 0
    _weights_bit_exact(mok, layer, inp, wl)
    if not ring:
        assert _gathered_rows_bit_exact(layer, inp, wl, wl.minibatch_rows) > 0


@pytest.mark.parametrize("name", [synth.EP64_MX, synth.EP64_MX4])
def test_full_mx_share_forward_operands_bit_exact(name):
    """The 262144-row pool, d=7168, 4 local experts + 1 shared expert (I=2048) in MXFP8 and in
    MXFP4: every weight byte the forward quantised and every gathered row of the ~32768 routes
    and 4096 own tokens."""
    import routing_grouped_expert_gemm_amd as mok
    wl = synth.WORKLOADS[name]
    inp = make_inputs(wl, DEV)
    topk = gpu_topk(inp["logits"], wl.k)
    layer = gpu_layer(wl, inp, topk=topk, flags=mok.MOK_FLAG_NO_RING)
    layer.forward()
    torch.cuda.synchronize()
    assert layer.device_error() == 0
    print(f"mx operands {wl.name}: forward done", flush=True)
    n_w = _weights_bit_exact(mok, layer, inp, wl)
    assert n_w == (wl.E_l * 3 * wl.d * wl.I + 3 * wl.d * wl.I_shared) // (2 if wl.dtype == "mxfp4" else 1)
    n_a = _gathered_rows_bit_exact(layer, inp, wl, wl.minibatch_rows)
    assert n_a == int(to_np(layer.inter["offsets"])[-1]) + wl.T_own
    print(f"mx operands {wl.name}: {n_w} weight codes, {n_a} gathered rows bit-exact", flush=True)
