"""Layer-level edge cases on the GPU against the oracle, graph capture of the forward, and
routing that repeats an expert within a token.

Edge cases (the news summary's "no token dropping" read as: every route is computed whatever
the load): a local expert that receives no route, every route on one expert, k = E through
the router, no shared expert, a share with no own tokens. Graph capture: the whole forward is
recorded into a HIP graph and replayed; a host synchronisation or a host read of a count
inside the forward would make the capture fail (the news summary: no CPU-GPU sync)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _layer import TOL, gpu_layer, make_inputs, rel_err, to_np
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _routing(T, E, k, rng, allowed=None, forced=None):
    """Host routing: k distinct expert ids per token (from `allowed`), the first slot forced
    to `forced` when given; weights positive, summing to 1 per token."""
    allowed = np.arange(E) if allowed is None else np.asarray(allowed)
    idx = np.empty((T, k), np.int32)
    for t in range(T):
        pool = allowed if forced is None else allowed[allowed != forced]
        pick = rng.choice(pool, size=k if forced is None else k - 1, replace=False)
        idx[t] = pick if forced is None else np.concatenate([[forced], pick])
    w = rng.random((T, k)).astype(np.float32) + 0.1
    w = (w / w.sum(1, keepdims=True)).astype(np.float32)
    return idx, w


def _compare(wl, inp, layer, topk_np=None):
    cpu = {k: (v.cpu() if v is not None else None) for k, v in inp.items()}
    kw = dict(wg=cpu["wg"], wu=cpu["wu"], wd=cpu["wd"], sg=cpu["sg"], su=cpu["su"], sd=cpu["sd"])
    if topk_np is None:
        ref = oracle.moe_forward(wl, cpu["x"], w_router=cpu["w_router"], **kw)
        assert np.array_equal(to_np(layer.inter["topk_idx"]), ref["idx"])
    else:
        ref = oracle.moe_forward(wl, cpu["x"], topk_in=topk_np, **kw)
    plan = ref["plan"]
    for key in ("counts", "offsets"):
        assert np.array_equal(to_np(layer.inter[key]), plan[key]), key
    assert np.array_equal(to_np(layer.inter["route_ids"])[:plan["n"]], plan["route_ids"])
    tol = TOL[wl.dtype]
    if plan["n"]:
        assert rel_err(to_np(layer.y_slots)[plan["route_ids"]], ref["P"]) <= tol
    if wl.n_shared and wl.T_own:
        assert rel_err(to_np(layer.y_shared), ref["y_shared"]) <= tol
    if wl.full_layer:
        assert rel_err(to_np(layer.y), ref["y"]) <= tol
    assert layer.device_error() == 0
    return plan


BASE = synth.scaled(synth.WORKLOADS[synth.EP1], name="edge", T_pool=768, d=256, E=16, k=4,
                    I=192, E_l=16, tokens_per_rank=768, T_own=768, n_shared=1, I_shared=128,
                    minibatch_rows=128, ring_rows=1024)


@pytest.mark.parametrize("ring", [False, True])
def test_local_expert_with_no_route(ring):
    import routing_grouped_expert_gemm_amd as mok
    wl = synth.scaled(BASE, E_l=4, e0=4, routing="logits", tokens_per_rank=256, T_own=256,
                      own_begin=256)
    inp = make_inputs(wl, DEV)
    rng = np.random.default_rng(1)
    idx, w = _routing(wl.T_pool, wl.E, wl.k, rng, allowed=[e for e in range(wl.E) if e != 6])
    layer = gpu_layer(wl, inp, topk=(torch.from_numpy(idx).to(DEV), torch.from_numpy(w).to(DEV)),
                      flags=0 if ring else mok.MOK_FLAG_NO_RING)
    layer.forward()
    torch.cuda.synchronize()
    plan = _compare(wl, inp, layer, (idx, w))
    assert plan["counts"][2] == 0 and plan["counts"].sum() > 0


@pytest.mark.parametrize("ring", [False, True])
def test_every_route_on_one_expert(ring):
    """k = 1 and every token picks expert 3: one expert holds all 768 routes (six minibatches),
    the other fifteen none."""
    import routing_grouped_expert_gemm_amd as mok
    wl = synth.scaled(BASE, k=1, routing="logits")
    inp = make_inputs(wl, DEV)
    idx = np.full((wl.T_pool, 1), 3, np.int32)
    w = np.ones((wl.T_pool, 1), np.float32)
    layer = gpu_layer(wl, inp, topk=(torch.from_numpy(idx).to(DEV), torch.from_numpy(w).to(DEV)),
                      flags=0 if ring else mok.MOK_FLAG_NO_RING)
    layer.forward()
    torch.cuda.synchronize()
    plan = _compare(wl, inp, layer, (idx, w))
    assert plan["counts"][3] == wl.T_pool


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_k_equals_E_through_the_router(dtype):
    """Top-k with k = E picks every expert: the layer is the dense softmax mixture."""
    import routing_grouped_expert_gemm_amd as mok
    wl = synth.scaled(BASE, dtype=dtype, E=8, k=8, E_l=8, name=f"edge_kE_{dtype}")
    inp = make_inputs(wl, DEV)
    layer = gpu_layer(wl, inp, flags=mok.MOK_FLAG_NO_RING)
    layer.forward()
    torch.cuda.synchronize()
    plan = _compare(wl, inp, layer)
    assert plan["counts"].tolist() == [wl.T_pool] * wl.E


@pytest.mark.parametrize("ring", [False, True])
def test_no_shared_expert(ring):
    import routing_grouped_expert_gemm_amd as mok
    wl = synth.scaled(BASE, n_shared=0)
    inp = make_inputs(wl, DEV)
    layer = gpu_layer(wl, inp, flags=0 if ring else mok.MOK_FLAG_NO_RING)
    layer.forward()
    torch.cuda.synchronize()
    _compare(wl, inp, layer)


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8", "mxfp4"])
def test_share_without_own_tokens(dtype):
    import routing_grouped_expert_gemm_amd as mok
    wl = synth.scaled(BASE, dtype=dtype, I=256, E_l=4, e0=0, routing="logits",
                      tokens_per_rank=256, T_own=0, own_begin=0, name=f"edge_noown_{dtype}",
                      I_shared=256)
    inp = make_inputs(wl, DEV)
    rng = np.random.default_rng(2)
    idx, w = _routing(wl.T_pool, wl.E, wl.k, rng)
    layer = gpu_layer(wl, inp, topk=(torch.from_numpy(idx).to(DEV), torch.from_numpy(w).to(DEV)))
    layer.forward()
    torch.cuda.synchronize()
    _compare(wl, inp, layer, (idx, w))


# ------------------------------------------------------------------- graph capture

def _written(layer):
    n = int(layer.inter["offsets"][-1])
    rid = layer.inter["route_ids"][:n].long()
    outs = [layer.y_slots[rid]] + [t for t in (layer.y_shared, layer.y) if t is not None]
    return [o.clone().view(torch.int32 if o.dtype == torch.float32 else torch.int16) for o in outs]


@pytest.mark.parametrize("name,ring", [("full_bf16", True), ("full_bf16", False),
                                       ("share_mxfp8", False), ("share_mxfp8", True),
                                       ("share_mxfp4", False), ("full_bf16", "loop"),
                                       ("share_mxfp8", "loop")])
def test_forward_captured_in_a_hip_graph(name, ring):
    """The forward records into a HIP graph (so it makes no host synchronisation and reads
    nothing back), and every replay -- with eager work and synchronisations between them --
    gives the eager result bit for bit."""
    import routing_grouped_expert_gemm_amd as mok
    from _layer import gpu_topk
    wl = SMALL[name]
    inp = make_inputs(wl, DEV)
    topk = gpu_topk(inp["logits"], wl.k) if wl.routing == "logits" else None
    flags = {True: 0, False: mok.MOK_FLAG_NO_RING, "loop": mok.MOK_FLAG_STAGE_LOOP}[ring]
    layer = gpu_layer(wl, inp, topk=topk, flags=flags)
    layer.forward()
    torch.cuda.synchronize()
    ref = _written(layer)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward()                   # warm-up on the capture stream's side
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        layer.forward()
    torch.cuda.synchronize()
    for rep in range(3):
        layer.y_slots.fill_(0)
        if layer.y is not None:
            layer.y.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert layer.device_error() == 0
        for a, b in zip(_written(layer), ref):
            assert torch.equal(a, b), rep


# ------------------------------------------------------------------- repeated expert ids

def test_repeated_expert_ids_never_write_past_capacity():
    """A token naming one local expert in several of its slots (not top-k output) makes more
    local routes than route_ids holds (T_pool * min(k, E_l)). The plan counts every route but
    writes only below the capacity; the forward runs no tile and sets the overflow bit."""
    import routing_grouped_expert_gemm_amd as mok
    T, k, E, E_l = 512, 8, 16, 4
    idx = np.zeros((T, k), np.int32)                  # every slot -> expert 0
    cap = T * min(k, E_l)
    i32 = dict(dtype=torch.int32, device=DEV)
    route_ids = torch.full((cap + 4096,), -7, **i32)  # canary past the capacity
    counts = torch.empty(E_l, **i32)
    offsets = torch.empty(E_l + 1, **i32)
    rank_counts = torch.empty((E_l, 1), **i32)
    ws = torch.empty(mok.mok_dispatch_plan_workspace_bytes(T, k, E_l), dtype=torch.uint8,
                     device=DEV)
    mok.mok_dispatch_plan(torch.from_numpy(idx).to(DEV), E, 0, E_l, T, counts, offsets,
                          rank_counts, route_ids, ws)
    torch.cuda.synchronize()
    assert to_np(counts).tolist() == [T * k, 0, 0, 0]
    assert int(offsets[-1]) == T * k > cap
    assert np.array_equal(to_np(route_ids)[:cap], np.arange(cap))
    assert (to_np(route_ids)[cap:] == -7).all()
    # the forward with that routing
    wl = synth.scaled(BASE, E=E, k=k, E_l=E_l, routing="logits", tokens_per_rank=T, T_pool=T,
                      T_own=T)
    inp = make_inputs(wl, DEV)
    w = np.full((T, k), 1.0 / k, np.float32)
    layer = gpu_layer(wl, inp, topk=(torch.from_numpy(idx).to(DEV), torch.from_numpy(w).to(DEV)),
                      flags=mok.MOK_FLAG_NO_RING)
    layer.forward()
    torch.cuda.synchronize()
    assert layer.device_error() == mok.MOK_DEVERR_OVERFLOW
