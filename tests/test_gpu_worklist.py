"""The device work list that the plan's last workgroup builds, read back from the forward's
workspace (MOK_REGION_WORKLIST) and compared entry by entry with the scheduling models of
test_tile_order (stage-ordered tables) and test_ring_order (ring order, slots), fed with the
oracle's per-expert counts. Covers work lists built in LDS (up to 1024 minibatches) and in
place in global memory (more)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _layer import gpu_layer, make_inputs, to_np
from test_ring_order import layout as ring_layout
from test_tile_order import stage_table

pytestmark = pytest.mark.gpu
DEV = "cuda"
BM, BN = 256, 256                 # GEMM tile rows and B-tile rows
XB_N, XB_ND = 4, 8                # N tiles per block of the up / down tables
G_ROWS = 64                       # rows of one gather item (MX ring)
KIND_SHIFT = 28
KINDS = {"U": 0, "D": 1, "G": 2}

CASES = {
    "share_bf16": synth.scaled(synth.WORKLOADS[synth.EP64], name="wl_share_bf16", T_pool=2048,
                               d=384, E=64, k=8, I=192, e0=8, E_l=4, tokens_per_rank=256,
                               own_begin=512, T_own=256, I_shared=256, minibatch_rows=128,
                               ring_rows=1024),
    "share_mxfp8": synth.scaled(synth.WORKLOADS[synth.EP64_MX], name="wl_share_mxfp8",
                                T_pool=2048, d=256, E=64, k=8, I=256, e0=4, E_l=4,
                                tokens_per_rank=256, own_begin=256, T_own=256, I_shared=128,
                                minibatch_rows=128, ring_rows=1024),
    # shared down tiles longer than the routed ones (n_shared * I_shared > I): listed first
    "layer_bf16": synth.scaled(synth.WORKLOADS[synth.EP1], name="wl_layer_bf16", T_pool=640,
                               d=256, E=16, k=4, I=128, E_l=16, tokens_per_rank=640, T_own=640,
                               n_shared=2, I_shared=256, minibatch_rows=128, ring_rows=2048),
    # more than 1024 minibatches: the tables are built in global memory, in two chunks, the
    # first holding exactly 1024 minibatches
    "many_mb_bf16": synth.scaled(synth.WORKLOADS[synth.EP1], name="wl_many_mb", T_pool=32768,
                                 d=256, E=64, k=6, I=128, E_l=64, tokens_per_rank=32768,
                                 T_own=32768, n_shared=1, I_shared=128, minibatch_rows=128,
                                 ring_rows=4096),
}


def _oracle_topk(wl, cpu):
    lg = (oracle.router_logits(cpu["x"], cpu["w_router"]) if wl.routing == "router"
          else cpu["logits"])
    return oracle.topk(lg, wl.k)


def _read(layer):
    import routing_grouped_expert_gemm_amd as mok
    buf, _ = layer.region(mok.MOK_REGION_WORKLIST)
    return parse_worklist(buf.view(torch.int32).cpu().numpy().astype(np.int64))


def parse_worklist(w):
    """The work list's header, per-minibatch tables and tile tables (int64 arrays)."""
    cap, cap_u, cap_d, cap_r = (int(v) for v in w[44:48])
    H = 48
    tab = (H + 15 * cap + 7 + 3) & ~3
    arr = lambda o, n: w[o:o + n]
    n_mb = int(w[0])
    return dict(
        n_mb=n_mb, n_u=int(w[1]), n_d=int(w[2]), err=int(w[4]), n_r=int(w[5]),
        affine=int(w[6]), xb=w[8:17], xr=w[17:26],
        grp=arr(H, n_mb), r0=arr(H + cap, n_mb), nr=arr(H + 2 * cap, n_mb),
        us=arr(H + 3 * cap, n_mb + 1), ds=arr(H + 4 * cap + 1, n_mb + 1),
        gs=arr(H + 5 * cap + 2, n_mb + 1), slot=arr(H + 9 * cap + 3, n_mb),
        prev=arr(H + 10 * cap + 3, n_mb), rpre=arr(H + 11 * cap + 3, n_mb + 1),
        utab=w[tab:tab + 4 * cap_u].reshape(-1, 4),
        dtab=w[tab + 4 * cap_u:tab + 4 * (cap_u + cap_d)].reshape(-1, 4),
        rtab=w[tab + 4 * (cap_u + cap_d):tab + 4 * (cap_u + cap_d + cap_r)].reshape(-1, 4))


def _check(wl, layer, counts, offsets, ring):
    return check_worklist(wl, _read(layer), counts, offsets, ring)


def check_loop_table(got, ent, nu, nd, grp, E_l, wl):
    """The persistent stage-order table: every gate/up and down tile exactly once; per queue
    (XCD segment; one queue without the split) all up tiles before all down tiles, and every
    down tile's minibatch with all its up tiles in the same queue (so each wait points earlier
    in its own queue and at data produced under the same L2); a whole expert keeps the stage
    table's order; the queues' work (K steps) within one unit of an even share."""
    n, n_r, xr = len(nu), got["n_r"], [int(v) for v in got["xr"]]
    rt = [tuple(int(v) for v in row) for row in got["rtab"][:n_r]]
    want = set()
    for m in range(n):
        for k, cnt in (("U", nu[m]), ("D", nd[m])):
            for l in range(cnt):
                e = ent(m, l)
                e[1] = (KINDS[k] << KIND_SHIFT) | l
                want.add(tuple(e))
    assert len(rt) == len(want) and set(rt) == want
    segs = [(xr[x], xr[x + 1]) for x in range(8)] if got["affine"] else [(0, n_r)]
    assert xr[0] == 0 and all(a <= b for a, b in segs) and segs[-1][1] == n_r
    kind = lambda e: e[1] >> KIND_SHIFT
    seg_of = {}
    for q, (a, b) in enumerate(segs):
        kinds = [kind(e) for e in rt[a:b]]
        assert kinds == sorted(kinds), "up tiles first"
        for e in rt[a:b]:
            seg_of.setdefault(e[0], set()).add(q)
    assert all(len(v) == 1 for v in seg_of.values()), "a minibatch in one queue"
    # an expert wholly in one queue keeps the stage tables' order there
    key = lambda e: (e[0], e[1] & ((1 << KIND_SHIFT) - 1))
    for tab, k in ((got["utab"], "U"), (got["dtab"], "D")):
        stage = [key(tuple(int(v) for v in row)) for row in tab[:got["n_u" if k == "U" else "n_d"]]]
        for g in set(grp):
            ms = [m for m in range(n) if grp[m] == g]
            qs = set().union(*(seg_of[m] for m in ms))
            if len(qs) != 1:
                continue
            a, b = segs[next(iter(qs))]
            inq = [key(e) for e in rt[a:b] if kind(e) == KINDS[k] and grp[e[0]] == g]
            assert inq == [e for e in stage if grp[e[0]] == g], (k, g)
    ks_u, ks_dr, ks_ds = wl.d // 64, wl.I // 64, wl.n_shared * wl.I_shared // 64
    if got["affine"]:
        work = [nu[m] * ks_u + nd[m] * (ks_dr if grp[m] < E_l else ks_ds) for m in range(n)]
        q_work = [0] * len(segs)
        for m in range(n):
            q_work[next(iter(seg_of[m]))] += work[m]
        total = sum(work)
        unit = max(sum(work[m] for m in range(n) if grp[m] == g) for g in set(grp) if g < E_l)
        unit = min(unit, total // 32 + max(work))
        assert max(q_work) <= total / 8 + unit, (q_work, total, unit)


def check_worklist(wl, got, counts, offsets, ring):
    """Compares a parsed work list with the models; returns the number of minibatches. ring:
    False (stage tables), True (ring order) or "loop" (stage tables and the persistent
    stage-order table)."""
    loop = ring == "loop"
    ring = ring is True
    assert got["err"] == 0
    E_l, mb = wl.E_l, wl.minibatch_rows
    I_sh = wl.n_shared * wl.I_shared
    nN_r, nN_s, nD = -(-wl.I // (BN // 2)), -(-I_sh // (BN // 2)), -(-wl.d // BN)
    n_own = wl.T_own if (wl.n_shared and wl.T_own) else 0
    mbs, us, _, upos = stage_table(list(counts), n_own, mb, BM, nN_r, nN_s, XB_N)
    n = len(mbs)
    assert got["n_mb"] == n
    first = []
    for m, (g, rows) in enumerate(mbs):
        i = sum(1 for q in range(m) if mbs[q][0] == g)
        first.append((int(offsets[g]) if g < E_l else 0) + i * mb)
    assert np.array_equal(got["grp"], [g for g, _ in mbs])
    assert np.array_equal(got["nr"], [r for _, r in mbs])
    assert np.array_equal(got["r0"], first)
    assert np.array_equal(got["us"], us)
    assert np.array_equal(got["rpre"], np.cumsum([0] + [r for _, r in mbs]))
    ent = lambda m, l: [m, l, first[m], (mbs[m][0] << 16) | mbs[m][1]]
    mx_gather = ring and wl.dtype in ("mxfp8", "mxfp4")
    nu = [-(-r // BM) * (nN_r if g < E_l else nN_s) for g, r in mbs]
    nd = [-(-r // BM) * nD for g, r in mbs]
    ng = [-(-r // G_ROWS) if mx_gather else 0 for g, r in mbs]
    assert np.array_equal(got["ds"], np.cumsum([0] + nd))
    assert np.array_equal(got["gs"], np.cumsum([0] + ng))
    if not ring:
        assert got["n_u"] == us[-1] and got["n_d"] == sum(nd)
        assert got["n_r"] == (got["n_u"] + got["n_d"] if loop else 0)
        for p, (m, l) in upos.items():
            assert list(got["utab"][p]) == ent(m, l), ("up", p)
        _, _, _, dpos = stage_table(list(counts), n_own, mb, BM, nD, nD, XB_ND)
        n_routed = sum(1 for g, _ in mbs if g < E_l)
        d_sh0 = sum(nd[:n_routed])
        d_sh = sum(nd) - d_sh0
        for p, (m, l) in dpos.items():
            if nN_s > nN_r:                            # shared experts' down tiles first
                p = p - d_sh0 if m >= n_routed else p + d_sh
            assert list(got["dtab"][p]) == ent(m, l), ("down", p)
        if loop:
            check_loop_table(got, ent, nu, nd, [g for g, _ in mbs], E_l, wl)
    else:
        n_slots = wl.ring_rows // mb
        lay = ring_layout(nu, nd, ng, n_slots)
        assert got["n_r"] == lay["total"]
        assert got["affine"] == int(lay["affine"])
        assert np.array_equal(got["xb"], lay["xb"])
        assert np.array_equal(got["xr"], lay["xr"])
        assert np.array_equal(got["slot"], [lay["slot"][m] for m in range(n)])
        assert np.array_equal(got["prev"], [lay["prev"][m] for m in range(n)])
        for (k, m, l), p in lay["pos"].items():
            e = ent(m, l)
            e[1] = (KINDS[k] << KIND_SHIFT) | l
            assert list(got["rtab"][p]) == e, (k, m, l, p)
    return n


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("ring", [False, True, "loop"])
def test_worklist_matches_the_scheduling_models(name, ring):
    import routing_grouped_expert_gemm_amd as mok
    wl = CASES[name]
    print(f"worklist {name} ring={ring}", flush=True)
    inp = make_inputs(wl, DEV)
    cpu = {k: (v.cpu() if v is not None else None) for k, v in inp.items()}
    idx, w = _oracle_topk(wl, cpu)
    plan = oracle.dispatch_plan(idx, wl.e0, wl.E_l, wl.tokens_per_rank)
    topk = (torch.from_numpy(idx).to(DEV), torch.from_numpy(w).to(DEV))
    flags = {False: mok.MOK_FLAG_NO_RING, True: 0, "loop": mok.MOK_FLAG_STAGE_LOOP}[ring]
    layer = gpu_layer(wl, inp, topk=topk, flags=flags)
    layer.forward()
    torch.cuda.synchronize()
    assert np.array_equal(to_np(layer.inter["counts"]), plan["counts"])
    n = _check(wl, layer, plan["counts"], plan["offsets"], ring)
    if name == "many_mb_bf16":
        assert n > 1024
    else:
        assert n <= 1024
    assert layer.device_error() == 0
