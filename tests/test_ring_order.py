"""The ring work loop's item order, as the work-list builder (k_build_worklist) lays it out,
checked on the CPU over random minibatch mixes and ring sizes:

  * the positions of all items form a permutation of 0..n_items-1;
  * with the XCD split (>= 8 slots) each XCD's items are one contiguous segment, its minibatches
    one contiguous range, its slots its own;
  * every dependency of an item (down <- the minibatch's up tiles; up <- its gather items and
    the down tiles of the slot's previous user; gather <- the previous user's up tiles) comes
    earlier in the same segment, so a loop that takes items in order cannot deadlock;
  * a minibatch's slot predecessor is the latest earlier minibatch on that slot.

This is a model of the scheduling rules (host logic), not of any arithmetic of the layer."""
import itertools
import random

N_XCD = 8


def layout(nu, nd, ng, n_slots, w_up=1, w_dr=1, w_g=1):
    n = len(nu)
    cs = lambda a: [0] + list(itertools.accumulate(a))
    us, ds, gs = cs(nu), cs(nd), cs(ng)
    affine = n_slots >= N_XCD
    wpre = cs([nu[m] * w_up + nd[m] * w_dr + ng[m] * w_g for m in range(n)])
    W = wpre[n]

    def xcd_of(m):
        pre, w = wpre[m], wpre[m + 1] - wpre[m]
        return min(N_XCD - 1, (N_XCD * (2 * pre + w)) // max(1, 2 * W))

    xb = [0] + [n] * N_XCD
    if affine:
        xb = [n] * (N_XCD + 1)
        for m in range(n):
            xm, xp = xcd_of(m), (xcd_of(m - 1) if m > 0 else -1)
            for x in range(xp + 1, xm + 1):
                xb[x] = m
    xr = [gs[b] + us[b] + ds[b] for b in xb]
    pos, slot, prev, owner = {}, {}, {}, {}
    for m in range(n):
        lo, hi, S, s0 = 0, n, n_slots, 0
        if affine:
            x = xcd_of(m)
            lo, hi, S, s0 = xb[x], xb[x + 1], n_slots // N_XCD, x * (n_slots // N_XCD)
        owner[m] = lo
        L = S // 2 if S >= 2 else 0
        slot[m] = s0 + (m - lo) % S
        prev[m] = m - S if m - S >= lo else -1
        ml, after = max(lo, m - L), min(m + L + 1, hi)
        r0 = gs[lo] + us[lo] + ds[lo]
        pg = r0 + (gs[m] - gs[lo]) + (us[m] - us[lo]) + (ds[ml] - ds[lo])
        pu = r0 + (gs[m + 1] - gs[lo]) + (us[m] - us[lo]) + (ds[ml] - ds[lo])
        pd = r0 + (gs[after] - gs[lo]) + (us[after] - us[lo]) + (ds[m] - ds[lo])
        for l in range(ng[m]):
            pos[("G", m, l)] = pg + l
        for l in range(nu[m]):
            pos[("U", m, l)] = pu + l
        for l in range(nd[m]):
            pos[("D", m, l)] = pd + l
    return dict(pos=pos, slot=slot, prev=prev, owner=owner, xb=xb, xr=xr, affine=affine,
                total=us[n] + ds[n] + gs[n])


def check(nu, nd, ng, n_slots):
    lay = layout(nu, nd, ng, n_slots)
    pos, slot, prev, owner, xb, xr = (lay[k] for k in ("pos", "slot", "prev", "owner", "xb", "xr"))
    n = len(nu)
    assert sorted(pos.values()) == list(range(lay["total"]))
    seg = lambda m: next(x for x in range(N_XCD) if xb[x] <= m < xb[x + 1])
    for (k, m, l), p in pos.items():
        if lay["affine"]:
            assert xr[seg(m)] <= p < xr[seg(m) + 1]
        pm = prev[m]
        deps = []
        if k == "D":
            deps = [("U", m, i) for i in range(nu[m])]
        elif k == "U":
            deps = [("G", m, i) for i in range(ng[m])]
            if pm >= 0:
                deps += [("D", pm, i) for i in range(nd[pm])]
        elif pm >= 0:
            deps = [("U", pm, i) for i in range(nu[pm])]
        for dep in deps:
            assert pos[dep] < p and owner[dep[1]] == owner[m]
    for m in range(n):
        same = [q for q in range(m) if slot[q] == slot[m]]
        assert prev[m] == (same[-1] if same else -1)
        if lay["affine"]:
            assert all(owner[q] == owner[m] for q in same)


def test_ring_order_random_mixes():
    rng = random.Random(3)
    affine = 0
    for _ in range(1500):
        n = rng.randint(0, 48)
        S = rng.choice([1, 2, 3, 4, 7, 8, 9, 16, 24, 32, 64, 256])
        nu = [rng.randint(1, 22) for _ in range(n)]
        nd = [rng.randint(1, 8) for _ in range(n)]
        ng = [rng.randint(0, 8) if rng.random() < 0.5 else 0 for _ in range(n)]
        check(nu, nd, ng, S)
        affine += S >= N_XCD
    assert affine > 500


def test_ring_order_one_slot_is_serial():
    lay = layout([2, 2, 2], [1, 1, 1], [0, 0, 0], 1)
    order = sorted(lay["pos"], key=lay["pos"].get)
    assert [(k, m) for k, m, _ in order] == [("U", 0), ("U", 0), ("D", 0), ("U", 1), ("U", 1),
                                            ("D", 1), ("U", 2), ("U", 2), ("D", 2)]
