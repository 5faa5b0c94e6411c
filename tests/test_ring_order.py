"""The ring work loop's item order, as the work-list builder (k_build_worklist) lays it out,
checked on the CPU over random minibatch mixes and ring sizes:

  * the positions of all items form a permutation of 0..n_items-1;
  * with the XCD split (>= 8 slots) XCD x owns minibatches x, x + 8, ...: its items are one
    contiguous segment and its slots its own;
  * every dependency of an item (down <- the minibatch's up tiles; up <- its gather items and
    the down tiles of the slot's previous user; gather <- the previous user's up tiles) comes
    earlier in the same segment, so a loop that takes items in order cannot deadlock;
  * a minibatch's slot predecessor is the latest earlier minibatch on that slot.

This is a model of the scheduling rules (host logic), not of any arithmetic of the layer."""
import itertools
import random

N_XCD = 8


def layout(nu, nd, ng, n_slots):
    n = len(nu)
    cs = lambda a: [0] + list(itertools.accumulate(a))
    affine = n_slots >= N_XCD
    # XCD x owns minibatches x, x + 8, ... (all of them without the split), XCD-major order
    n_of = lambda x: (n - x + N_XCD - 1) // N_XCD if affine else (n if x == 0 else 0)
    base = cs([n_of(x) for x in range(N_XCD)])
    order = [x + N_XCD * j for x in range(N_XCD) for j in range(n_of(x))] if affine else list(range(n))
    pg, pu, pd = (cs([a[m] for m in order]) for a in (ng, nu, nd))
    xb = base
    xr = [pg[b] + pu[b] + pd[b] for b in xb]
    pos, slot, prev, owner = {}, {}, {}, {}
    for m in range(n):
        S, s0, j, pb, nx, step = n_slots, 0, m, 0, n, 1
        if affine:
            x = m % N_XCD
            S, s0, j, pb, nx, step = n_slots // N_XCD, x * (n_slots // N_XCD), m // N_XCD, base[x], n_of(x), N_XCD
        owner[m] = m % N_XCD if affine else 0
        L = S // 2 if S >= 2 else 0
        G = 1 if S >= 2 else 0            # gather items run one block ahead of their up tiles
        slot[m] = s0 + j % S
        prev[m] = m - step * S if j >= S else -1
        # block b of the XCD's order: gather items of b + G, up tiles of b, down tiles of b - L
        at = lambda i: pb + min(max(i, 0), nx)
        for l in range(ng[m]):
            pos[("G", m, l)] = pg[at(j)] + pu[at(j - G)] + pd[at(j - G - L)] + l
        for l in range(nu[m]):
            pos[("U", m, l)] = pg[at(j + G + 1)] + pu[at(j)] + pd[at(j - L)] + l
        for l in range(nd[m]):
            pos[("D", m, l)] = pg[at(j + L + G + 1)] + pu[at(j + L + 1)] + pd[at(j)] + l
    return dict(pos=pos, slot=slot, prev=prev, owner=owner, xb=xb, xr=xr, affine=affine,
                total=pg[n] + pu[n] + pd[n])


def check(nu, nd, ng, n_slots):
    lay = layout(nu, nd, ng, n_slots)
    pos, slot, prev, owner, xb, xr = (lay[k] for k in ("pos", "slot", "prev", "owner", "xb", "xr"))
    n = len(nu)
    assert sorted(pos.values()) == list(range(lay["total"]))
    for (k, m, l), p in pos.items():
        if lay["affine"]:
            assert xr[m % N_XCD] <= p < xr[m % N_XCD + 1]
            assert slot[m] // (n_slots // N_XCD) == m % N_XCD
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
