"""The stage-ordered GEMM tables' tile order, as the work-list builder (k_build_worklist) lays
it out, checked on the CPU over random expert mixes:

  * every (minibatch, local tile) entry gets one position, and the positions of a group (a
    routed expert, or the shared experts) fill the group's own range of the table;
  * within a group, tiles come in blocks of XB N tiles; in each block the group's M tiles in
    order, each with the block's N tiles -- so 32 consecutive entries (one XCD's round) of a
    group with at least 32 / XB M tiles touch 32 / XB M tiles and XB N tiles.

This is a model of the scheduling rules (host logic), not of any arithmetic of the layer."""
import itertools
import random


def cs(a):
    return [0] + list(itertools.accumulate(a))


def stage_table(counts, n_own, mb, bm, nN_r, nN_s, XB):
    """Entries {position: (minibatch, local tile)}; local tile l = mt + n_mt * nt."""
    mbs = []                                          # (group, rows) per minibatch, in order
    for g, c in enumerate(counts):
        mbs += [(g, min(mb, c - i * mb)) for i in range((c + mb - 1) // mb)]
    E_l = len(counts)
    mbs += [(E_l, min(mb, n_own - i * mb)) for i in range((n_own + mb - 1) // mb)]
    mpm = (mb + bm - 1) // bm
    nt_of = lambda g: nN_r if g < E_l else nN_s
    ntiles = [((r + bm - 1) // bm) * nt_of(g) for g, r in mbs]
    us = cs(ntiles)
    first = {}
    for m, (g, _) in enumerate(mbs):
        first.setdefault(g, m)
    pos = {}
    for m, (g, rows) in enumerate(mbs):
        f = first[g]
        f_end = max(q for q, (gg, _) in enumerate(mbs) if gg == g) + 1
        mt_m = (rows + bm - 1) // bm
        mo = (m - f) * mpm
        MT = (f_end - 1 - f) * mpm + (mbs[f_end - 1][1] + bm - 1) // bm
        nN = nt_of(g)
        for l in range(ntiles[m]):
            mt, nt = l % mt_m, l // mt_m
            nb, w = nt // XB, min(XB, nN - (nt // XB) * XB)
            pos[us[f] + nb * MT * XB + (mo + mt) * w + (nt - nb * XB)] = (m, l)
    return mbs, us, first, pos


def test_stage_table_is_a_blocked_permutation():
    rng = random.Random(5)
    for _ in range(300):
        E_l = rng.randint(1, 9)
        mb = rng.choice([128, 256, 512, 1024])
        bm = 256
        counts = [rng.randint(1, 5000) for _ in range(E_l)]
        n_own = rng.choice([0, rng.randint(1, 3000)])
        nN_r, nN_s = rng.randint(1, 30), rng.randint(1, 30)
        XB = rng.choice([1, 2, 4, 8, 16])
        mbs, us, first, pos = stage_table(counts, n_own, mb, bm, nN_r, nN_s, XB)
        total = us[-1]
        assert sorted(pos) == list(range(total))
        assert len(set(pos.values())) == total
        # each group's tiles fill [us[first], us[first] + its tile count)
        for g, f in first.items():
            ms = [m for m, (gg, _) in enumerate(mbs) if gg == g]
            lo, hi = us[f], us[ms[-1] + 1]
            assert all(lo <= p < hi for p, (m, _) in pos.items() if mbs[m][0] == g)
        # a round of 32 entries inside one large group spans 32 / XB M tiles and XB N tiles
        for g, f in first.items():
            ms = [m for m, (gg, _) in enumerate(mbs) if gg == g]
            nN = nN_r if g < E_l else nN_s
            n_mt = sum((mbs[m][1] + bm - 1) // bm for m in ms)
            if XB > nN or n_mt * XB < 32 or 32 % XB:
                continue
            rnd = [pos[us[f] + i] for i in range(32)]
            mts, nts = set(), set()
            for m, l in rnd:
                mt_m = (mbs[m][1] + bm - 1) // bm
                mts.add((m, l % mt_m))
                nts.add(l // mt_m)
            assert len(nts) == XB and len(mts) == 32 // XB
