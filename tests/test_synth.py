"""The seeded input generator (CPU): standard normal values, reproducible, row-addressable;
the Zipf bias and permutation of the skewed workload. These are input recipes, not layer
arithmetic: the checks are on the distribution the configs state (x ~ N(0,1), weights
~ N(0, 1/d_in))."""
import math

import numpy as np
import torch

import synth


def test_normals_are_standard_normal():
    from scipy import stats
    v = synth.normal_flat(0, 1, 0, 1 << 21, 1.0).double().numpy()
    assert abs(v.mean()) < 3e-3 and abs(v.std() - 1.0) < 3e-3
    assert abs(stats.skew(v)) < 1e-2 and abs(stats.kurtosis(v)) < 2e-2   # excess kurtosis 0
    assert stats.kstest(v[:100000], "norm").pvalue > 1e-3
    # tails a bounded sum would not reach (P(|z| > 4) = 6.3e-5)
    assert (np.abs(v) > 4.0).sum() > 50


def test_weight_scale_and_rows_are_addressable():
    wl = synth.scaled(synth.WORKLOADS[synth.EP1], T_pool=64, d=256, E=8, k=2, I=128, E_l=8,
                      tokens_per_rank=64, T_own=64)
    wg, wu, wd = synth.expert_weights(wl)
    assert abs(wg.float().std().item() * math.sqrt(wl.d) - 1.0) < 0.02
    assert abs(wd.float().std().item() * math.sqrt(wl.I) - 1.0) < 0.02
    x = synth.x_rows(wl, range(64))
    assert torch.equal(x, synth.x_rows(wl, range(64)))                       # reproducible
    rows = torch.tensor([3, 17, 63])
    assert torch.equal(synth.x_rows(wl, rows).view(torch.int16), x[rows].view(torch.int16))
    # a share's experts are rows of the global expert streams
    sub = synth.scaled(wl, e0=3, E_l=2)
    assert torch.equal(synth.expert_weights(sub)[0], wg[3:5])


def test_zipf_bias_and_permutation():
    wl = synth.WORKLOADS[synth.EP96]
    b = synth.zipf_bias(wl).double().numpy()
    ranks = np.exp(-b / (wl.zipf_beta * synth.ZIPF_S))
    assert np.allclose(np.sort(ranks), np.arange(1, wl.E + 1), rtol=1e-5)
    assert np.allclose(ranks[:4], [1, 16, 128, 384], rtol=1e-5)
    p = synth.seeded_permutation(0, 10, 100)
    assert sorted(p.tolist()) == list(range(100))
