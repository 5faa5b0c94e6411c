"""Find the Zipf bias strength of the skewed 384-expert workload with the oracle's own top-k.

The workload's router logits are N(0,1) plus beta * (-1.1 * ln rank_e) per expert; beta is
set so that local expert 0 (Zipf rank 1) receives 4.0x the mean number of routes. This script
bisects beta on the oracle's top-k counts and prints the value stored in synth.

    python -m oracle.calibrate_zipf
"""
import sys
import os

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle  # noqa: E402
import synth   # noqa: E402


def expert0_ratio(beta: float, z: np.ndarray, wl) -> tuple:
    w = synth.scaled(wl, zipf_beta=beta)
    bias = synth.zipf_bias(w).numpy()
    logits = (z + bias[None, :]).astype(np.float32)
    idx, _ = oracle.topk(logits, wl.k)
    counts = np.bincount(idx.reshape(-1), minlength=wl.E)
    mean = wl.T_pool * wl.k / wl.E
    return counts[0] / mean, counts[:4]


def main():
    wl = synth.WORKLOADS[synth.EP96]
    z = synth.normal_rows(synth.SEED, synth.S_LOGITS, wl.E, range(wl.T_pool), 1.0).numpy()
    lo, hi = 0.0, 2.0
    for _ in range(16):
        mid = 0.5 * (lo + hi)
        r, _ = expert0_ratio(mid, z, wl)
        if r < 4.0:
            lo = mid
        else:
            hi = mid
    beta = float(np.float32(0.5 * (lo + hi)))
    r, c = expert0_ratio(beta, z, wl)
    print(f"beta={beta!r} ratio={r:.4f} local counts={c.tolist()}")


if __name__ == "__main__":
    main()
