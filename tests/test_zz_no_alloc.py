"""mok_dispatch_plan_noalloc (scratch in a fixed device array) against mok_dispatch_plan (scratch
from the caller's workspace), through the C ABI: bit-identical counts, offsets, per-rank counts
and route ids on two calls in a row, the second smaller than the first (the array keeps the
first call's contents), and requests beyond the fixed scratch rejected before any launch."""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _plan(mok, idx_np, E, e0, E_l, tpr, noalloc):
    T, k = idx_np.shape
    R = T // tpr
    i32 = dict(dtype=torch.int32, device=DEV)
    out = dict(counts=torch.full((E_l,), -7, **i32), offsets=torch.full((E_l + 1,), -7, **i32),
               rank_counts=torch.full((E_l, R), -7, **i32),
               route_ids=torch.full((max(1, T * min(k, E_l)),), -7, **i32))
    idx = torch.from_numpy(idx_np).to(DEV)
    if noalloc:
        mok.mok_dispatch_plan_noalloc(idx, E, e0, E_l, tpr, out["counts"], out["offsets"],
                                      out["rank_counts"], out["route_ids"])
    else:
        ws = torch.empty(mok.mok_dispatch_plan_workspace_bytes(T, k, E_l), dtype=torch.uint8,
                         device=DEV)
        mok.mok_dispatch_plan(idx, E, e0, E_l, tpr, out["counts"], out["offsets"],
                              out["rank_counts"], out["route_ids"], ws)
    torch.cuda.synchronize()
    return {k_: v.cpu().numpy() for k_, v in out.items()}


@pytest.mark.parametrize("first,second", [
    ((262144, 8, 256, 0, 4, 4096), (8192, 6, 64, 0, 64, 8192)),
    ((8192, 6, 64, 0, 64, 8192), (300, 2, 8, 3, 2, 100)),
])
def test_noalloc_plan_matches_workspace_plan(first, second):
    import routing_grouped_expert_gemm_amd as mok
    for i, (T, k, E, e0, E_l, tpr) in enumerate((first, second)):
        rng = np.random.default_rng(100 + i + T)
        idx = np.argsort(rng.random((T, E), dtype=np.float32), axis=1)[:, :k].astype(np.int32)
        print(f"noalloc plan call {i}: T={T} k={k} E={E} e0={e0} E_l={E_l}", flush=True)
        got = _plan(mok, idx, E, e0, E_l, tpr, True)
        ref = _plan(mok, idx, E, e0, E_l, tpr, False)
        for key in ref:
            assert np.array_equal(got[key], ref[key]), (i, key)
        assert int(got["offsets"][-1]) > 0
