"""The plan's kernels (k_plan_count; k_plan_scatter with its work-list workgroup) run on the CPU:
their own source text, compiled by g++ against a small emulation of a HIP workgroup
(tests/simt: one thread per work-item, barriers for __syncthreads and for the wave-level
shuffles and ballots) under AddressSanitizer and UBSan. The plan must equal the oracle's and
the work list the scheduling models (test_gpu_worklist.check_worklist), with every buffer
sized exactly, so that any out-of-bounds access stops the run. Cases are small but reach the
builder's corners: a chunk of exactly 1024 minibatches (LDS tables), more than 1024 (tables in
global memory, two chunks), shared experts first in the down table, and the ring order with
and without the XCD split. Host logic of the device code, no GPU needed."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import synth
from test_gpu_worklist import check_worklist, parse_worklist

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "routing_grouped_expert_gemm_amd", "csrc")


def _extract(src, head, whole_function=True):
    a = src.index(head)
    return src[a:src.index("\n}\n", a) + 3] if whole_function else src[a:src.index("\n", a) + 1]


def _kernels_source() -> str:
    dc = open(os.path.join(CSRC, "device_common.h")).read()
    helpers = (_extract(dc, "MOK_DEV int32_t block_excl_scan_1024") +
               _extract(dc, "MOK_DEV uint64_t ballot", False) +
               _extract(dc, "MOK_DEV uint64_t lanemask_lt") +
               _extract(dc, "MOK_DEV int uniform(", False))
    wl = open(os.path.join(CSRC, "worklist.h")).read().replace('#include "device_common.h"', "")
    pl = open(os.path.join(CSRC, "plan.hip")).read()
    kern = pl[pl.index("constexpr int PLAN_THREADS"):pl.index("// Chunks of whole multiples")]
    kern = kern.replace("extern __shared__ int32_t hist[];", "int32_t* hist = (int32_t*)g_block->lds;")
    kern = kern.replace("extern __shared__ int32_t sm[];", "int32_t* sm = (int32_t*)g_block->lds;")
    body = wl.rstrip()
    assert body.endswith("}  // namespace mok")
    return ('#include "device_common.h"\n' + helpers + body[:-len("}  // namespace mok")] + kern +
            "\n}  // namespace mok\n")


@pytest.fixture(scope="module")
def sim(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("simt")
    for f in ("simt.h", "device_common.h", "sim_plan.cpp"):
        shutil.copy(os.path.join(HERE, "simt", f), d / f)
    (d / "kernels_gen.h").write_text(_kernels_source())
    exe = d / "sim_plan"
    subprocess.check_call(["g++", "-std=c++20", "-O1", "-g", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                           "-I", str(d), str(d / "sim_plan.cpp"), "-o", str(exe), "-pthread"])
    return str(exe)


def _cdiv(a, b):
    return -(-a // b)


def _params(wl, ring):
    """The plan and work-list arguments the forward passes (the layout of api.hip); ring is
    False (stage order), True (ring order) or "loop" (stage order run by the persistent loop)."""
    loop = ring == "loop"
    ring = ring is True
    mb = wl.minibatch_rows
    mx = wl.dtype in ("mxfp8", "mxfp4")
    n_cap = wl.T_pool * min(wl.k, wl.E_l)
    I_sh = wl.n_shared * wl.I_shared
    max_mb = max(1, _cdiv(n_cap, mb) + wl.E_l + (_cdiv(wl.T_own, mb) if I_sh > 0 else 0))
    n_slots = wl.ring_rows // mb if ring else max_mb
    mt, nU, nD = _cdiv(mb, 256), max(_cdiv(wl.I, 128), _cdiv(I_sh, 128)), _cdiv(wl.d, 256)
    cap_u, cap_d = max_mb * mt * nU, max_mb * mt * nD
    cap_g = max_mb * _cdiv(mb, 64) if (ring and mx) else 0
    cap_r = cap_u + cap_d + cap_g if ring else (cap_u + cap_d if loop else 0)
    T_own = wl.T_own if wl.n_shared > 0 else 0
    return [wl.T_pool, wl.k, wl.e0, wl.E_l, wl.tokens_per_rank, T_own, mb, 256, _cdiv(wl.I, 128),
            _cdiv(I_sh, 128), nD, int(ring and mx), int(ring), 1, n_slots, max_mb, cap_u, cap_d,
            cap_r, max(1, n_cap), int(loop), wl.d // 64, wl.I // 64, I_sh // 64]


def _run(sim, tmp_path, wl, idx, ring):
    with open(tmp_path / "in.bin", "wb") as f:
        f.write(np.array(_params(wl, ring), np.int64).tobytes())
        f.write(np.ascontiguousarray(idx, np.int32).tobytes())
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    r = subprocess.run([sim, str(tmp_path)], capture_output=True, text=True, env=env)
    assert r.returncode == 0, r.stderr[-4000:]
    raw = open(tmp_path / "out.bin", "rb").read()
    nb, wl_ints, route_cap, nrc = (int(v) for v in np.frombuffer(raw[:32], np.int64))
    a = np.frombuffer(raw[32:], np.int32).astype(np.int64)
    E_l = wl.E_l
    out = {}
    for key, n in (("counts", E_l), ("offsets", E_l + 1), ("route_ids", route_cap),
                   ("rank_counts", nrc), ("wl", wl_ints)):
        out[key], a = a[:n], a[n:]
    plan = oracle.dispatch_plan(idx, wl.e0, wl.E_l, wl.tokens_per_rank)
    assert np.array_equal(out["counts"], plan["counts"])
    assert np.array_equal(out["offsets"], plan["offsets"])
    assert np.array_equal(out["rank_counts"].reshape(plan["rank_counts"].shape),
                          plan["rank_counts"])
    assert np.array_equal(out["route_ids"][:plan["n"]], plan["route_ids"])
    return check_worklist(wl, parse_worklist(out["wl"]), plan["counts"], plan["offsets"], ring)


def _balanced(T, k, E, seed):
    """Top-k ids with no repeat in a token: each token's k experts are a random draw."""
    rng = np.random.default_rng(seed)
    return np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)


BASE = synth.WORKLOADS[synth.EP1]
CASES = {
    # 64 experts x 16 minibatches of 8 rows: exactly one full chunk of 1024 minibatches
    "exact_1024": (synth.scaled(BASE, name="sim_1024", T_pool=1024, d=256, E=64, k=8, I=128,
                                E_l=64, tokens_per_rank=1024, T_own=0, n_shared=0,
                                I_shared=128, minibatch_rows=8, ring_rows=512),
                   lambda: ((np.arange(1024)[:, None] * 8 + np.arange(8)[None, :]) % 64)
                   .astype(np.int32)),
    # ~1500 minibatches: the tables in global memory, a full chunk and a partial one; shared
    # down tiles longer than the routed ones (listed first)
    "global_tables": (synth.scaled(BASE, name="sim_global", T_pool=1024, d=256, E=40, k=6,
                                   I=128, E_l=40, tokens_per_rank=1024, T_own=1024, n_shared=2,
                                   I_shared=256, minibatch_rows=5, ring_rows=400),
                      lambda: _balanced(1024, 6, 40, 1)),
    # a share of the pool: 4 local experts of 64, source ranks of 128 tokens, small ring
    # (fewer than 8 slots: no XCD split)
    "share": (synth.scaled(synth.WORKLOADS[synth.EP64], name="sim_share", T_pool=2048, d=256,
                           E=64, k=8, I=256, e0=12, E_l=4, tokens_per_rank=128, own_begin=256,
                           T_own=128, I_shared=256, minibatch_rows=64, ring_rows=256),
              lambda: _balanced(2048, 8, 64, 2)),
    "share_mxfp8": (synth.scaled(synth.WORKLOADS[synth.EP64_MX], name="sim_share_mx",
                                 T_pool=2048, d=256, E=64, k=8, I=256, e0=4, E_l=4,
                                 tokens_per_rank=256, own_begin=256, T_own=256, I_shared=128,
                                 minibatch_rows=32, ring_rows=512),
                    lambda: _balanced(2048, 8, 64, 3)),
}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("ring", [False, True, "loop"])
def test_plan_and_worklist_kernels_on_cpu(sim, tmp_path, name, ring):
    wl, make_idx = CASES[name]
    n = _run(sim, tmp_path, wl, make_idx(), ring)
    if name == "exact_1024":
        assert n == 1024
    if name == "global_tables":
        assert n > 1024
