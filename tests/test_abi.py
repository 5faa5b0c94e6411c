"""The C-ABI library loads, exports every symbol include/mok.h declares, and validates
arguments before touching the GPU (no compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mok.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mok_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def mok():
    import routing_grouped_expert_gemm_amd as m
    return m


def test_header_declares_the_boundary():
    names = _declared()
    for n in ["mok_route", "mok_topk", "mok_dispatch_plan", "mok_dispatch_plan_workspace_bytes",
              "mok_moe_forward", "mok_moe_workspace_bytes", "mok_quantize_mxfp8",
              "mok_get_device_error", "mok_status_string", "mok_version"]:
        assert n in names


def test_library_exports_every_declared_symbol(mok):
    lib = ctypes.CDLL(mok.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), n
    assert sorted(mok.EXPORTS) == _declared()


def test_status_strings_and_version(mok):
    assert mok.status_string(0) == "MOK_OK"
    assert "invalid" in mok.status_string(1)
    assert "workspace" in mok.status_string(3)
    assert mok.status_string(99) == "unknown mok status"
    assert "gfx950" in mok.version()


def test_struct_layout_matches_header(mok, tmp_path):
    """Every field of mok_moe_args sits at the offset a C compiler gives it."""
    import subprocess
    fields = [f[0] for f in mok.MoeArgs._fields_]
    src = tmp_path / "layout.c"
    body = "".join(f'printf("%s %zu\\n", "{f}", offsetof(mok_moe_args, {f}));' for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "mok.h"\n'
                   'int main(void){' + body + 'printf("sizeof %zu\\n", sizeof(mok_moe_args));'
                   'return 0;}\n')
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src),
                           "-o", str(exe)])
    out = dict(line.split() for line in subprocess.check_output([str(exe)], text=True).splitlines())
    for f in fields:
        assert int(out[f]) == getattr(mok.MoeArgs, f).offset, f
    assert int(out["sizeof"]) == ctypes.sizeof(mok.MoeArgs)


def _args(mok, **kw):
    a = mok.MoeArgs()
    base = dict(dtype=1, d=256, E=16, k=4, I=192, e0=0, E_l=16, tokens_per_rank=512, T_pool=512,
                own_begin=0, T_own=512, n_shared=1, I_shared=128, minibatch_rows=128,
                ring_rows=1024, x=16, w_router=16, w_gate=16, w_up=16, w_down=16, ws_gate=16,
                ws_up=16, ws_down=16, y_slots=16, y_shared=16, y=16)
    base.update(kw)
    for k, v in base.items():
        setattr(a, k, v)
    return a


def test_workspace_query_and_validation(mok):
    a = _args(mok)
    n = mok.mok_moe_workspace_bytes(a)
    assert n > 0
    bad = [dict(d=200), dict(I=100), dict(k=0), dict(k=17), dict(E_l=0), dict(e0=10),
           dict(minibatch_rows=100), dict(ring_rows=100), dict(T_pool=500),
           dict(y=0), dict(w_router=0), dict(topk_idx_in=16), dict(dtype=7),
           dict(E_l=8, y=16), dict(n_shared=0), dict(I_shared=100), dict(E=2000)]
    for kw in bad:
        with pytest.raises(mok.MokError) as ei:
            mok.mok_moe_workspace_bytes(_args(mok, **kw))
        assert ei.value.status == mok.MOK_EINVAL, kw
    # valid variants
    mok.mok_moe_workspace_bytes(_args(mok, n_shared=0, y_shared=0, ws_gate=0, ws_up=0, ws_down=0))
    mok.mok_moe_workspace_bytes(_args(mok, E_l=4, y=0, w_router=0, topk_idx_in=16,
                                      topk_w_in=16, T_own=128, own_begin=128, tokens_per_rank=128))
    # MXFP8 needs K multiples of 128
    with pytest.raises(mok.MokError):
        mok.mok_moe_workspace_bytes(_args(mok, dtype=2))
    mok.mok_moe_workspace_bytes(_args(mok, dtype=2, I=256))


def test_entry_points_reject_before_launch(mok):
    L = ctypes.CDLL(mok.LIB_PATH)
    P = ctypes.c_void_p
    L.mok_route.argtypes = [P, P, ctypes.c_int64] + [ctypes.c_int32] * 4 + [P, P, P, P]
    assert L.mok_route(16, 16, 10, 64, 8, 9, 1, 16, 16, 16, None) == 1      # k > E
    assert L.mok_route(16, 16, 10, 64, 8, 2, 5, 16, 16, 16, None) == 1      # dtype
    assert L.mok_route(None, 16, 0, 64, 8, 2, 1, None, None, None, None) == 0  # T == 0: no-op
    L.mok_quantize_mxfp8.argtypes = [P, ctypes.c_int64, ctypes.c_int32, P, P, P]
    assert L.mok_quantize_mxfp8(16, 4, 40, 16, 16, None) == 1                # K % 32
    L.mok_dispatch_plan.argtypes = [P, ctypes.c_int64] + [ctypes.c_int32] * 5 + [P] * 5 + [
        ctypes.c_size_t, P]
    assert L.mok_dispatch_plan(16, 10, 2, 8, 0, 4, 3, 16, 16, 16, 16, 16, 1 << 20, None) == 1
    assert L.mok_dispatch_plan(16, 12, 2, 8, 0, 4, 3, 16, 16, 16, 16, 16, 0, None) == 3
    assert mok.mok_dispatch_plan_workspace_bytes(12, 2, 4) > 0


def test_plan_scratch_fits_the_fixed_no_alloc_array(mok):
    """The plan's scratch (its chunk histograms) is bounded for every valid argument set, so
    mok_dispatch_plan_noalloc's fixed 256 KiB array always holds it."""
    limit = 1 << 18
    for E_l in (1, 4, 8, 64, 100, 256, 257, 512, 1000, 1024):
        for T, k in ((1, 1), (64, 2), (8192, 6), (262144, 8), (1 << 20, 8), ((1 << 31) // 64 - 1, 64)):
            assert mok.mok_dispatch_plan_workspace_bytes(T, k, E_l) <= limit, (T, k, E_l)
    assert mok.mok_dispatch_plan_workspace_bytes((1 << 31) // 64 - 1, 64, 1024) > limit // 8


def test_product_path_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "routing_grouped_expert_gemm_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in txt and "from oracle" not in txt, f
                assert "mok_oracle" not in txt, f


def test_workspace_regions(mok):
    """Regions of the forward's intermediates: inside the workspace, disjoint, sized as the
    header states, and present only where the configuration has them."""
    a = _args(mok, dtype=2, I=256, minibatch_rows=128, ring_rows=1024)
    total = mok.mok_moe_workspace_bytes(a)
    spans = []
    for reg in range(17):
        off, n, rows = mok.mok_moe_workspace_region(a, reg)
        assert off % 256 == 0 and n > 0 and off + n <= total, reg
        spans.append((off, off + n))
    spans.sort()
    assert all(b[0] >= a_[1] for a_, b in zip(spans, spans[1:]))
    d, I, E_l, Is = 256, 256, 16, 128
    assert mok.mok_moe_workspace_region(a, mok.MOK_REGION_WG_CODES)[1:] == (E_l * I * d, I)
    assert mok.mok_moe_workspace_region(a, mok.MOK_REGION_WD_SCALES)[1:] == (E_l * d * I // 32, d)
    assert mok.mok_moe_workspace_region(a, mok.MOK_REGION_SU_CODES)[1:] == (Is * d, Is)
    assert mok.mok_moe_workspace_region(a, mok.MOK_REGION_SD_SCALES)[1:] == (d * Is // 32, d)
    assert mok.mok_moe_workspace_region(a, mok.MOK_REGION_A_CODES)[1:] == (1024 * d, 1024)
    assert mok.mok_moe_workspace_region(a, mok.MOK_REGION_H_SCALES)[1:] == (1024 * I // 32, 1024)
    # a bf16 forward has H (bf16) and the work list, no MX regions
    b = _args(mok)
    assert mok.mok_moe_workspace_region(b, mok.MOK_REGION_H)[1] == 1024 * 192 * 2
    for reg in (mok.MOK_REGION_A_CODES, mok.MOK_REGION_WG_SCALES, mok.MOK_REGION_H_SCALES, 99, -1):
        with pytest.raises(mok.MokError):
            mok.mok_moe_workspace_region(b, reg)
    # no shared experts: no shared regions
    c = _args(mok, dtype=2, I=256, n_shared=0, y_shared=0, ws_gate=0, ws_up=0, ws_down=0)
    with pytest.raises(mok.MokError):
        mok.mok_moe_workspace_region(c, mok.MOK_REGION_SG_CODES)
    mok.mok_moe_workspace_region(c, mok.MOK_REGION_WG_CODES)
