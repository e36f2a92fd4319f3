"""C-ABI checks that need no GPU: the library loads, exports every function
include/mgemm.h declares, answers the plan table of the metrale_circuit
hardware::exec documentation (exec_of, fp4_fallback, kind_of, pair_name),
and rejects bad arguments on the host before any HIP call."""
import ctypes as C
import os
import re

import pytest
import torch

import block_scaled_precision_tn_amd as mg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mgemm.h")


@pytest.fixture(scope="module")
def lib():
    if not mg.available():
        from block_scaled_precision_tn_amd import build
        build.build()
    return mg.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mgemm_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 11, names
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


GFX950 = "gfx950:sramecc+:xnack-"
F = (mg.FMT_BF16, mg.FMT_NVFP4, mg.FMT_FP8_E4M3_TOKEN, mg.FMT_MXFP8)


def test_plan_table_gfx950(lib):
    want = {
        (mg.FMT_BF16, mg.FMT_BF16): (mg.EXEC_NATIVE, mg.MMA_BF16, 0),
        (mg.FMT_NVFP4, mg.FMT_BF16): (mg.EXEC_NATIVE, mg.MMA_BF16, 0),
        (mg.FMT_NVFP4, mg.FMT_FP8_E4M3_TOKEN): (mg.EXEC_FP8_EXACT, mg.MMA_FP8, 4),
        (mg.FMT_NVFP4, mg.FMT_NVFP4): (mg.EXEC_FP8_EXACT, mg.MMA_FP8, 3),
        (mg.FMT_MXFP8, mg.FMT_MXFP8): (mg.EXEC_NATIVE, mg.MMA_MX_F8F6F4, 0),
    }
    for w in F:
        for a in F:
            got = mg.mgemm_plan_arch(GFX950, w, a)
            if (w, a) in want:
                assert got == want[(w, a)], (w, a, got)
            else:
                # no native or exact path: NoPath, never a wider format
                assert got[0] == mg.EXEC_NOPATH and got[1] == mg.MMA_NONE, (w, a, got)
    assert mg.mgemm_plan_arch("gfx950", mg.FMT_NVFP4, mg.FMT_NVFP4)[0] == mg.EXEC_FP8_EXACT


@pytest.mark.parametrize("arch", ["gfx942:sramecc+:xnack-", "gfx90a", "gfx9500", "sm_90", ""])
def test_plan_other_devices_have_no_path(lib, arch):
    for w in F:
        for a in F:
            assert mg.mgemm_plan_arch(arch, w, a) == (mg.EXEC_NOPATH, mg.MMA_NONE, 5)


def test_plan_rejects_bad_enums(lib):
    p = mg._Plan()
    assert lib.mgemm_plan_arch(GFX950.encode(), 7, 0, C.byref(p)) == -1
    assert lib.mgemm_plan_arch(GFX950.encode(), 0, -1, C.byref(p)) == -1
    assert lib.mgemm_plan_arch(GFX950.encode(), 0, 0, None) == -1
    assert lib.mgemm_plan_arch(None, 0, 0, C.byref(p)) == -1


def test_pair_names(lib):
    assert mg.mgemm_pair_name(mg.FMT_NVFP4, mg.FMT_BF16) == "W4A16"
    assert mg.mgemm_pair_name(mg.FMT_BF16, mg.FMT_BF16) == "W16A16"
    assert mg.mgemm_pair_name(mg.FMT_NVFP4, mg.FMT_NVFP4) == "W4A4"
    assert mg.mgemm_pair_name(mg.FMT_NVFP4, mg.FMT_FP8_E4M3_TOKEN) == "W4A8"
    assert mg.mgemm_pair_name(mg.FMT_MXFP8, mg.FMT_MXFP8) == "W8A8"
    buf = C.create_string_buffer(3)
    assert lib.mgemm_pair_name(1, 0, buf, 3) == -1       # does not fit
    assert lib.mgemm_pair_name(9, 0, C.create_string_buffer(8), 8) == -1


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4, -5):
        assert mg.status_string(s) and mg.status_string(s) != "unknown status"
    assert mg.status_string(-99) == "unknown status"
    assert "gfx950" in mg.version()


def test_workspace_sizes(lib):
    # BF16: 336 tiles of 256x256 on 256 CUs leave a last round of 80 tiles,
    # split 3 ways along K (FP32 partial tiles); 256 tiles fill one round
    assert mg.mgemm_workspace_bytes(mg.OP_BF16, 4096, 5376, 14336) == 80 * 3 * 256 * 256 * 4
    assert mg.mgemm_workspace_bytes(mg.OP_BF16, 4096, 4096, 14336) == 0
    assert mg.mgemm_workspace_bytes(mg.OP_W4A4, 8192, 5376, 14336) == 0
    # W4A16: the split-K partials (14 splits of 1024 up to 16 tokens, 28 of
    # 512 above; 64 rows at a time) through 128 tokens, nothing above
    for M, ks in ((1, 14), (16, 14), (17, 28), (64, 28), (128, 28)):
        assert mg.mgemm_workspace_bytes(mg.OP_W4A16, M, 5376, 14336) == ks * min(M, 128) * 5376 * 4
    assert mg.mgemm_workspace_bytes(mg.OP_W4A16, 129, 5376, 14336) == 0
    for M in (1, 8, 32, 128):
        assert mg.mgemm_workspace_bytes(mg.OP_W4A8, M, 5376, 14336) > 5376 * 4 * M
    moe = mg.mgemm_workspace_bytes(mg.OP_MOE, T=4096, H=4096, I=1536, E=64, topk=8)
    assert moe > 4096 * 4096 * 4 + 4096 * 8 * 1536
    assert mg.mgemm_workspace_bytes(mg.OP_MOE, T=4096, H=4096, I=1500, E=64, topk=8) == 0
    assert mg.mgemm_workspace_bytes(mg.OP_W4A8, 1, 5376, 100) == 0  # invalid K
    assert mg.mgemm_workspace_bytes(99, 1, 1, 32) == 0
    moe4 = mg.mgemm_workspace_bytes(mg.OP_MOE_NVFP4, T=4096, H=4096, I=1536, E=64, topk=8)
    assert moe4 > 4096 * 8 * 4096 * 4 + 4096 * 8 * (1536 // 2 + 1536 // 16)
    assert mg.mgemm_workspace_bytes(mg.OP_MOE_NVFP4, T=4096, H=4096, I=1504, E=64, topk=8) == 0


def test_host_side_argument_errors(lib):
    """Argument errors are returned before any device work (so no GPU needed)."""
    p = 4096  # a 16-byte aligned dummy address, never dereferenced on these paths
    assert lib.mgemm_w4a4(None, p, p, p, p, p, p, 32, 32, 32, 0, None) == -1
    assert lib.mgemm_w4a4(p, p, p, p, p, p, p, 32, 32, 48, 0, None) == -2   # K % 32
    assert lib.mgemm_w4a4(p, p, p, p, p, p, p, 0, 32, 32, 0, None) == -2    # M = 0
    assert lib.mgemm_w4a4(p + 8, p, p, p, p, p, p, 32, 32, 32, 0, None) == -1  # misaligned
    assert lib.mgemm_w4a4(p, p, p, p, p, p, p, 32, 32, 32, 2, None) == -1   # bad out flag
    assert lib.mgemm_bf16(p, p, None, 32, 32, 32, 0, None, 0, None) == -1
    assert lib.mgemm_bf16(p, p, p, 32, -1, 32, 0, None, 0, None) == -2
    assert lib.mgemm_w4a16(p, p, p, p, p, 32, 32, 16, 0, p, 0, None) == -2
    assert lib.mgemm_w4a16(p, p, p, p, p, 8, 32, 32, 0, None, 0, None) == -4   # no workspace
    assert lib.mgemm_w4a16(p, p, p, p, p, 8, 32, 32, 0, p + 8, 1 << 20, None) == -4  # misaligned
    assert lib.mgemm_w4a16(p, p, p, p, p, 8, 32, 32, 0, p, 16, None) == -4   # too small
    assert lib.mgemm_w4a8(p, p, p, p, p, p, 8, 32, 0, 0, p, 0, None) == -2
    assert lib.mgemm_w4a8(p, None, p, p, p, p, 8, 32, 32, 0, p, 0, None) == -1
    assert lib.mgemm_w4a8(p, p, p, p, p, p, 8, (1 << 30) + 128, 14336, 0, p, 1 << 40, None) == -2
    moe = lambda **kw: lib.mgemm_moe_mxfp8_glu(  # noqa: E731
        p, p, p, p, kw.get("T", 64), kw.get("H", 128), kw.get("I", 128), kw.get("E", 4),
        kw.get("topk", 2), p, p, p, p, p, p, 1 << 30, None, None)
    assert moe(H=96) == -2
    assert moe(I=160) == -2
    assert moe(topk=17) == -2
    assert moe(E=0) == -2
    assert lib.mgemm_moe_mxfp8_glu(p, p, None, p, 64, 128, 128, 4, 2, p, p, p, p, p, p,
                                   1 << 30, None, None) == -1
    moe4 = lambda **kw: lib.mgemm_moe_nvfp4_glu(  # noqa: E731
        p, p, kw.get("Sx", p), p, p, kw.get("T", 64), kw.get("H", 128), kw.get("I", 128),
        kw.get("E", 4), kw.get("topk", 2), p, p, p, p, p, p, p, p, p, 1 << 30, None, None)
    assert moe4(H=48) == -2          # H % 32
    assert moe4(I=96) == -2          # I % 64
    assert moe4(topk=17) == -2
    assert moe4(T=0) == -2
    assert moe4(Sx=None) == -1
    assert moe4(Sx=p + 2) == -1      # FP32 scale not 4-byte aligned
    assert lib.mgemm_moe_route_topk(None, 8, 64, 8, p, p, None) == -1
    assert lib.mgemm_moe_route_topk(p, 8, 64, 65, p, p, None) == -2    # topk > E
    assert lib.mgemm_moe_route_topk(p, 8, 1025, 8, p, p, None) == -2   # E > 1024
    assert lib.mgemm_moe_route_topk(p, 0, 64, 8, p, p, None) == -2
    assert lib.mgemm_moe_route_topk(p + 2, 8, 64, 8, p, p, None) == -1


def test_binding_refuses_cpu_tensors(lib):
    a = torch.zeros((32, 32), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mg.mgemm_bf16(a, a, torch.zeros((32, 32), dtype=torch.bfloat16))
