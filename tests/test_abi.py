"""The C-ABI library loads and exports every entry point include/bsp.h declares; host-side
argument validation returns the documented status codes before anything touches a GPU."""
import ctypes
import os
import re

import pytest

import block_scaled_precision_nvfp4_amd as bsp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    hdr = open(os.path.join(ROOT, "include", "bsp.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+(bsp_\w+)\s*\(", hdr, re.M)))


def test_library_exports_every_declared_symbol():
    lib = bsp.lib()
    names = declared_symbols()
    assert len(names) >= 11, names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(bsp.SIGNATURES), "binding signatures must cover the header exactly"


def test_version_and_sf_bytes():
    assert bsp.bsp_version() == 100
    assert bsp.bsp_nvfp4_sf_bytes(32760, 5120) == 32768 * 320
    assert bsp.bsp_nvfp4_sf_bytes(1, 16) == 128 * 4
    assert bsp.bsp_nvfp4_sf_bytes(0, 64) == 0
    assert bsp.bsp_nvfp4_sf_bytes(129, 80) == 256 * 8
    assert bsp.bsp_mxfp4_sf_bytes(32760, 5120) == 32768 * 160
    assert bsp.bsp_mxfp4_sf_bytes(1, 32) == 128 * 4


def _st(fn, *args):
    st = getattr(bsp.lib(), fn)(*args)
    return st, bsp.lib().bsp_last_error().decode()


P = ctypes.c_void_p(16)  # never dereferenced: validation fails (or returns) before any launch


def test_quantize_shape_errors():
    st, msg = _st("bsp_nvfp4_quantize", P, 4, 24, 24, P, P, P, None)
    assert st == -2 and "multiple of 16" in msg
    st, _ = _st("bsp_nvfp4_quantize", P, 4, 32, 16, P, P, P, None)   # ld < K
    assert st == -2
    st, _ = _st("bsp_nvfp4_quantize", P, -1, 32, 32, P, P, P, None)
    assert st == -1
    st, _ = _st("bsp_nvfp4_quantize", None, 4, 32, 32, P, P, P, None)
    assert st == -1
    assert _st("bsp_nvfp4_quantize", None, 0, 32, 32, None, None, None, None)[0] == 0   # M == 0: no-op
    st, _ = _st("bsp_mxfp8_quantize", P, 4, 48, 48, P, P, None)
    assert st == -2


def test_gemm_shape_and_dtype_errors():
    st, msg = _st("bsp_mm_fp4", P, P, P, P, P, 8, 8, 96, P, 8, 0, None)
    assert st == -2 and "multiple of 64" in msg
    st, _ = _st("bsp_mm_fp4", P, P, P, P, P, 8, 8, 128, P, 8, 7, None)
    assert st == -3
    st, _ = _st("bsp_mm_fp4", P, P, P, P, P, 8, 16, 128, P, 8, 0, None)   # ldc < N
    assert st == -2
    st, msg = _st("bsp_mm_fp4", P, P, P, P, P, 8, 8, (1 << 24) + 64, P, 8, 0, None)
    assert st == -2 and "at most 16777216" in msg
    assert _st("bsp_mm_fp4", None, None, None, None, None, 0, 8, 128, None, 8, 0, None)[0] == 0
    st, _ = _st("bsp_mm_mxfp8", P, P, P, P, 8, 8, 64, P, 8, 0, None)
    assert st == -2
    st, _ = _st("bsp_mm_fp4", None, P, P, P, P, 8, 8, 128, P, 8, 0, None)
    assert st == -1
    st, _ = _st("bsp_mm_mxfp4", P, P, P, P, None, 8, 8, 64, P, 8, 0, None)
    assert st == -2
    assert _st("bsp_mm_mxfp4", None, None, None, None, None, 8, 0, 128, None, 8, 0, None)[0] == 0
    assert _st("bsp_mxfp4_quantize", P, 4, 48, 48, P, P, None)[0] == -2


def test_prequantize_and_alpha_null_checks():
    assert _st("bsp_nvfp4_prequantize_weight", P, 8, 40, 40, P, P, P, P, P, None)[0] == -2
    assert _st("bsp_nvfp4_alpha", None, P, P, None)[0] == -1
    assert _st("bsp_nvfp4_global_sf", P, 2, 8, 8, None, P, P, None)[0] == -1
    assert _st("bsp_gelu_tanh_bf16", P, P, -1, None)[0] == -1
    # prequantization checks the quantize step's arguments before launching its global-scale step
    st, msg = _st("bsp_nvfp4_prequantize_weight", P, 8, 64, 64, ctypes.c_void_p(18), P, P, P, P, None)
    assert st == -1 and "aligned" in msg
    st, msg = _st("bsp_nvfp4_prequantize_weight", P, 8, 64, 32, P, P, P, P, P, None)
    assert st == -2 and "ld" in msg


def test_python_binding_rejects_bad_inputs_before_the_library():
    import torch
    with pytest.raises(TypeError):
        bsp.bsp_nvfp4_quantize(torch.zeros(4, 16, dtype=torch.int32), torch.ones(1))
    with pytest.raises(ValueError):
        bsp.bsp_nvfp4_quantize(torch.zeros(4, 16, dtype=torch.bfloat16), torch.ones(1))  # CPU tensor


def test_producer_fused_per_token_and_8x4_entry_point_errors():
    # GELU-fused quantize: same rules as the plain quantize
    assert _st("bsp_nvfp4_quantize_gelu", P, 4, 24, 24, P, P, P, None)[0] == -2
    assert _st("bsp_nvfp4_quantize_gelu", None, 0, 32, 32, None, None, None, None)[0] == 0
    # per-token quantize and GEMM
    assert _st("bsp_nvfp4_quantize_per_token", P, 4, 24, 24, P, P, P, None)[0] == -2
    assert _st("bsp_nvfp4_quantize_per_token", P, 4, 32, 32, P, P, None, None)[0] == -1   # gsf_rows
    assert _st("bsp_nvfp4_quantize_per_token", None, 0, 32, 32, None, None, None, None)[0] == 0
    assert _st("bsp_mm_fp4_per_token", P, P, P, P, P, P, 8, 8, 96, P, 8, 0, None)[0] == -2
    assert _st("bsp_mm_fp4_per_token", P, P, P, P, None, P, 8, 8, 128, P, 8, 0, None)[0] == -1
    assert _st("bsp_mm_fp4_per_token", P, P, P, P, P, P, 8, 8, 128, P, 8, 5, None)[0] == -3
    # layout_8x4 and the 4over6 scale
    assert _st("bsp_nvfp4_quantize_8x4", P, 4, 40, 40, P, P, P, None)[0] == -2
    assert _st("bsp_mm_fp4_8x4", P, P, P, P, P, 8, 8, 96, P, 8, 0, None)[0] == -2
    assert _st("bsp_mm_fp4_8x4", None, None, None, None, None, 0, 8, 128, None, 8, 0, None)[0] == 0
    assert _st("bsp_nvfp4_global_sf_4over6", P, 2, 8, 8, None, P, P, None)[0] == -1
    assert _st("bsp_nvfp4_global_sf_4over6", P, 2, 8, 4, P, P, P, None)[0] == -2        # ld < K


def test_sf_bytes_8x4():
    assert bsp.bsp_nvfp4_sf_bytes_8x4(1, 5120) == 8 * 320
    assert bsp.bsp_nvfp4_sf_bytes_8x4(13, 80) == 16 * 8
    assert bsp.bsp_nvfp4_sf_bytes_8x4(0, 64) == 0


def test_plain_c_consumer_compiles_links_and_runs(tmp_path):
    """include/bsp.h is a C header: a C99 program compiles against it, links libbsp.so and gets
    the documented results from the host-side paths (no GPU needed)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    libdir = os.path.dirname(bsp.lib()._name)
    exe = str(tmp_path / "c_consumer")
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "c_consumer.c"), "-L", libdir, "-lbsp",
                        f"-Wl,-rpath,{libdir}", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "c consumer ok" in r.stdout, (r.stdout, r.stderr)


def test_bias_entry_point_errors():
    """Null or misaligned bias pointers are rejected before any launch; M == 0 is a no-op."""
    st, msg = _st("bsp_mm_fp4_bias", P, P, P, P, P, None, 8, 8, 128, P, 8, 0, None)
    assert st == -1 and "bias" in msg
    assert _st("bsp_mm_fp4_bias", P, P, P, P, P, ctypes.c_void_p(17), 8, 8, 128, P, 8, 0, None)[0] == -1
    assert _st("bsp_mm_fp4_bias", P, P, P, P, P, P, 8, 8, 96, P, 8, 0, None)[0] == -2
    assert _st("bsp_mm_fp4_bias", None, None, None, None, None, None, 0, 8, 128, None, 8, 0, None)[0] == 0
    st, msg = _st("bsp_mm_mxfp8_bias", P, P, P, P, ctypes.c_void_p(18), 8, 8, 128, P, 8, 0, None)
    assert st == -1 and "bias" in msg
    assert _st("bsp_mm_mxfp8_bias", P, P, P, P, P, 8, 8, 64, P, 8, 0, None)[0] == -2
    assert _st("bsp_mm_mxfp4_bias", P, P, P, P, P, None, 8, 8, 128, P, 8, 0, None)[0] == -1
    assert _st("bsp_mm_mxfp4_bias", P, P, P, P, P, P, 8, 8, 128, P, 8, 9, None)[0] == -3


def test_gelu_nvfp4_epilogue_entry_point_errors():
    """bsp_mm_fp4_gelu_nvfp4: N must be a multiple of 128, the scale output and the global scale
    must be given and the outputs aligned; M == 0 is a no-op."""
    args = (P, P, P, P, P, P)
    st, msg = _st("bsp_mm_fp4_gelu_nvfp4", *args, 8, 192, 128, P, P, None)
    assert st == -2 and "128" in msg
    assert _st("bsp_mm_fp4_gelu_nvfp4", P, P, P, P, P, None, 8, 256, 128, P, P, None)[0] == -1
    assert _st("bsp_mm_fp4_gelu_nvfp4", *args, 8, 256, 128, P, None, None)[0] == -1
    assert _st("bsp_mm_fp4_gelu_nvfp4", *args, 8, 256, 128, ctypes.c_void_p(18), P, None)[0] == -1
    assert _st("bsp_mm_fp4_gelu_nvfp4", *args, 8, 256, 128, P, ctypes.c_void_p(20), None)[0] == -1
    assert _st("bsp_mm_fp4_gelu_nvfp4", *args, 8, 256, 96, P, P, None)[0] == -2          # K % 64
    assert _st("bsp_mm_fp4_gelu_nvfp4", None, None, None, None, None, None, 0, 256, 128, None, None,
               None)[0] == 0


def test_mxfp8_gemm_scale_alignment():
    """The MXFP8 GEMMs read scale dwords: scale matrices must be 4-byte aligned."""
    st, msg = _st("bsp_mm_mxfp8", P, ctypes.c_void_p(18), P, P, 8, 8, 128, P, 8, 0, None)
    assert st == -1 and "4-byte" in msg
    assert _st("bsp_mm_mxfp8_bias", P, P, P, ctypes.c_void_p(22), P, 8, 8, 128, P, 8, 0, None)[0] == -1


def test_rmsnorm_entry_point_errors():
    """bsp_rmsnorm_bf16 / bsp_nvfp4_quantize_rmsnorm: eps must be positive and finite, K % 16 == 0,
    ld (and ldo) >= K, null pointers rejected, M == 0 is a no-op; nothing is launched on error."""
    P = ctypes.c_void_p(256)
    f = ctypes.c_float
    assert _st("bsp_rmsnorm_bf16", P, 4, 32, 32, None, f(0.0), P, 32, None)[0] == -1
    assert _st("bsp_rmsnorm_bf16", P, 4, 32, 32, None, f(-1e-6), P, 32, None)[0] == -1
    assert _st("bsp_rmsnorm_bf16", P, 4, 32, 32, None, f(float("inf")), P, 32, None)[0] == -1
    assert _st("bsp_rmsnorm_bf16", None, 0, 32, 32, None, f(3.4028234e38), None, 32, None)[0] == 0
    assert _st("bsp_rmsnorm_bf16", P, 4, 32, 32, None, f(float("nan")), P, 32, None)[0] == -1
    st, msg = _st("bsp_rmsnorm_bf16", P, 4, 24, 24, None, f(1e-6), P, 24, None)
    assert st == -2 and "multiple of 16" in msg
    assert _st("bsp_rmsnorm_bf16", P, 4, 32, 16, None, f(1e-6), P, 32, None)[0] == -2
    assert _st("bsp_rmsnorm_bf16", P, 4, 32, 32, None, f(1e-6), P, 16, None)[0] == -2
    assert _st("bsp_rmsnorm_bf16", P, 4, 32, 32, None, f(1e-6), None, 32, None)[0] == -1
    assert _st("bsp_rmsnorm_bf16", None, 0, 32, 32, None, f(1e-6), None, 32, None)[0] == 0
    q = "bsp_nvfp4_quantize_rmsnorm"
    assert _st(q, P, 4, 24, 24, None, f(1e-6), P, P, P, None)[0] == -2
    assert _st(q, P, 4, 32, 32, None, f(0.0), P, P, P, None)[0] == -1
    assert _st(q, P, 4, 32, 32, None, f(1e-6), None, P, P, None)[0] == -1
    assert _st(q, P, 4, 32, 32, None, f(1e-6), P, P, None, None)[0] == -1
    assert _st(q, P, 4, 32, 32, None, f(1e-6), P, ctypes.c_void_p(258), P, None)[0] == -1
    assert _st(q, P, 4, 32, 32, None, f(1e-6), P, P, ctypes.c_void_p(264), None)[0] == -1
    assert _st(q, None, 0, 32, 32, None, f(1e-6), None, None, None, None)[0] == 0


def test_size_limits_rejected_on_the_host():
    """One past each documented maximum returns BSP_ESHAPE before any launch (the maxima themselves
    run on the GPU in tests/test_gpu_limits.py)."""
    P = ctypes.c_void_p(256)
    m_over = 65535 * 128 + 1
    for fn in ("bsp_nvfp4_quantize", "bsp_nvfp4_quantize_gelu", "bsp_nvfp4_quantize_8x4"):
        st, msg = _st(fn, P, m_over, 32, 32, P, P, P, None)
        assert st == -2 and "too large" in msg, (fn, st, msg)
    assert _st("bsp_mxfp4_quantize", P, m_over, 32, 32, P, P, None)[0] == -2
    assert _st("bsp_mxfp8_quantize", P, 65535 * 64 + 1, 32, 32, P, P, None)[0] == -2
    st, msg = _st("bsp_mm_fp4", P, P, P, P, P, 4, 4, (1 << 24) + 64, P, 4, 0, None)
    assert st == -2 and "at most" in msg


def test_probe_library_exports_its_header():
    """libbsp_probe.so (the benchmark's ceiling probes) exports what include/bsp_probe.h declares."""
    hdr = open(os.path.join(ROOT, "include", "bsp_probe.h")).read()
    names = sorted(set(re.findall(r"^\s*int\s+(bsp_probe_\w+)\s*\(", hdr, re.M)))
    assert names == ["bsp_probe_mfma_loop", "bsp_probe_stream"], names
    lib = ctypes.CDLL(os.path.join(ROOT, "block_scaled_precision_nvfp4_amd", "libbsp_probe.so"))
    for n in names:
        assert hasattr(lib, n), n
    # argument checks return -1 before anything touches a GPU
    lib.bsp_probe_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.bsp_probe_mfma_loop(4, 1, 1, P, None) == -1
    assert lib.bsp_probe_mfma_loop(0, 0, 1, P, None) == -1
    lib.bsp_probe_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_int, ctypes.c_void_p]
    assert lib.bsp_probe_stream(2, P, P, 1, 1, None) == -1
    assert lib.bsp_probe_stream(0, ctypes.c_void_p(8), P, 1, 1, None) == -1


def test_alignment_rules_match_the_header():
    """layout_8x4 scale buffers need 4-byte alignment (dword stores and loads), 128x4 ones 16-byte:
    a 4-byte aligned 8x4 buffer passes validation (the call then fails only for want of a gfx950
    device here), a 2-byte aligned one is rejected; the same 4-byte address is rejected for 128x4."""
    a4 = ctypes.c_void_p(0x1004)
    a2 = ctypes.c_void_p(0x1002)
    st, msg = _st("bsp_nvfp4_quantize_8x4", P, 8, 64, 64, P, P, a4, None)
    assert st != -1, msg
    st, msg = _st("bsp_nvfp4_quantize_8x4", P, 8, 64, 64, P, P, a2, None)
    assert st == -1 and "4-byte aligned" in msg
    st, msg = _st("bsp_nvfp4_quantize", P, 8, 64, 64, P, P, a4, None)
    assert st == -1 and "16-byte aligned" in msg
    st, msg = _st("bsp_mm_fp4_8x4", P, a4, P, P, P, 8, 8, 128, P, 8, 0, None)
    assert st != -1, msg
    st, msg = _st("bsp_mm_fp4", P, a4, P, P, P, 8, 8, 128, P, 8, 0, None)
    assert st == -1 and "16-byte" in msg
    st, msg = _st("bsp_mxfp8_quantize", P, 4, 64, 64, a4, P, None)
    assert st == -1 and "8-byte" in msg


def test_mxfp4_frag_entry_points():
    """Fragment-layout MXFP4: sizes, and every argument rule rejected on the host before a launch."""
    pb, sb = ctypes.c_int64(0), ctypes.c_int64(0)
    assert bsp.lib().bsp_mxfp4_frag_bytes(33, 512, ctypes.byref(pb), ctypes.byref(sb)) == 0
    assert (pb.value, sb.value) == (64 * 256, 64 * 16)
    assert bsp.lib().bsp_mxfp4_frag_bytes(0, 256, ctypes.byref(pb), ctypes.byref(sb)) == 0
    assert (pb.value, sb.value) == (0, 0)
    assert bsp.lib().bsp_mxfp4_frag_bytes(4, 384, ctypes.byref(pb), ctypes.byref(sb)) == -2
    assert bsp.lib().bsp_mxfp4_frag_bytes(4, 256, None, ctypes.byref(sb)) == -1
    assert bsp.bsp_mxfp4_frag_bytes(300, 1280) == (320 * 640, 320 * 40)
    q = "bsp_mxfp4_quantize_frag"
    st, msg = _st(q, P, 4, 384, 384, P, P, None)
    assert st == -2 and "multiple of 256" in msg
    assert _st(q, P, 4, 256, 128, P, P, None)[0] == -2             # ld < K
    assert _st(q, None, 4, 256, 256, P, P, None)[0] == -1
    assert _st(q, P, 4, 256, 256, ctypes.c_void_p(20), P, None)[0] == -1   # packed not 16-aligned
    assert _st(q, P, 4, 256, 256, P, ctypes.c_void_p(24), None)[0] == -1   # sf not 16-aligned
    assert _st(q, P, 65535 * 128 + 1, 256, 256, P, P, None)[0] == -2
    assert _st(q, None, 0, 256, 256, None, None, None)[0] == 0     # M == 0: no-op
    g = "bsp_mm_mxfp4_frag"
    st, msg = _st(g, P, P, P, P, None, None, 4, 4, 384, P, 4, 0, None)
    assert st == -2 and "multiple of 256" in msg
    assert _st(g, P, P, P, P, None, None, 4, 4, 256, P, 4, 2, None)[0] == -3   # bad out dtype
    assert _st(g, P, P, P, P, None, None, 4, 8, 256, P, 4, 0, None)[0] == -2   # ldc < N
    assert _st(g, ctypes.c_void_p(24), P, P, P, None, None, 4, 4, 256, P, 4, 0, None)[0] == -1
    assert _st(g, P, ctypes.c_void_p(18), P, P, None, None, 4, 4, 256, P, 4, 0, None)[0] == -1
    assert _st(g, P, P, P, P, None, ctypes.c_void_p(17), 4, 4, 256, P, 4, 0, None)[0] == -1
    assert _st(g, P, None, P, P, None, None, 4, 4, 256, P, 4, 0, None)[0] == -1
    assert _st(g, None, None, None, None, None, None, 0, 4, 256, None, 4, 0, None)[0] == 0
    # the aligned call passes validation and fails only for want of a gfx950 device here
    st = _st(g, P, ctypes.c_void_p(20), P, P, None, ctypes.c_void_p(18), 4, 4, 256, P, 4, 0, None)[0]
    assert st not in (-1, -2, -3), st
    st, msg = _st(g, P, P, P, P, None, None, 4, 4, (1 << 24) + 256, P, 4, 0, None)
    assert st == -2 and "at most" in msg


def test_mxfp8_frag_entry_points():
    qb, sb = ctypes.c_int64(0), ctypes.c_int64(0)
    assert bsp.lib().bsp_mxfp8_frag_bytes(33, 512, ctypes.byref(qb), ctypes.byref(sb)) == 0
    assert (qb.value, sb.value) == (64 * 512, 64 * 16)
    assert bsp.lib().bsp_mxfp8_frag_bytes(4, 128, ctypes.byref(qb), ctypes.byref(sb)) == -2
    assert bsp.bsp_mxfp8_frag_bytes(300, 1280) == (320 * 1280, 320 * 40)
    q = "bsp_mxfp8_quantize_frag"
    st, msg = _st(q, P, 4, 384, 384, P, P, None)
    assert st == -2 and "multiple of 256" in msg
    assert _st(q, P, 4, 256, 128, P, P, None)[0] == -2
    assert _st(q, P, 4, 256, 256, ctypes.c_void_p(24), P, None)[0] == -1
    assert _st(q, P, 4, 256, 256, P, ctypes.c_void_p(20), None)[0] == -1
    assert _st(q, P, 65535 * 64 + 1, 256, 256, P, P, None)[0] == -2
    assert _st(q, None, 0, 256, 256, None, None, None)[0] == 0
    g = "bsp_mm_mxfp8_frag"
    st, msg = _st(g, P, P, P, P, None, 4, 4, 640, P, 4, 0, None)
    assert st == -2 and "multiple of 256" in msg
    assert _st(g, P, P, P, P, None, 4, 4, 256, P, 4, 3, None)[0] == -3
    assert _st(g, P, P, P, P, None, 4, 8, 256, P, 4, 0, None)[0] == -2
    assert _st(g, ctypes.c_void_p(24), P, P, P, None, 4, 4, 256, P, 4, 0, None)[0] == -1
    assert _st(g, P, ctypes.c_void_p(18), P, P, None, 4, 4, 256, P, 4, 0, None)[0] == -1
    assert _st(g, P, P, P, P, ctypes.c_void_p(18), 4, 4, 256, P, 4, 0, None)[0] == -1   # bias
    assert _st(g, None, None, None, None, None, 4, 0, 256, None, 4, 0, None)[0] == 0
    st = _st(g, P, ctypes.c_void_p(20), P, P, ctypes.c_void_p(20), 4, 4, 256, P, 4, 0, None)[0]
    assert st not in (-1, -2, -3), st
    st, msg = _st(g, P, P, P, P, None, 4, 4, (1 << 24) + 256, P, 4, 0, None)
    assert st == -2 and "at most" in msg


def test_nvfp4_frag_entry_points():
    """Fragment-layout NVFP4: sizes, and every argument rule rejected on the host before a launch."""
    pb = ctypes.c_int64(0)
    assert bsp.lib().bsp_nvfp4_frag_bytes(33, 192, ctypes.byref(pb)) == 0 and pb.value == 64 * 96
    assert bsp.lib().bsp_nvfp4_frag_bytes(0, 64, ctypes.byref(pb)) == 0 and pb.value == 0
    assert bsp.lib().bsp_nvfp4_frag_bytes(4, 96, ctypes.byref(pb)) == -2
    assert bsp.lib().bsp_nvfp4_frag_bytes(4, 64, None) == -1
    assert bsp.bsp_nvfp4_frag_bytes(32760, 5120) == 32768 * 2560
    for q in ("bsp_nvfp4_quantize_frag", "bsp_nvfp4_quantize_gelu_frag"):
        st, msg = _st(q, P, 4, 96, 96, P, P, P, None)
        assert st == -2 and "multiple of 64" in msg, q
        assert _st(q, P, 4, 24, 24, P, P, P, None)[0] == -2             # not even a multiple of 16
        assert _st(q, P, 4, 128, 64, P, P, P, None)[0] == -2            # ld < K
        assert _st(q, None, 4, 128, 128, P, P, P, None)[0] == -1
        assert _st(q, P, 4, 128, 128, None, P, P, None)[0] == -1        # gsf
        assert _st(q, P, 4, 128, 128, P, ctypes.c_void_p(20), P, None)[0] == -1   # packed 4- not 16-aligned
        assert _st(q, P, 4, 128, 128, P, P, ctypes.c_void_p(24), None)[0] == -1   # sf not 16-aligned
        assert _st(q, P, 65535 * 128 + 1, 128, 128, P, P, P, None)[0] == -2
        assert _st(q, None, 0, 128, 128, None, None, None, None)[0] == 0      # M == 0: no-op
    g = "bsp_mm_fp4_frag"
    st, msg = _st(g, P, P, P, P, P, None, 4, 4, 96, P, 4, 0, None)
    assert st == -2 and "multiple of 64" in msg
    assert _st(g, P, P, P, P, P, None, 4, 4, 64, P, 4, 2, None)[0] == -3   # bad out dtype
    assert _st(g, P, P, P, P, P, None, 4, 8, 64, P, 4, 0, None)[0] == -2   # ldc < N
    assert _st(g, ctypes.c_void_p(24), P, P, P, P, None, 4, 4, 64, P, 4, 0, None)[0] == -1
    assert _st(g, P, ctypes.c_void_p(20), P, P, P, None, 4, 4, 64, P, 4, 0, None)[0] == -1
    assert _st(g, P, P, P, ctypes.c_void_p(20), P, None, 4, 4, 64, P, 4, 0, None)[0] == -1
    assert _st(g, P, P, P, P, None, None, 4, 4, 64, P, 4, 0, None)[0] == -1   # alpha
    assert _st(g, P, P, P, P, P, ctypes.c_void_p(17), 4, 4, 64, P, 4, 0, None)[0] == -1   # bias
    assert _st(g, None, None, None, None, None, None, 0, 4, 64, None, 4, 0, None)[0] == 0
    # the aligned call passes validation and fails only for want of a gfx950 device here
    st = _st(g, P, P, P, P, P, ctypes.c_void_p(18), 4, 4, 64, P, 4, 0, None)[0]
    assert st not in (-1, -2, -3), st
    st, msg = _st(g, P, P, P, P, P, None, 4, 4, (1 << 24) + 64, P, 4, 0, None)
    assert st == -2 and "at most" in msg
    w = "bsp_nvfp4_prequantize_weight_frag"
    st, msg = _st(w, P, 4, 96, 96, P, P, P, P, P, None)
    assert st == -2 and "multiple of 64" in msg
    assert _st(w, P, 4, 128, 64, P, P, P, P, P, None)[0] == -2               # ld < K
    assert _st(w, P, 0, 128, 128, P, P, P, P, P, None)[0] == -1              # no rows
    assert _st(w, None, 4, 128, 128, P, P, P, P, P, None)[0] == -1
    assert _st(w, P, 4, 128, 128, P, P, P, None, P, None)[0] == -1           # inv_gsf
    assert _st(w, P, 4, 128, 128, ctypes.c_void_p(20), P, P, P, P, None)[0] == -1   # packed alignment
    assert _st(w, P, 4, 128, 128, P, ctypes.c_void_p(24), P, P, P, None)[0] == -1   # sf alignment
    assert _st(w, P, 65535 * 128 + 1, 128, 128, P, P, P, P, P, None)[0] == -2
