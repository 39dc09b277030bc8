"""CPU-side checks of the C ABI (no GPU needed, no compute calls):
the library loads, exports every function include/nvfp4.h declares, and the
host-only entry points (status strings, recipe, workspace sizes, argument
validation that fails before any launch) behave as documented."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")
LIB = os.environ.get("NVFP4_LIB_PATH") or os.path.join(ROOT, "precision_moe_gemm_amd", "libnvfp4.so")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s+\*?([a-z][a-z0-9_]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(n for n in names if n.startswith(("nvfp4_", "mxfp4_", "mxfp8_", "mx_"))))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from precision_moe_gemm_amd import build
        build.build()
    from precision_moe_gemm_amd import _lib
    return _lib.load()


def test_header_declares_the_boundary():
    names = _declared()
    for n in ["nvfp4_quantize", "nvfp4_dequantize", "mxfp4_to_nvfp4", "nvfp4_gemm",
              "nvfp4_moe_grouped_gemm", "nvfp4_kv_quant", "nvfp4_kv_dequant"]:
        assert n in names, n


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(LIB)
    for n in _declared():
        assert hasattr(raw, n), f"{n} not exported"
    from precision_moe_gemm_amd import _lib
    assert set(_declared()) == set(_lib.SIGNATURES), "binding and header disagree"


def test_status_strings_and_recipe(lib):
    import precision_moe_gemm_amd as nv
    assert nv.status_string(0) == "ok"
    assert "range" in nv.status_string(3)
    assert nv.nvfp4_recipe() == [16, 2, 1, 4, 3, 450]


def test_workspace_sizes(lib):
    import precision_moe_gemm_amd as nv
    from precision_moe_gemm_amd import _lib
    assert nv.nvfp4_workspace_size(_lib.OP_QUANTIZE) == 4096
    assert nv.nvfp4_workspace_size(_lib.OP_GEMM) == 0
    # few-row GEMMs with a long K split it: partial sums M x N fp32 per split
    sk = nv.nvfp4_workspace_size(_lib.OP_GEMM, 1, 0, 0, 17408, 5120)
    assert sk >= 2 * 5120 * 4 and sk % 256 == 0
    assert nv.nvfp4_workspace_size(_lib.OP_GEMM, 32, 0, 0, 17408, 5120) <= 32 << 20
    # many rows (MFMA-bound tiles) or a K that is not a multiple of 256: no split
    assert nv.nvfp4_workspace_size(_lib.OP_GEMM, 8192, 0, 0, 5120, 34816) == 0
    assert nv.nvfp4_workspace_size(_lib.OP_GEMM, 1, 0, 0, 192, 5120) == 0
    a = nv.nvfp4_workspace_size(_lib.OP_MOE, 4096, 10, 512, 4096, 1024)
    b = nv.nvfp4_workspace_size(_lib.OP_MOE, 4096, 10, 512, 4096, 2048)
    assert 0 < a < b
    # the dominant terms: h bf16, hq, y fp32 over T*k rows
    assert a > 40960 * (1024 * 2 + 1024 // 2 + 4096 * 4)
    assert nv.nvfp4_workspace_size(_lib.OP_MOE_ROUTE, 64, 8, 384) > 0


def test_host_validation_fails_before_launch(lib):
    from precision_moe_gemm_amd import _lib
    T = _lib.NVFP4TensorC(0, 0, 0, 4, 32, 1)
    # null global -> invalid argument
    assert lib.nvfp4_quantize(None, 4, 32, 32, None, ctypes.byref(T), None, 0, None) == _lib.INVALID_ARG
    # cols not a multiple of 16 -> shape
    T2 = _lib.NVFP4TensorC(16, 16, 16, 4, 24, 1)
    assert lib.nvfp4_dequantize(ctypes.byref(T2), ctypes.c_void_p(16), 0, None) == _lib.SHAPE
    # misaligned packed pointer -> invalid argument
    T3 = _lib.NVFP4TensorC(8, 16, 16, 4, 32, 1)
    assert lib.nvfp4_dequantize(ctypes.byref(T3), ctypes.c_void_p(16), 0, None) == _lib.INVALID_ARG
    # bad dtype
    T4 = _lib.NVFP4TensorC(16, 16, 16, 4, 32, 1)
    assert lib.nvfp4_dequantize(ctypes.byref(T4), ctypes.c_void_p(16), 7, None) == _lib.INVALID_ARG
    # GEMM: K any multiple of 16 (80 passes validation; mismatched K -> shape)
    A = _lib.NVFP4TensorC(16, 16, 16, 4, 80, 1)
    W = _lib.NVFP4TensorC(16, 16, 16, 8, 80, 1)
    # a workspace smaller than the split needs -> workspace error
    A1 = _lib.NVFP4TensorC(16, 16, 16, 1, 4096, 1)
    W1 = _lib.NVFP4TensorC(16, 16, 16, 256, 4096, 1)
    assert lib.nvfp4_gemm(ctypes.byref(A1), ctypes.byref(W1), ctypes.c_void_p(16), 0, ctypes.c_void_p(256), 64,
                          None) == _lib.WORKSPACE
    W2 = _lib.NVFP4TensorC(16, 16, 16, 8, 96, 1)
    assert lib.nvfp4_gemm(ctypes.byref(A), ctypes.byref(W2), ctypes.c_void_p(16), 0, None, 0, None) == _lib.SHAPE
    # remap: cols % 32
    O = _lib.NVFP4TensorC(16, 16, 16, 4, 48, 1)
    assert lib.mxfp4_to_nvfp4(ctypes.c_void_p(16), ctypes.c_void_p(16), 4, 48, 1, ctypes.byref(O),
                              ctypes.c_void_p(256), 1 << 20, None) == _lib.SHAPE
    # MoE: too many experts, workspace too small
    w13 = _lib.NVFP4TensorC(16, 16, 16, 256, 128, 5000)
    w2 = _lib.NVFP4TensorC(16, 16, 16, 128, 128, 5000)
    assert lib.nvfp4_moe_grouped_gemm(ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), 8, 2,
                                      5000, ctypes.byref(w13), ctypes.byref(w2), None, ctypes.c_void_p(16),
                                      ctypes.c_void_p(256), 1 << 30, None) == _lib.SHAPE
    w13 = _lib.NVFP4TensorC(16, 16, 16, 256, 128, 4)
    w2 = _lib.NVFP4TensorC(16, 16, 16, 128, 128, 4)
    assert lib.nvfp4_moe_grouped_gemm(ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), 8, 2,
                                      4, ctypes.byref(w13), ctypes.byref(w2), None, ctypes.c_void_p(16),
                                      ctypes.c_void_p(256), 64, None) == _lib.WORKSPACE
    # MoE: hidden size not a multiple of 16 -> shape (I = 40 is one: tensor cols)
    w13 = _lib.NVFP4TensorC(16, 16, 16, 80, 40, 4)
    w2 = _lib.NVFP4TensorC(16, 16, 16, 40, 40, 4)
    assert lib.nvfp4_moe_grouped_gemm(ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), 8, 2,
                                      4, ctypes.byref(w13), ctypes.byref(w2), None, ctypes.c_void_p(16),
                                      ctypes.c_void_p(256), 1 << 30, None) == _lib.SHAPE
    # KV write past the cache end -> shape
    kc = _lib.NVFP4TensorC(16, 16, 16, 64, 256, 1)
    assert lib.nvfp4_kv_quant(ctypes.c_void_p(16), None, 9, 4, 8, ctypes.byref(kc), ctypes.byref(kc),
                              None) == _lib.SHAPE


def test_tiled_scale_rules_fail_before_launch(lib):
    """NVFP4_TILED_SCALES: whole 128-row x 256-column tiles only, weight
    operands only, and the conversion refuses bad shapes, tiled inputs and
    overlapping buffers, all on the host."""
    from precision_moe_gemm_amd import _lib
    TL = _lib.TILED_SCALES
    # conversion: rows % 128, cols % 256
    assert lib.nvfp4_tile_scales(ctypes.byref(_lib.NVFP4TensorC(16, 16, 16, 64, 256, 1)), ctypes.c_void_p(4096),
                                 None) == _lib.SHAPE
    assert lib.nvfp4_tile_scales(ctypes.byref(_lib.NVFP4TensorC(16, 16, 16, 128, 128, 1)), ctypes.c_void_p(4096),
                                 None) == _lib.SHAPE
    # an already tiled input, an overlapping output, a misaligned output
    assert lib.nvfp4_tile_scales(ctypes.byref(_lib.NVFP4TensorC(16, 16, 16, 128, 256, 1, TL)),
                                 ctypes.c_void_p(1 << 20), None) == _lib.INVALID_ARG
    assert lib.nvfp4_tile_scales(ctypes.byref(_lib.NVFP4TensorC(16, 4096, 16, 128, 256, 1)),
                                 ctypes.c_void_p(4096 + 1024), None) == _lib.INVALID_ARG
    assert lib.nvfp4_tile_scales(ctypes.byref(_lib.NVFP4TensorC(16, 4096, 16, 128, 256, 1)),
                                 ctypes.c_void_p(1 << 20 | 4), None) == _lib.INVALID_ARG
    # tiled tensors outside weight operands are refused
    t = _lib.NVFP4TensorC(16, 16, 16, 128, 256, 1, TL)
    assert lib.nvfp4_dequantize(ctypes.byref(t), ctypes.c_void_p(16), 0, None) == _lib.UNSUPPORTED
    assert lib.nvfp4_gather_dequantize(ctypes.byref(t), ctypes.c_void_p(16), 1, ctypes.c_void_p(16), 0,
                                       None) == _lib.UNSUPPORTED
    W = _lib.NVFP4TensorC(16, 16, 16, 128, 256, 1)
    assert lib.nvfp4_gemm(ctypes.byref(t), ctypes.byref(W), ctypes.c_void_p(16), 0, None, 0,
                          None) == _lib.UNSUPPORTED
    # a tiled weight with a partial 128-row tile -> shape
    W3 = _lib.NVFP4TensorC(16, 16, 16, 96, 256, 1, TL)
    A = _lib.NVFP4TensorC(16, 16, 16, 4, 256, 1)
    assert lib.nvfp4_gemm(ctypes.byref(A), ctypes.byref(W3), ctypes.c_void_p(16), 0, None, 0, None) == _lib.SHAPE


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    from precision_moe_gemm_amd import _lib
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError):
        _lib.load()


def test_stale_library_is_refused(lib, monkeypatch):
    """The loader compares the library's build stamp (a hash of the sources
    and flags it was built from) with the source tree."""
    from precision_moe_gemm_amd import _lib, build
    assert lib.nvfp4_build_stamp().decode() == build.source_hash()
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(build, "source_hash", lambda: "0123456789abcdef")
    with pytest.raises(ImportError, match="other sources"):
        _lib.load()


def test_check_switch_is_host_state(lib):
    """nvfp4_set_checks returns the previous setting (host only, no launch)."""
    prev = lib.nvfp4_set_checks(1)
    assert lib.nvfp4_set_checks(0) == 1
    assert lib.nvfp4_set_checks(prev) == 0
    import precision_moe_gemm_amd as nv
    assert "invalid data" in nv.status_string(7)
