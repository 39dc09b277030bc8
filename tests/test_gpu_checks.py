"""The operand data checks (nvfp4_set_checks / NVFP4_CHECK): NaN-pattern and
negative block scales, a non-positive global and a non-finite bf16 input
raise the sticky NVFP4_ERR_DATA; with the checks off the same calls report
nothing.  Planted values only change data, never addresses, so every kernel
still reads and writes inside its buffers."""
import pytest
import torch

import precision_moe_gemm_amd as nv
from precision_moe_gemm_amd import _lib, synth
from tests.gpu_util import step

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture
def checks():
    prev = nv.nvfp4_set_checks(True)
    assert nv.nvfp4_get_error() == 0
    yield
    nv.nvfp4_set_checks(prev)
    nv.nvfp4_get_error()


def _operands():
    A = nv.nvfp4_quantize(synth.normal_bf16((8, 256), 1.0, (90, 0), DEV))
    W = nv.nvfp4_quantize(synth.normal_bf16((64, 256), 0.02, (90, 1), DEV))
    return A, W


@pytest.mark.parametrize("byte", [0x7F, 0xFF, 0xB8, 0x80])
def test_bad_scale_byte_raises(checks, byte):
    A, W = _operands()
    W.scales[0, 5, 3] = byte
    step(f"checks: scale byte {byte:#x}")
    nv.nvfp4_gemm(A, W)
    assert nv.nvfp4_get_error() == _lib.DATA


def test_good_operands_pass(checks):
    A, W = _operands()
    step("checks: clean operands")
    nv.nvfp4_gemm(A, W)
    nv.nvfp4_dequantize(W)
    assert nv.nvfp4_get_error() == 0


def test_bad_global_raises(checks):
    A, W = _operands()
    W.global_.fill_(-1.0)
    step("checks: negative global")
    nv.nvfp4_dequantize(W)
    assert nv.nvfp4_get_error() == _lib.DATA


def test_non_finite_input_raises(checks):
    x = synth.normal_bf16((4, 64), 1.0, (90, 2), DEV)
    x[2, 17] = float("inf")
    step("checks: inf input to quantize")
    nv.nvfp4_quantize(x)
    assert nv.nvfp4_get_error() == _lib.DATA


def test_moe_weights_checked(checks):
    cfg = synth.MoE(seed=91, E=3, k=2, H=256, I=128, T=20)
    from precision_moe_gemm_amd import workloads
    W = workloads.build_moe_weights(cfg, DEV)
    x = cfg.x(DEV)
    ids, w = workloads.routing(cfg, DEV)
    nv.nvfp4_moe_grouped_gemm(x, ids, w, W.w13, W.w2)
    assert nv.nvfp4_get_error() == 0
    W.w2.scales[2, 100, 4] = 0x7F
    step("checks: NaN scale in one expert's w2")
    nv.nvfp4_moe_grouped_gemm(x, ids, w, W.w13, W.w2)
    assert nv.nvfp4_get_error() == _lib.DATA


def test_checks_off_report_nothing():
    prev = nv.nvfp4_set_checks(False)
    try:
        A, W = _operands()
        W.scales[0, 5, 3] = 0x7F
        step("checks off: NaN scale byte")
        nv.nvfp4_gemm(A, W)
        assert nv.nvfp4_get_error() == 0
    finally:
        nv.nvfp4_set_checks(prev)
