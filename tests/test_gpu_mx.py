"""GPU parity: MXFP4 encode and the lossless MXFP4 -> NVFP4 remap vs the oracle.

Bar: bit-exact codes, E8M0 bytes, E4M3 scale bytes and globals; the remapped
tensor dequantizes to exactly the MXFP4 values; out-of-range exponent spreads
raise the sticky range error.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_moe_gemm_amd as nv
from precision_moe_gemm_amd import synth, workloads
from tests.gpu_util import assert_same_nvfp4, step, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _mx_cases():
    yield "tiny_linear_w", synth.bits(synth.C1.w())
    yield "normal", synth.bits(synth.normal_bf16((96, 1024), 1.0, (400, 0)))
    rows = np.zeros((4, 128), np.float32)
    rows[0, :32] = 0                                  # zero block
    rows[0, 32:] = np.linspace(-3, 3, 96)
    rows[1] = np.r_[np.full(32, 1e-39), np.full(96, 2.0)]  # bf16 subnormal block
    rows[2] = np.r_[np.full(64, 3e38), np.full(64, -1e-30)]
    rows[3] = np.r_[np.full(32, 6.0), np.full(32, 5.0), np.full(32, 0.75), np.full(32, -0.25)]
    yield "edges", synth.bits(torch.from_numpy(rows).to(torch.bfloat16))


@pytest.mark.parametrize("case", ["tiny_linear_w", "normal", "edges"])
def test_mxfp4_encode(orc, case):
    xb = dict(_mx_cases())[case]
    step(f"mxfp4 encode {case}")
    p, e = nv.mxfp4_quantize(synth.from_bits(xb, DEV))
    rp, re = orc.mxfp4_encode(xb)
    np.testing.assert_array_equal(u8(e), re)
    np.testing.assert_array_equal(u8(p), rp)


@pytest.mark.parametrize("in_place", [False, True])
def test_remap_single(orc, in_place):
    xb = synth.bits(synth.C1.w())
    rp, re = orc.mxfp4_encode(xb)
    ref = orc.mxfp4_to_nvfp4(rp, re)
    step(f"remap tiny linear in_place={in_place}")
    p = torch.from_numpy(rp).to(DEV)
    e = torch.from_numpy(re).to(DEV)
    nvt = nv.mxfp4_to_nvfp4(p, e, 256, 512, 1, in_place=in_place)
    assert_same_nvfp4(nvt, ref)
    assert nv.nvfp4_get_error() == 0
    # lossless: the NVFP4 values are exactly the MXFP4 values
    f = nv.nvfp4_dequantize(nvt).cpu().numpy()
    np.testing.assert_array_equal(f.view(np.uint32), orc.mxfp4_dequantize(rp, re).view(np.uint32))


def test_remap_batched_per_expert_globals(orc):
    mats = [synth.bits(synth.normal_bf16((64, 256), 10.0 ** (i - 2), (401, i))) for i in range(5)]
    enc = [orc.mxfp4_encode(m) for m in mats]
    p = torch.from_numpy(np.stack([a for a, _ in enc])).to(DEV)
    e = torch.from_numpy(np.stack([b for _, b in enc])).to(DEV)
    step("remap batched")
    nvt = nv.mxfp4_to_nvfp4(p, e, 64, 256, 5)
    for i, (a, b) in enumerate(enc):
        ref = orc.mxfp4_to_nvfp4(a, b)
        np.testing.assert_array_equal(u8(nvt.packed[i]), ref.packed)
        np.testing.assert_array_equal(u8(nvt.scales[i]), ref.scales)
        assert np.float32(nvt.global_[i].item()) == ref.G
    assert nv.nvfp4_get_error() == 0


def test_remap_zero_blocks_and_spread(orc):
    packed = np.full((2, 64), 0x22, np.uint8)     # every code 1.0
    packed[1, 16:32] = 0x88                        # a zero block (negative zeros)
    e8 = np.full((2, 4), 127, np.uint8)
    e8[0, 0] = 136
    e8[1, 0] = 119                                  # spread exactly 17 octaves
    e8[1, 1] = 250                                  # zero block: its exponent is ignored
    ref = orc.mxfp4_to_nvfp4(packed, e8)
    step("remap spread 17")
    nvt = nv.mxfp4_to_nvfp4(torch.from_numpy(packed).to(DEV), torch.from_numpy(e8).to(DEV), 2, 128, 1)
    assert_same_nvfp4(nvt, ref)
    assert nv.nvfp4_get_error() == 0


def test_remap_range_error_is_raised(orc):
    packed = np.full((1, 64), 0x22, np.uint8)
    e8 = np.array([[140, 127, 127, 122]], np.uint8)  # 18 octaves
    with pytest.raises(orc.OracleError):
        orc.mxfp4_to_nvfp4(packed, e8)
    step("remap spread 18 (range error expected)")
    nv.mxfp4_to_nvfp4(torch.from_numpy(packed).to(DEV), torch.from_numpy(e8).to(DEV), 1, 128, 1)
    assert nv.nvfp4_get_error() == 3
    assert nv.nvfp4_get_error() == 0  # cleared by the read


def test_moe_experts_mx_build_sampled(orc):
    """384-expert layer share (w1/w3 2048x7168, w2 7168x2048), reduced to 6
    experts here; encode + remap of [w1; w3] as one tensor, bit-exact."""
    cfg = synth.C4_DECODE.scaled(E=6)
    step("mx experts build E=6 H=7168 I=2048")
    W = workloads.build_moe_weights(cfg, DEV, keep_mx=True)
    for e in (0, 5):
        w13 = synth.bits(cfg.w13(e, DEV))
        rp, re = orc.mxfp4_encode(w13)
        np.testing.assert_array_equal(u8(W.mx13[1][e]), re)
        np.testing.assert_array_equal(u8(W.mx13[0][e]), rp)
        ref = orc.mxfp4_to_nvfp4(rp, re)
        np.testing.assert_array_equal(u8(W.w13.scales[e]), ref.scales)
        np.testing.assert_array_equal(u8(W.w13.packed[e]), ref.packed)
        assert np.float32(W.w13.global_[e].item()) == ref.G
        w2 = synth.bits(cfg.w2(e, DEV))
        rp2, re2 = orc.mxfp4_encode(w2)
        ref2 = orc.mxfp4_to_nvfp4(rp2, re2)
        np.testing.assert_array_equal(u8(W.w2.scales[e]), ref2.scales)
        assert np.float32(W.w2.global_[e].item()) == ref2.G
    assert nv.nvfp4_get_error() == 0
