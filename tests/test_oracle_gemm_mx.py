"""Pins of the oracle's exact W4A4 GEMM and MXFP4 codec / remap (CPU only).

GEMM: the integer special case (all scales 1, G = 1) is an integer matmul of
E2M1 values (numpy); general operands agree with a float64 numpy matmul of the
exactly dequantized operands.  MXFP4: closed-form OCP cases, the pages'
error statements (NVFP4 more accurate than MXFP4, MXFP4 about 12% relative L2,
page "DeepSeek-V4.1-Flash-NVFP4" sections 二 and 三), the lossless remap
(sections 一/四/六) checked element by element against the MXFP4 values, and
the storage arithmetic (+1/32 byte per element).
"""
import math
import os

import numpy as np
import pytest
import torch

from precision_moe_gemm_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _mags():
    return np.array([float(l) for l in open(os.path.join(GOLDEN, "e2m1_magnitudes.txt"))
                     if l.strip() and not l.startswith("#")])


def _codes_to_values(packed):
    mags = _mags()
    nib = np.stack([packed & 15, packed >> 4], -1).reshape(packed.shape[0], -1)
    return np.where(nib & 8, -1.0, 1.0) * mags[nib & 7]


def _e4m3(b):
    return torch.from_numpy(np.ascontiguousarray(b)).view(torch.float8_e4m3fn).double().numpy()


def _exact_values(t):
    """float64 values of q * s (no global): exact."""
    v = _codes_to_values(t.packed)
    s = np.repeat(_e4m3(t.scales), 16, axis=1)
    return v * s


def test_gemm_integer_special_case(orc):
    rng = np.random.default_rng(0)
    M, N, K = 5, 7, 48
    a = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    w = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    one = np.full((1, 1), 0x38, np.uint8)
    A = orc.NVFP4(a, np.repeat(np.repeat(one, M, 0), K // 16, 1), 1.0)
    W = orc.NVFP4(w, np.repeat(np.repeat(one, N, 0), K // 16, 1), 1.0)
    C = orc.gemm(A, W)
    ref = _codes_to_values(a) @ _codes_to_values(w).T
    assert np.array_equal(C, ref)


def test_gemm_matches_float64_matmul(orc):
    x = synth.bits(synth.C1.x())
    w = synth.bits(synth.C1.w())
    A = orc.quantize(x)
    W = orc.quantize(w)
    C = orc.gemm(A, W)
    ref = (_exact_values(A) @ _exact_values(W).T) * float(A.G) * float(W.G)
    assert C.shape == (16, 256)
    np.testing.assert_allclose(C, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_gemm_row_selection_and_orientation(orc):
    x = synth.bits(synth.normal_bf16((9, 96), 1.0, (93, 0)))
    w = synth.bits(synth.normal_bf16((13, 96), 0.02, (93, 1)))
    A, W = orc.quantize(x), orc.quantize(w)
    full = orc.gemm(A, W)
    sub = orc.gemm_rows(A, W, a_rows=[8, 2, 2], w_rows=[12, 0])
    assert np.array_equal(sub, full[np.ix_([8, 2, 2], [12, 0])])
    ref = (_exact_values(A) @ _exact_values(W).T) * float(A.G) * float(W.G)
    np.testing.assert_allclose(full, ref, rtol=1e-12, atol=1e-15)


# ----------------------------------------------------------------- MXFP4

def test_mx_encode_closed_forms(orc):
    # one non-zero 2^p in a block: floor(log2 amax) - 2 = p - 2, code 4.0
    for p in (-20, -1, 0, 3, 17):
        row = np.zeros((1, 32), np.float32)
        row[0, 9] = 2.0 ** p
        xb = synth.bits(torch.from_numpy(row).to(torch.bfloat16))
        packed, e8 = orc.mxfp4_encode(xb)
        assert e8[0, 0] == p - 2 + 127
        v = _codes_to_values(packed)[0]
        assert v[9] == 4.0 and np.count_nonzero(v) == 1
    # block maximum 6 * 2^e exactly (e = 1): code 6.0
    row = np.zeros((1, 32), np.float32)
    row[0, 0] = 12.0
    row[0, 1] = -3.0
    packed, e8 = orc.mxfp4_encode(synth.bits(torch.from_numpy(row).to(torch.bfloat16)))
    assert e8[0, 0] == 1 + 127
    v = _codes_to_values(packed)[0]
    assert v[0] == 6.0 and v[1] == -1.5
    # all-zero block
    packed, e8 = orc.mxfp4_encode(np.zeros((1, 64), np.uint16))
    assert (e8 == 0).all() and (packed == 0).all()


def _e2m1_rne(a):
    """numpy round-half-even on the E2M1 grid (step 0.5 / 1 / 2), saturating at 6."""
    step = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    return np.minimum(np.round(a / step) * step, 6.0)


def test_mx_encode_values_are_nearest_on_the_block_grid(orc):
    x = synth.bits(synth.normal_bf16((8, 256), 1.0, (94, 0)))
    packed, e8 = orc.mxfp4_encode(x)
    deq = orc.mxfp4_dequantize(packed, e8).astype(np.float64)
    xv = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for r in range(8):
        for b in range(8):
            blk = xv[r, 32 * b:32 * b + 32]
            e = math.floor(math.log2(np.abs(blk).max())) - 2
            assert e8[r, b] == e + 127
            want = _e2m1_rne(np.abs(blk) / 2.0 ** e) * 2.0 ** e
            assert np.array_equal(np.abs(deq[r, 32 * b:32 * b + 32]), want)
            assert np.array_equal(np.signbit(deq[r, 32 * b:32 * b + 32]) | (want == 0),
                                  np.signbit(blk) | (want == 0))


def test_nvfp4_beats_mxfp4_and_mx_error_near_12_percent(orc):
    rec = {}
    for l in open(os.path.join(GOLDEN, "nvfp4_recipe.txt")):
        if l.strip() and not l.startswith("#"):
            k, v = l.split()
            rec[k] = float(v)
    x = synth.bits(synth.normal_bf16((256, 512), 1.0, (95, 0)))
    xv = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nv = orc.dequantize(orc.quantize(x)).astype(np.float64)
    mx = orc.mxfp4_dequantize(*orc.mxfp4_encode(x)).astype(np.float64)
    rel = lambda d: np.linalg.norm(d - xv) / np.linalg.norm(xv)
    assert rel(nv) < rel(mx)
    assert abs(rel(mx) - rec["mxfp4_rel_l2_approx"]) < 0.03


def test_remap_is_lossless_and_keeps_nibbles(orc):
    for x in (synth.bits(synth.C1.w()), synth.bits(synth.normal_bf16((64, 1024), 1.0, (96, 0)))):
        packed, e8 = orc.mxfp4_encode(x)
        nv = orc.mxfp4_to_nvfp4(packed, e8)
        assert np.array_equal(nv.packed, packed)
        mxv = orc.mxfp4_dequantize(packed, e8)
        nvv = orc.dequantize(nv)
        assert np.array_equal(mxv.view(np.uint32), nvv.view(np.uint32))
        # scales are powers of two, the largest block maps to 256 (0x78)
        assert nv.scales.max() == 0x78
        mant, _ = np.frexp(_e4m3(nv.scales))
        assert (mant == 0.5).all()
        # G is a power of two
        m, ex = math.frexp(float(nv.G))
        assert m == 0.5


def test_remap_inverse_recovers_e8m0(orc):
    x = synth.bits(synth.normal_bf16((16, 512), 1.0, (97, 0)))
    packed, e8 = orc.mxfp4_encode(x)
    nv = orc.mxfp4_to_nvfp4(packed, e8)
    s = _e4m3(nv.scales[:, 0::2]) * float(nv.G)
    back = np.log2(s) + 127
    assert np.array_equal(back.astype(np.int64), e8.astype(np.int64))
    assert np.array_equal(nv.scales[:, 0::2], nv.scales[:, 1::2])


def test_remap_wide_spread_and_range_error(orc):
    R, K = 2, 64
    packed = np.full((R, K // 2), 0x22, np.uint8)  # every code 1.0
    e8 = np.full((R, K // 32), 127, np.uint8)
    e8[0, 0] = 127 + 9
    e8[1, 1] = 127 + 9 - 17  # spread of exactly 17 octaves: allowed
    nv = orc.mxfp4_to_nvfp4(packed, e8)
    assert np.array_equal(orc.dequantize(nv).view(np.uint32),
                          orc.mxfp4_dequantize(packed, e8).view(np.uint32))
    assert nv.scales[1, 2] == 0x01  # 2^-9
    e8[1, 1] = 127 + 9 - 18
    with pytest.raises(orc.OracleError) as ei:
        orc.mxfp4_to_nvfp4(packed, e8)
    assert ei.value.code == orc.RANGE


def test_remap_zero_blocks_and_zero_tensor(orc):
    packed = np.zeros((2, 32), np.uint8)
    packed[0, :16] = 0x31
    packed[1, 16:] = 0x88  # negative zeros only: a zero block
    e8 = np.array([[120, 200], [130, 130]], np.uint8)
    nv = orc.mxfp4_to_nvfp4(packed, e8)
    assert nv.G == 2.0 ** (120 - 127 - 8)
    assert list(nv.scales[0]) == [0x78, 0x78, 0x01, 0x01]
    assert list(nv.scales[1]) == [0x01] * 4
    nv0 = orc.mxfp4_to_nvfp4(np.zeros((1, 16), np.uint8), np.full((1, 1), 50, np.uint8))
    assert nv0.G == 1.0 and (nv0.scales == 1).all()


def test_remap_storage_grows_by_one_32nd_byte_per_element(orc):
    R, K = 384, 2048
    mx_bytes = R * K // 2 + R * K // 32
    nv_bytes = R * K // 2 + R * K // 16
    assert (nv_bytes - mx_bytes) * 32 == R * K
