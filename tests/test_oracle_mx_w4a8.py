"""Pins of the oracle's MX-native W4A8 path (CPU only): MXFP8 activation
encode and the MXFP8 x MXFP4 GEMM.

Page "DeepSeek-V4.1-Flash-NVFP4", section 二: the reference FP8 x FP4 GEMM
quantizes activations in blocks and weights in 32-element blocks with
power-of-two scales and applies the block scales inside the accumulation.
The encoder is checked element by element against a nearest search over
torch's E4M3 value table (ties to the even code) and against the scale rule
(the block maximum lands in (224, 448] after scaling); the GEMM against an
exact rational sum of independently decoded operands and an integer matmul.
"""
import os
from fractions import Fraction

import numpy as np
import torch

from precision_moe_gemm_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _e4m3_table():
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def _mags():
    return np.array([float(l) for l in open(os.path.join(GOLDEN, "e2m1_magnitudes.txt"))
                     if l.strip() and not l.startswith("#")])


def _fp4_values(packed):
    nib = np.stack([packed & 15, packed >> 4], -1).reshape(packed.shape[0], -1)
    return np.where(nib & 8, -1.0, 1.0) * _mags()[nib & 7]


def _bf16_to_f64(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _nearest_e4m3_codes(y):
    """Nearest non-negative finite E4M3 code to |y| (ties: even code)."""
    tab = _e4m3_table()[:0x7F]  # codes 0x00..0x7E
    d = np.abs(np.abs(y)[..., None] - tab[None, :])
    best = d.min(-1, keepdims=True)
    cand = np.where(d == best, np.arange(0x7F), 1 << 20)
    even = np.where(cand % 2 == 0, cand, 1 << 20).min(-1)
    return np.where(even < (1 << 20), even, cand.min(-1)).astype(np.uint8)


def test_mxfp8_encode_bruteforce(orc):
    x = synth.normal_bf16((7, 256), 1.0, (120, 0))
    x = synth.with_outliers(x, 0.03, 30.0, (120, 1))
    xb = synth.bits(x)
    q, e8 = orc.mxfp8_encode(xb)
    xv = _bf16_to_f64(xb).reshape(7, 8, 32)
    amax = np.abs(xv).max(-1)
    e = e8.astype(np.int64) - 127
    # scale rule: the block maximum lands in (224, 448] after scaling
    scaled = amax * np.exp2(-e.astype(np.float64))
    assert np.all((scaled > 224) & (scaled <= 448))
    # elements: nearest E4M3 of |x| 2^-e, sign of x
    y = np.abs(xv) * np.exp2(-e.astype(np.float64))[..., None]
    ref = _nearest_e4m3_codes(y.reshape(7, 256)) | np.where(np.signbit(_bf16_to_f64(xb)), 0x80, 0).astype(np.uint8)
    assert np.array_equal(q, ref)


def test_mxfp8_encode_ties_zero_block_and_signs(orc):
    # block 0: amax 448 (e = 0), then exact midpoints between E4M3 values:
    # 1.0625 lies between 1.0 (0x38) and 1.125 (0x39): ties to even -> 0x38;
    # 1.1875 between 1.125 (0x39) and 1.25 (0x3A) -> 0x3A
    vals = np.zeros((2, 32), np.float32)
    vals[0, 0] = 448.0
    vals[0, 1] = 1.0625
    vals[0, 2] = -1.1875
    vals[0, 3] = -0.0
    bits = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bits[1, :] = 0x8000  # block of -0.0: all-zero block
    q, e8 = orc.mxfp8_encode(bits)
    assert e8[0, 0] == 127 and e8[1, 0] == 127
    assert q[0, 0] == 0x7E and q[0, 1] == 0x38 and q[0, 2] == 0xBA and q[0, 3] == 0x80
    assert np.all(q[1] == 0x80)
    # 450 (the next bf16 above 448) would saturate at e = 0: the scale steps
    # up one octave instead (450 / 2 = 225 -> 224)
    bits2 = torch.tensor([[450.0] + [1.0] * 31]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    q2, e82 = orc.mxfp8_encode(bits2)
    assert e82[0, 0] == 128 and _e4m3_table()[q2[0, 0]] == 224.0


def test_mx_w4a8_exact_rational_sum(orc):
    a, ae = orc.mxfp8_encode(synth.bits(synth.normal_bf16((3, 64), 1.0, (121, 0))))
    wp, we = orc.mxfp4_encode(synth.bits(synth.normal_bf16((4, 64), 0.02, (121, 1))))
    C = orc.mx_gemm_w4a8(a, ae, wp, we)
    tab = _e4m3_table()
    av, wv = tab[a], _fp4_values(wp)
    for i in range(3):
        for j in range(4):
            exact = Fraction(0)
            for b in range(2):
                s = Fraction(2) ** (int(ae[i, b]) - 127 + int(we[j, b]) - 127)
                exact += s * sum(Fraction(av[i, k]) * Fraction(wv[j, k]) for k in range(32 * b, 32 * b + 32))
            assert abs(Fraction(C[i, j]) - exact) <= abs(exact) * Fraction(1, 2 ** 50)


def test_mx_w4a8_integer_special_case(orc):
    """All scales 2^0 and small-integer operands: an integer matmul."""
    rng = np.random.default_rng(122)
    M, N, K = 5, 6, 96
    tab = _e4m3_table()
    ints = [c for c in range(0x7F) if float(tab[c]).is_integer() and tab[c] <= 16]
    a = rng.choice(ints, (M, K)).astype(np.uint8) | (rng.integers(0, 2, (M, K)) * 0x80).astype(np.uint8)
    wp = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    ae = np.full((M, K // 32), 127, np.uint8)
    we = np.full((N, K // 32), 127, np.uint8)
    C = orc.mx_gemm_w4a8(a, ae, wp, we)
    ref = tab[a] @ _fp4_values(wp).T
    assert np.array_equal(C, ref)
