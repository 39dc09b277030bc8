"""Pins of the oracle's NVFP4 quantize / dequantize (CPU only).

What fixes the answer here, besides the oracle itself:
  * the pages' printed facts: 4.5 bits per element, block 16 along the last
    dimension, every scale finite and positive with maximum 448
    (page "Qwen3.8-Flash-Next-NVFP4", sections 核心 and 证据链);
  * exact rational brute force on small tensors: the scale byte is the
    E4M3 value nearest to a_b / (6 G) and each code the E2M1 grid point
    nearest to x / (s G), decided in exact arithmetic (Fractions) by this
    test's own block walk and nibble unpacking;
  * closed forms (the tensor maximum dequantizes to 6 * 448 * G ~ amax) and
    invariants (idempotence, static G == dynamic G, row independence).
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from precision_moe_gemm_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _recipe():
    d = {}
    for line in open(os.path.join(GOLDEN, "nvfp4_recipe.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            d[k] = float(v)
    return d


def _e2m1_mags():
    return [Fraction(v) for v in
            [l.strip() for l in open(os.path.join(GOLDEN, "e2m1_magnitudes.txt"))
             if l.strip() and not l.startswith("#")]]


def _e4m3_table():
    t = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).double().tolist()
    return [Fraction(v) for v in t]


def _unpack(packed):
    lo = packed & 15
    hi = packed >> 4
    return np.stack([lo, hi], axis=-1).reshape(packed.shape[0], -1)


def _bf16_values(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _nearest(cands, target):
    """index of the nearest candidate, and whether the runner-up ties within 1e-6 relative."""
    d = [abs(c - target) for c in cands]
    order = sorted(range(len(cands)), key=lambda i: d[i])
    i0, i1 = order[0], order[1]
    near_tie = (d[i1] - d[i0]) <= Fraction(1, 10 ** 6) * max(abs(target), Fraction(1, 10 ** 30))
    return i0, near_tie


def test_storage_is_4_5_bits(orc):
    rec = _recipe()
    x = synth.bits(synth.normal_bf16((48, 1024), 1.0, (90, 1)))
    q = orc.quantize(x)
    nbits = 8 * (q.packed.nbytes + q.scales.nbytes)
    assert nbits / x.size == rec["effective_bits"] == 4.5
    assert q.scales.shape[1] * rec["block_size"] == x.shape[1]


def test_scale_audit_on_workload_tensors(orc):
    """Every block scale finite and positive; the dynamic global puts the
    block holding the tensor maximum on 448 (0x7E)."""
    c = synth.C1
    for t in (c.x(), c.w()):
        q = orc.quantize(synth.bits(t))
        a = orc.audit_scales(q)
        assert a["nonfinite"] == 0 and a["nonpositive"] == 0
        assert a["at_max"] >= 1
        assert q.scales.max() == 0x7E


def test_global_is_amax_over_2688(orc):
    x = synth.bits(synth.C1.x())
    q = orc.quantize(x)
    amax = np.abs(_bf16_values(x)).max()
    assert q.G == np.float32(amax) / np.float32(6 * 448)
    # closed form: the maximum decodes to 6 * 448 * G, within 2 ulp of amax
    deq = orc.dequantize(q)
    m = np.abs(deq).max()
    assert abs(float(m) - float(amax)) <= 2 * np.spacing(np.float32(amax))


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_bruteforce_exact_rational(orc, seed):
    """Scale bytes and codes equal the exact-arithmetic nearest choices."""
    rng = np.random.default_rng(seed)
    R, K = 3, 64
    f = (rng.standard_normal((R, K)) * np.exp(rng.uniform(-3, 3, (R, 1)))).astype(np.float32)
    f[0, 5] = 0.0
    f[1, 17] = -0.0
    x = torch.from_numpy(f).to(torch.bfloat16)
    xb = synth.bits(x)
    xv = _bf16_values(xb)
    q = orc.quantize(xb)
    G = Fraction(float(q.G))
    e4 = _e4m3_table()
    mags = _e2m1_mags()
    codes = _unpack(q.packed)
    skipped = 0
    for r in range(R):
        for b in range(K // 16):
            blk = [Fraction(float(v)) for v in xv[r, 16 * b:16 * b + 16]]
            ab = max(abs(v) for v in blk)
            s_real = ab / (6 * G)
            want_s, tie = _nearest(e4, s_real)
            if tie:
                skipped += 1
                continue
            assert q.scales[r, b] == want_s
            s = e4[want_s]
            for i, v in enumerate(blk):
                c = int(codes[r, 16 * b + i])
                sign = 1 if c & 8 else 0
                assert sign == (1 if np.signbit(xv[r, 16 * b + i]) else 0)
                if s == 0:
                    assert c & 7 == 0
                    continue
                target = abs(v) / (s * G)
                if target > 6:
                    assert c & 7 == 7
                    continue
                want_c, tie = _nearest(mags, target)
                if tie:
                    skipped += 1
                    continue
                assert c & 7 == want_c, (r, b, i, float(target))
    assert skipped <= 2


def test_ties_resolve_to_even(orc):
    """Elements exactly on an E2M1 midpoint (after scaling) take the even code.
    Block: max 6 so s = 1 when G is static 1; the elements are x = midpoints."""
    vals = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -5.0, 0, 0, 0, 0, 0]
    x = synth.bits(torch.tensor([vals], dtype=torch.float32).to(torch.bfloat16))
    q = orc.quantize(x, static_G=1.0)
    assert q.scales[0, 0] == 0x38  # 1.0 = 6 / (6 * 1)
    mags = [float(m) for m in _e2m1_mags()]
    got = [mags[c & 7] for c in _unpack(q.packed)[0]]
    assert got[:11] == [6.0, 0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 0.0, 1.0, 4.0]


def test_zero_block_and_zero_tensor(orc):
    x = np.zeros((2, 32), np.uint16)
    q = orc.quantize(x)
    assert q.G == 1.0
    assert (q.scales == 0).all() and (q.packed == 0).all()
    y = synth.bits(synth.normal_bf16((2, 32), 1.0, (91, 0)))
    y[1, 16:] = 0
    q = orc.quantize(y)
    assert q.scales[1, 1] == 0
    assert (orc.dequantize(q)[1, 16:] == 0).all()


def test_negative_zero_and_tiny_negatives_decode_to_zero(orc):
    x = torch.tensor([[100.0] + [-0.0, -1e-9, 1e-9] + [0.0] * 12]).to(torch.bfloat16)
    q = orc.quantize(synth.bits(x))
    deq = orc.dequantize(q)
    assert (deq[0, 1:4] == 0).all()
    nib = _unpack(q.packed)[0]
    assert nib[1] == 8 and nib[2] == 8 and nib[3] == 0  # sign kept on zero codes


def test_idempotent_through_bf16_dequant(orc):
    x = synth.bits(synth.C1.x())
    q1 = orc.quantize(x)
    _, deq_b = orc.dequantize(q1, want_bf16=True)
    q2 = orc.quantize(deq_b)
    assert np.array_equal(q1.scales, q2.scales)
    assert np.array_equal(q1.packed, q2.packed)
    assert abs(float(q2.G) / float(q1.G) - 1) <= 2 ** -8


def test_static_global_equal_to_dynamic_gives_same_bytes(orc):
    x = synth.bits(synth.C1.w())
    q = orc.quantize(x)
    q2 = orc.quantize(x, static_G=float(q.G))
    assert q2.G == q.G
    assert np.array_equal(q.packed, q2.packed) and np.array_equal(q.scales, q2.scales)


def test_rows_are_independent_given_the_global(orc):
    x = synth.bits(synth.normal_bf16((40, 256), 1.0, (92, 0)))
    q = orc.quantize(x)
    idx = np.array([7, 3, 3, 39, 0])
    qg = orc.quantize(np.ascontiguousarray(x[idx]), static_G=float(q.G))
    assert np.array_equal(qg.packed, q.packed[idx]) and np.array_equal(qg.scales, q.scales[idx])


def test_dequantize_products_are_exact(orc):
    """With G = 1 every (code, scale) pair decodes to e2m1 * e4m3 exactly."""
    mags = [float(m) for m in _e2m1_mags()]
    e4 = [float(v) for v in _e4m3_table()]
    R = 127
    packed = np.zeros((R, 8), np.uint8)
    scales = np.zeros((R, 1), np.uint8)
    for r in range(R):
        scales[r, 0] = r
        for j in range(8):
            packed[r, j] = (2 * j) | ((2 * j + 1) << 4)  # nibbles 0..15
    t = orc.NVFP4(packed, scales, 1.0)
    deq = orc.dequantize(t)
    for r in range(R):
        for n in range(16):
            want = mags[n & 7] * e4[r] * (-1 if n & 8 else 1)
            assert deq[r, n] == np.float32(want)


def test_dequantize_bf16_is_rne_of_f32(orc):
    x = synth.bits(synth.C1.x())
    q = orc.quantize(x)
    f, b = orc.dequantize(q, want_bf16=True)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)


def test_rejects_bad_shapes_and_values(orc):
    with pytest.raises(orc.OracleError):
        orc.quantize(np.zeros((2, 24), np.uint16))
    bad = np.zeros((1, 16), np.uint16)
    bad[0, 3] = 0x7FC0  # NaN
    with pytest.raises(orc.OracleError):
        orc.quantize(bad)


def test_subnormal_scale_regime(orc):
    """Tiny blocks next to a large one use subnormal E4M3 scales; the exact
    nearest rules still hold (checked by value)."""
    vals = np.zeros((1, 64), np.float32)
    vals[0, :16] = 1000.0
    vals[0, 16:32] = np.linspace(-0.01, 0.01, 16)
    vals[0, 32:48] = np.linspace(0.001, 0.003, 16)
    xb = synth.bits(torch.from_numpy(vals).to(torch.bfloat16))
    q = orc.quantize(xb)
    assert q.scales[0, 0] == 0x7E
    assert 0 < q.scales[0, 1] < 0x08  # subnormal E4M3
    assert q.scales[0, 3] == 0


def test_gather_dequantize_selects_rows(orc):
    """Gather-dequantize is the row selection of the dequantized table: ids
    0..R-1 give the whole table, a repeated / shuffled list gives those rows
    of it, and each element is e2m1 * e4m3 * G (brute force, exact for a
    power-of-two G); ids outside [0, R) give zero rows."""
    R, K = 37, 64
    rng = np.random.default_rng(5)
    packed = rng.integers(0, 256, (R, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 127, (R, K // 16), dtype=np.uint8)
    t = orc.NVFP4(packed, scales, 0.25)
    full = orc.dequantize(t)
    assert np.array_equal(orc.gather_dequantize(t, np.arange(R)), full)
    ids = np.array([5, 0, 36, 5, 17, 17, 2], np.int32)
    g = orc.gather_dequantize(t, ids)
    assert np.array_equal(g, full[ids])
    mags = [float(m) for m in _e2m1_mags()]
    e4 = [float(v) for v in _e4m3_table()]
    for i, r in enumerate(ids):
        for c in range(K):
            nib = (packed[r, c // 2] >> (4 * (c & 1))) & 15
            want = mags[nib & 7] * e4[scales[r, c // 16]] * 0.25 * (-1 if nib & 8 else 1)
            assert g[i, c] == np.float32(want)
    bad = orc.gather_dequantize(t, np.array([3, -1, R, 4], np.int32))
    assert np.array_equal(bad[[0, 3]], full[[3, 4]]) and not bad[[1, 2]].any()
    f, b = orc.gather_dequantize(t, ids, want_bf16=True)
    assert np.array_equal(f, g)
    assert np.array_equal(b, orc.dequantize(t, want_bf16=True)[1][ids])


# Planted scale bytes for the audit (page "Qwen3.8-Flash-Next-NVFP4", section
# 证据链: every scale must be finite and positive).  E4M3FN has one NaN
# pattern per sign (0x7F, 0xFF) and no infinities; zero is 0x00 or 0x80 and
# a set sign bit makes a scale negative.  Counts written out by hand:
AUDIT_PLANT = {0x7F: 3, 0xFF: 2, 0x00: 4, 0x80: 5, 0xB8: 6, 0x7E: 7, 0x38: 9}
AUDIT_EXPECT = dict(total=36, nonfinite=3 + 2, nonpositive=2 + 4 + 5 + 6, at_max=7)


def audit_planted_scales():
    """A [3, 12]-byte scale array (36 blocks) holding the planted bytes in a
    fixed shuffled order; the codes are irrelevant to the audit."""
    vals = [b for b, n in AUDIT_PLANT.items() for _ in range(n)]
    assert len(vals) == 36
    order = np.random.default_rng(4).permutation(36)
    return np.asarray(vals, np.uint8)[order].reshape(3, 12)


def test_audit_counts_planted_bytes(orc):
    s = audit_planted_scales()
    t = orc.NVFP4(np.zeros((3, 96), np.uint8), s, 1.0)
    a = orc.audit_scales(t)
    assert a == AUDIT_EXPECT


def test_tile_scales_matches_the_index_rule(orc):
    """The tiled scale order against its defining index rule, byte by byte
    (plain loops, two matrices of 256 x 512): every byte lands where the rule
    puts it, so the permutation is one to one; a wrong stride, a transposed
    tile or a mixed-up matrix offset would misplace some byte."""
    rng = np.random.default_rng(11)
    B, R, C = 2, 256, 512
    s = rng.integers(0, 256, (B, R, C // 16), dtype=np.uint8)
    t = orc.tile_scales(s)
    assert t.shape == (B * R * C // 16,)
    want = np.zeros_like(t)
    hit = np.zeros(t.size, np.int32)
    for m in range(B):
        for r in range(R):
            for b in range(C // 16):
                o = m * R * (C // 16) + ((r // 128 * (C // 256) + b // 16) * 128 + r % 128) * 16 + b % 16
                want[o] = s[m, r, b]
                hit[o] += 1
    assert (hit == 1).all()
    np.testing.assert_array_equal(t, want)
    # a tile's first 2 KB run: the 16 bytes of 256 elements of rows 0..127
    np.testing.assert_array_equal(t[:2048].reshape(128, 16), s[0, :128, :16])
    with pytest.raises(orc.OracleError):
        orc.tile_scales(s[:, :200])
