"""Pins of the oracle's scalar codecs (CPU only).

Each check compares the oracle with something other than itself: the pages'
printed values (tests/golden), torch's own float8_e4m3fn / bfloat16
conversions (library routines), or numpy's round-half-even on the E2M1 grid.
"""
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_values(name):
    vals = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            vals.append(line)
    return vals


def _recipe():
    d = {}
    for line in _golden_values("nvfp4_recipe.txt"):
        k, v = line.split()
        d[k] = float(v)
    return d


def test_e2m1_table_matches_page(orc):
    mags = [float(v) for v in _golden_values("e2m1_magnitudes.txt")]
    assert len(mags) == 8
    for c in range(16):
        want = mags[c & 7] * (-1.0 if c & 8 else 1.0)
        assert orc.e2m1_value(c) == want


def test_e4m3_values_match_torch(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double()
    for b in range(256):
        v = orc.e4m3_value(b)
        r = ref[b].item()
        if math.isnan(r):
            assert math.isnan(v), hex(b)
        else:
            assert v == r, hex(b)


def test_e4m3_audit_max_is_448(orc):
    rec = _recipe()
    assert orc.e4m3_value(0x7E) == rec["scale_audit_max"]
    # the printed audit minimum is below the smallest E4M3 value, so it must be
    # a per-tensor fp32 scale, not a block scale
    assert rec["scale_audit_min"] < orc.e4m3_value(0x01) == 2.0 ** -9
    finite = [orc.e4m3_value(b) for b in range(0x7F)]
    assert all(finite[i] < finite[i + 1] for i in range(len(finite) - 1))
    assert max(finite) == 448.0


def test_e4m3_encode_matches_torch_rne(orc):
    """Nearest-even E4M3 of random, midpoint and boundary values vs torch."""
    rng = np.random.default_rng(7)
    vals = list(np.exp(rng.uniform(np.log(1e-5), np.log(470.0), 4000)).astype(np.float32))
    vals += [0.0, 2.0 ** -10, 2.0 ** -9, 3 * 2.0 ** -11, 448.0, 460.0, 464.0, 479.0]
    table = [orc.e4m3_value(b) for b in range(0x7F)]
    for i in range(len(table) - 1):  # every midpoint and its float neighbours
        mid = np.float32((table[i] + table[i + 1]) / 2)
        vals += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))]
    # torch turns values past the 448/480 midpoint into NaN; the oracle
    # saturates them instead (checked below), so compare up to that midpoint
    vals = [v for v in vals if v <= 464.0]
    x = torch.tensor(np.array(vals, np.float32))
    ref = x.to(torch.float8_e4m3fn).view(torch.uint8)
    for v, r in zip(vals, ref.tolist()):
        assert orc.e4m3_encode(float(v)) == r, (v, r)


def test_e4m3_encode_saturates(orc):
    for v in [448.0, 464.5, 480.0, 1e4, 3.0e38, float("inf")]:
        assert orc.e4m3_encode(v) == 0x7E


def _e2m1_rne_numpy(a):
    """Round-half-even on the E2M1 grid: step 0.5 below 2, 1 below 4, 2 up to 6."""
    a = np.asarray(a, np.float64)
    step = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    v = np.round(a / step) * step          # numpy rounds half to even
    return np.minimum(v, 6.0)


def test_e2m1_encode_is_round_half_even(orc):
    mags = [float(v) for v in _golden_values("e2m1_magnitudes.txt")]
    rng = np.random.default_rng(11)
    vals = list(rng.uniform(0, 7, 5000).astype(np.float32))
    for i in range(7):  # midpoints and their neighbours
        m = np.float32((mags[i] + mags[i + 1]) / 2)
        vals += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(10))]
    vals += [0.0, 6.0, 6.5, 100.0, float("inf")]
    for v in vals:
        code = orc.e2m1_encode(float(v))
        assert mags[code] == _e2m1_rne_numpy(v), (v, code)


def test_e2m1_nan_gives_zero(orc):
    assert orc.e2m1_encode(float("nan")) == 0


def test_bf16_rounding_matches_torch(orc):
    rng = np.random.default_rng(3)
    f = (rng.standard_normal(3000) * np.exp(rng.uniform(-30, 30, 3000))).astype(np.float32)
    # exact bf16 midpoints: a bf16 pattern plus half an ulp
    base = rng.integers(0, 0x7F00, 1000).astype(np.uint32) << 16
    mids = (base | 0x8000).view(np.float32)
    vals = np.concatenate([f, mids, -mids, np.float32([3.3895314e38, 3.39e38])])
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for v, r in zip(vals, ref):
        assert orc.bf16_from_double(float(v)) == r, (v, hex(r))


def test_e8m0_values(orc):
    assert orc.e8m0_value(127) == 1.0
    assert orc.e8m0_value(0) == 2.0 ** -127
    assert orc.e8m0_value(254) == 2.0 ** 127
    assert math.isnan(orc.e8m0_value(255))
