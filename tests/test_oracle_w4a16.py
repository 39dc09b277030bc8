"""Pins of the oracle's W4A16 path: bf16 activations x NVFP4 weights (CPU only).

Page "Qwen3.8-Flash-Next-FP4-Local", section 3.2: the MTP head's routed
experts keep BF16 activations and NVFP4 weights (W4A16).  The GEMM is checked
against an exact rational sum on a tiny case (E2M1 magnitudes from the golden
table, E4M3 scales and bf16 activations decoded by torch, Python fractions),
against the int64 W4A4 oracle when the activations are NVFP4 values exactly
representable in bf16, and with one-hot activation rows (orientation,
global).  The MoE composition is checked by brute force in token order
(float64 numpy matmuls of the exactly dequantized weights, torch's silu), by
its E=1, k=1 reduction to the dense MLP and by duplicated slots.
"""
import os
from fractions import Fraction

import numpy as np
import torch

from precision_moe_gemm_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _mags():
    return np.array([float(l) for l in open(os.path.join(GOLDEN, "e2m1_magnitudes.txt"))
                     if l.strip() and not l.startswith("#")])


def _exact_values(t):
    """float64 q * s of every element (no global): exact."""
    mags = _mags()
    nib = np.stack([t.packed & 15, t.packed >> 4], -1).reshape(t.packed.shape[0], -1)
    v = np.where(nib & 8, -1.0, 1.0) * mags[nib & 7]
    s = torch.from_numpy(np.ascontiguousarray(t.scales)).view(torch.float8_e4m3fn).double().numpy()
    return v * np.repeat(s, 16, axis=1)


def _bf16_to_f64(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_w4a16_gemm_exact_rational_sum(orc):
    a = synth.bits(synth.normal_bf16((3, 48), 1.0, (110, 0)))
    W = orc.quantize(synth.bits(synth.normal_bf16((5, 48), 0.02, (110, 1))))
    C = orc.gemm_w4a16(a, W)
    av = _bf16_to_f64(a)
    wv = _exact_values(W)
    for i in range(3):
        for j in range(5):
            exact = sum(Fraction(av[i, k]) * Fraction(wv[j, k]) for k in range(48)) * Fraction(float(W.G))
            assert abs(Fraction(C[i, j]) - exact) <= abs(exact) * Fraction(1, 2 ** 50)


def test_w4a16_equals_w4a4_on_nvfp4_valued_activations(orc):
    """Activations that are NVFP4 values with a power-of-two global are exact
    in bf16, so the W4A16 product must equal the int64 W4A4 product."""
    x = synth.bits(synth.normal_bf16((7, 256), 1.0, (111, 0)))
    Aq = orc.quantize(x, static_G=2.0 ** -6)
    _, a_bits = orc.dequantize(Aq, want_bf16=True)
    assert np.array_equal(_bf16_to_f64(a_bits), _exact_values(Aq) * 2.0 ** -6)  # exact in bf16
    W = orc.quantize(synth.bits(synth.normal_bf16((9, 256), 0.02, (111, 1))))
    ref = orc.gemm(Aq, W)
    got = orc.gemm_w4a16(a_bits, W)
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-14 * np.abs(ref).max())


def test_w4a16_one_hot_rows_pick_dequantized_weights(orc):
    W = orc.quantize(synth.bits(synth.normal_bf16((6, 64), 0.02, (112, 0))))
    deq = _exact_values(W) * float(W.G)  # (q * s) * G in float64: exact
    cols = [0, 17, 63, 32]
    a = np.zeros((4, 64), np.uint16)
    for m, c in enumerate(cols):
        a[m, c] = 0x4000  # bf16 2.0
    C = orc.gemm_w4a16(a, W)
    for m, c in enumerate(cols):
        assert np.array_equal(C[m], 2.0 * deq[:, c])
    sub = orc.gemm_w4a16(a, W, a_rows=[3, 0], w_rows=[5, 1, 1])
    assert np.array_equal(sub, C[np.ix_([3, 0], [5, 1, 1])])


def _tiny(orc, seed, T=6, E=4, k=2, H=64, I=32):
    m = synth.MoE(seed=seed, E=E, k=k, H=H, I=I, T=T)
    x = synth.bits(m.x())
    ids, w = m.routing()
    w13 = orc.Experts.stack([orc.quantize(synth.bits(m.w13(e))) for e in range(E)])
    w2 = orc.Experts.stack([orc.quantize(synth.bits(m.w2(e))) for e in range(E)])
    return m, x, ids.numpy(), w.numpy(), w13, w2


def test_moe_w4a16_matches_token_order_bruteforce(orc):
    m, x, ids, w, w13, w2 = _tiny(orc, 113)
    T, k = ids.shape
    res = orc.moe_w4a16_forward(x, ids, w, w13, w2)
    xv = _bf16_to_f64(x)
    out = np.zeros((T, m.H))
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            q = res["inv"][t * k + j]
            W13 = w13.expert(e)
            gu = xv[t] @ (_exact_values(W13) * float(W13.G)).T
            g, u = torch.from_numpy(gu[:m.I]), torch.from_numpy(gu[m.I:])
            h = (torch.nn.functional.silu(g) * u).numpy()
            np.testing.assert_allclose(_bf16_to_f64(res["h"][q]), h, rtol=2 ** -8, atol=1e-30)
            W2 = w2.expert(e)
            y = _bf16_to_f64(res["h"][q]) @ (_exact_values(W2) * float(W2.G)).T
            np.testing.assert_allclose(res["y"][q], y, rtol=1e-12, atol=1e-12 * np.abs(y).max())
            out[t] += w[t, j] * y
    np.testing.assert_allclose(_bf16_to_f64(res["out"]), out, rtol=2 ** -8, atol=1e-30)


def test_single_expert_w4a16_moe_is_dense_mlp(orc):
    T, H, I = 5, 64, 48
    x = synth.bits(synth.normal_bf16((T, H), 1.0, (114, 0)))
    W13 = orc.quantize(synth.bits(synth.normal_bf16((2 * I, H), 0.02, (114, 1))))
    W2 = orc.quantize(synth.bits(synth.normal_bf16((H, I), 0.02, (114, 2))))
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    res = orc.moe_w4a16_forward(x, ids, w, orc.Experts.stack([W13]), orc.Experts.stack([W2]))
    gu = orc.gemm_w4a16(x, W13)
    g, u = torch.from_numpy(gu[:, :I]), torch.from_numpy(gu[:, I:])
    hb = orc.bf16_round_array((torch.nn.functional.silu(g) * u).numpy())
    assert np.array_equal(hb, res["h"])
    assert np.array_equal(orc.bf16_round_array(orc.gemm_w4a16(hb, W2)), res["out"])


def test_moe_w4a16_duplicate_slots_halve(orc):
    """Two slots on the same expert with weights 1/2 give the one-slot output."""
    m, x, ids, w, w13, w2 = _tiny(orc, 115, k=1)
    r1 = orc.moe_w4a16_forward(x, ids, np.ones_like(w), w13, w2)
    ids2 = np.repeat(ids, 2, axis=1)
    r2 = orc.moe_w4a16_forward(x, ids2, np.full(ids2.shape, 0.5, np.float32), w13, w2)
    assert np.array_equal(r1["out"], r2["out"])
