"""Pins of the oracle's MX-native W4A8 routed-expert projections (CPU only).

Pages "DeepSeek-V4.1-Flash-NVFP4" (section 二: MXFP4 expert weights, FP8
activations with block scales) and "Qwen3.8-Flash-Next-NVFP4" (section 核心:
the routed-expert layer).  The MX projections are checked against the NVFP4
ones, an independent code path: the MXFP4 experts are remapped losslessly to
NVFP4, and the activations are chosen so that MXFP8 and NVFP4 both represent
them exactly (E2M1 grid values with a +-6 in every 16-element block: block
scale 256 at the static global 2^-8 for NVFP4, scale 2^-6 for MXFP8).  The two
layers then multiply the same real numbers, so h and y must agree bit for
bit; a planted mistake in either (a wrong expert, row, scale or SwiGLU
operand) breaks the equality.
"""
import numpy as np
import pytest

import oracle as orc

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
G_EXACT = 2.0 ** -8  # static NVFP4 global: a +-6 block takes scale 256, codes = values


def _bf16_bits(x):
    return (np.ascontiguousarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _grid_rows(rng, R, K):
    """bf16 rows of E2M1 grid values, every 16-element block holding a +-6."""
    x = rng.choice(GRID, (R, K)) * rng.choice([-1.0, 1.0], (R, K))
    x[:, ::16] = 6.0 * rng.choice([-1.0, 1.0], (R, K // 16))
    return _bf16_bits(x)


def _experts(rng, E, R, K):
    """MXFP4 experts from random bf16 weights, and their NVFP4 remaps."""
    packed, e8, nv = [], [], []
    for _ in range(E):
        w = _bf16_bits(rng.standard_normal((R, K)) * rng.choice([0.02, 0.3]))
        p, s = orc.mxfp4_encode(w)
        packed.append(p)
        e8.append(s)
        nv.append(orc.mxfp4_to_nvfp4(p, s))
    return np.stack(packed), np.stack(e8), orc.Experts.stack(nv)


def test_exact_activations_encode_identically():
    rng = np.random.default_rng(5)
    x = _grid_rows(rng, 7, 256)
    xv = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    q = orc.quantize(x, G_EXACT)
    assert (q.scales == orc.e4m3_encode(256.0)).all()
    np.testing.assert_array_equal(orc.dequantize(q), xv)
    xq, xe = orc.mxfp8_encode(x)
    assert (xe == 127 - 6).all()
    vals = np.array([orc.e4m3_value(int(b)) for b in xq.ravel()]).reshape(xq.shape)
    np.testing.assert_array_equal(vals * 2.0 ** -6, xv)


@pytest.mark.parametrize("E,k,T,H,I", [(3, 2, 9, 256, 128), (5, 3, 6, 512, 256)])
def test_mx_gate_up_and_down_equal_nvfp4_on_exact_operands(E, k, T, H, I):
    rng = np.random.default_rng(E * 100 + T)
    w13p, w13e, w13nv = _experts(rng, E, 2 * I, H)
    w2p, w2e, w2nv = _experts(rng, E, H, I)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    perm, offsets, inv = orc.moe_route(ids, E)
    rows = np.arange(T * k)
    x = _grid_rows(rng, T, H)
    xq, xe = orc.mxfp8_encode(x)
    h_mx = orc.mx_moe_gate_up(xq, xe, perm, offsets, k, w13p, w13e, rows)
    h_nv = orc.moe_gate_up(orc.quantize(x, G_EXACT), perm, offsets, k, w13nv, rows)
    np.testing.assert_array_equal(h_mx, h_nv)
    assert np.any(h_mx != 0)
    # down on exactly representable h rows (list order)
    hx = _grid_rows(rng, T * k, I)
    hq, he = orc.mxfp8_encode(hx)
    y_mx = orc.mx_moe_down(hq, he, offsets, w2p, w2e, rows)
    y_nv = orc.moe_down(orc.quantize(hx, G_EXACT), offsets, w2nv, rows)
    np.testing.assert_array_equal(y_mx, y_nv)


def test_row_subsets_and_expert_of_each_row():
    """Listed rows give the same values as the full list, and a row's value
    uses its own expert: swapping two experts' weights changes exactly the
    rows routed to them."""
    rng = np.random.default_rng(11)
    E, k, T, H, I = 4, 2, 8, 256, 128
    w13p, w13e, _ = _experts(rng, E, 2 * I, H)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    perm, offsets, _ = orc.moe_route(ids, E)
    xq, xe = orc.mxfp8_encode(_bf16_bits(rng.standard_normal((T, H))))
    full = orc.mx_moe_gate_up(xq, xe, perm, offsets, k, w13p, w13e, np.arange(T * k))
    sub = np.array([T * k - 1, 0, 5])
    np.testing.assert_array_equal(orc.mx_moe_gate_up(xq, xe, perm, offsets, k, w13p, w13e, sub), full[sub])
    sw_p, sw_e = w13p.copy(), w13e.copy()
    sw_p[[0, 1]], sw_e[[0, 1]] = w13p[[1, 0]], w13e[[1, 0]]
    swapped = orc.mx_moe_gate_up(xq, xe, perm, offsets, k, sw_p, sw_e, np.arange(T * k))
    moved = np.zeros(T * k, bool)
    moved[offsets[0]:offsets[2]] = True
    assert (np.any(swapped != full, axis=1) == moved).all()
