"""Pins of the oracle's MoE routed-expert path and NVFP4 KV cache (CPU only).

MoE: the permutation equals numpy's stable argsort; SwiGLU and the two
projections agree with a brute-force token-by-token float64 evaluation
(numpy matmuls of exactly dequantized operands, torch's silu), which walks
tokens in their own order rather than expert by expert; the combine is
checked with one-hot router weights; E=1, k=1, w=1 reduces to the dense MLP.
KV: writing 2048-token chunks at their offsets gives the same bytes as
quantizing the whole tensor with the same static global, and the cache costs
4.5/16 of bf16 (page "Qwen3.8-2.4T-A95B-NVFP4": about a quarter).
"""
import os

import numpy as np
import pytest
import torch

from precision_moe_gemm_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _mags():
    return np.array([float(l) for l in open(os.path.join(GOLDEN, "e2m1_magnitudes.txt"))
                     if l.strip() and not l.startswith("#")])


def _exact_values(t):
    mags = _mags()
    nib = np.stack([t.packed & 15, t.packed >> 4], -1).reshape(t.packed.shape[0], -1)
    v = np.where(nib & 8, -1.0, 1.0) * mags[nib & 7]
    s = torch.from_numpy(np.ascontiguousarray(t.scales)).view(torch.float8_e4m3fn).double().numpy()
    return v * np.repeat(s, 16, axis=1)


def _bf16_to_f64(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _tiny_moe(orc, T=6, E=4, k=2, H=64, I=32, seed=98):
    m = synth.MoE(seed=seed, E=E, k=k, H=H, I=I, T=T)
    x = synth.bits(m.x())
    ids, w = m.routing()
    ids, w = ids.numpy(), w.numpy()
    w13 = orc.Experts.stack([orc.quantize(synth.bits(m.w13(e))) for e in range(E)])
    w2 = orc.Experts.stack([orc.quantize(synth.bits(m.w2(e))) for e in range(E)])
    return m, x, ids, w, w13, w2


def test_route_is_stable_sort(orc):
    rng = np.random.default_rng(5)
    ids = rng.integers(0, 9, (37, 3)).astype(np.int32)
    perm, offsets, inv = orc.moe_route(ids, 9)
    ref = np.argsort(ids.ravel(), kind="stable")
    assert np.array_equal(perm, ref)
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(ids.ravel(), minlength=9))]))
    assert np.array_equal(perm[inv], np.arange(ids.size))
    bad = ids.copy()
    bad[3, 1] = 9
    with pytest.raises(orc.OracleError):
        orc.moe_route(bad, 9)


def test_moe_matches_token_order_bruteforce(orc):
    m, x, ids, w, w13, w2 = _tiny_moe(orc)
    T, k = ids.shape
    I = m.I
    res = orc.moe_forward(x, ids, w, w13, w2)
    xq = res["xq"]
    xv = _exact_values(xq) * float(xq.G)
    # gate_up + SwiGLU per (token, slot), in token order
    h_bf = np.zeros((T * k, I), np.uint16)
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            W = w13.expert(e)
            gu = xv[t] @ (_exact_values(W) * float(W.G)).T
            g, u = torch.from_numpy(gu[:I]), torch.from_numpy(gu[I:])
            h = (torch.nn.functional.silu(g) * u).numpy()
            q = res["inv"][t * k + j]
            got = _bf16_to_f64(res["h"][q])
            np.testing.assert_allclose(got, h, rtol=2 ** -8, atol=1e-30)
            h_bf[t * k + j] = res["h"][q]
    # down + combine from the oracle's hq, again in token order
    hq = res["hq"]
    hv = _exact_values(hq) * float(hq.G)
    out = np.zeros((T, m.H))
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            q = res["inv"][t * k + j]
            W = w2.expert(e)
            y = hv[q] @ (_exact_values(W) * float(W.G)).T
            np.testing.assert_allclose(res["y"][q], y, rtol=1e-12, atol=1e-12 * np.abs(y).max())
            out[t] += w[t, j] * y
    got = _bf16_to_f64(res["out"])
    np.testing.assert_allclose(got, out, rtol=2 ** -8, atol=1e-30)
    # h is quantized with one dynamic global over all T*k rows
    assert hq.G == np.float32(np.abs(_bf16_to_f64(res["h"])).max()) / np.float32(2688)


def test_h_quantization_is_row_order_free(orc):
    """Quantizing h in token order and in expert order gives the same rows."""
    m, x, ids, w, w13, w2 = _tiny_moe(orc, seed=99)
    res = orc.moe_forward(x, ids, w, w13, w2)
    h_tok = np.ascontiguousarray(res["h"][res["inv"]])
    q_tok = orc.quantize(h_tok)
    assert q_tok.G == res["hq"].G
    assert np.array_equal(q_tok.packed, res["hq"].packed[res["inv"]])


def test_combine_one_hot_selects_slot(orc):
    rng = np.random.default_rng(8)
    T, k, H = 5, 3, 16
    y = rng.standard_normal((T * k, H))
    inv = rng.permutation(T * k).astype(np.int32)
    w = np.zeros((T, k), np.float32)
    w[np.arange(T), [0, 2, 1, 1, 0]] = 1.0
    out = orc.moe_combine(y, inv, w)
    for t in range(T):
        j = int(np.argmax(w[t]))
        ref = torch.from_numpy(y[inv[t * k + j]]).float().to(torch.bfloat16)
        assert np.array_equal(out[t], ref.view(torch.int16).numpy().view(np.uint16))


def test_single_expert_moe_is_dense_mlp(orc):
    T, H, I = 5, 64, 48
    x = synth.bits(synth.normal_bf16((T, H), 1.0, (100, 0)))
    W13 = orc.quantize(synth.bits(synth.normal_bf16((2 * I, H), 0.02, (100, 1))))
    W2 = orc.quantize(synth.bits(synth.normal_bf16((H, I), 0.02, (100, 2))))
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    res = orc.moe_forward(x, ids, w, orc.Experts.stack([W13]), orc.Experts.stack([W2]))
    xq = orc.quantize(x)
    gu = orc.gemm(xq, W13)
    g, u = torch.from_numpy(gu[:, :I]), torch.from_numpy(gu[:, I:])
    h = (torch.nn.functional.silu(g) * u).numpy()
    hb = orc.bf16_round_array(h)
    assert np.array_equal(hb, res["h"])
    y = orc.gemm(orc.quantize(hb), W2)
    assert np.array_equal(orc.bf16_round_array(y), res["out"])


def test_static_in_globals_equal_dynamic(orc):
    m, x, ids, w, w13, w2 = _tiny_moe(orc, seed=101)
    r1 = orc.moe_forward(x, ids, w, w13, w2)
    r2 = orc.moe_forward(x, ids, w, w13, w2, static_in_globals=(float(r1["xq"].G), float(r1["hq"].G)))
    assert np.array_equal(r1["out"], r2["out"])


# ---------------------------------------------------------------- KV cache

def test_kv_chunked_writes_equal_whole_tensor(orc):
    kv = synth.KVCache(tokens=96, chunk=32)
    k = kv.k()
    kb = synth.bits(k)
    G = float(orc.global_from_amax(orc.amax_bf16(kb.reshape(-1, kv.dim))))
    cache = orc.kv_empty(kv.tokens, kv.heads, kv.dim)
    for c0 in (64, 0, 32):  # any write order
        orc.kv_write(cache, kb[c0:c0 + kv.chunk], c0, G)
    whole = orc.quantize(np.ascontiguousarray(kb.reshape(-1, kv.dim)), static_G=G)
    assert np.array_equal(cache.packed, whole.packed)
    assert np.array_equal(cache.scales, whole.scales)
    assert orc.audit_scales(whole)["at_max"] >= 1


def test_kv_storage_about_a_quarter_of_bf16():
    rec = {}
    for l in open(os.path.join(GOLDEN, "nvfp4_recipe.txt")):
        if l.strip() and not l.startswith("#"):
            kk, v = l.split()
            rec[kk] = float(v)
    n = int(rec["kv_max_model_len"]) * int(rec["kv_heads"]) * int(rec["kv_head_dim"])
    nv_bytes = n // 2 + n // 16
    ratio = nv_bytes / (2 * n)
    assert ratio == 4.5 / 16
    assert abs(ratio - 0.25) < 0.04
