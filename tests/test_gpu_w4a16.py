"""GPU parity: W4A16 (bf16 activations x NVFP4 weights) vs the oracle.

Page "Qwen3.8-Flash-Next-FP4-Local", section 3.2 (W4A16 NVFP4 MTP experts).
Bar: the dense GEMM max|C - R| / max|R| <= 1e-3 (fp32 accumulation order)
for fp32 output, 1e-3 + 2^-8 for bf16; the fused MoE layer's output within
1e-3 + 2^-8 of the oracle's (route, gate_up + SwiGLU, down and combine on the
same bytes, no activation quantized).  The power-of-two weight-scale path
equals the general path bit for bit; repeated calls are bit-identical.
"""
import numpy as np
import pytest
import torch

import precision_moe_gemm_amd as nv
from precision_moe_gemm_amd import synth, workloads
from tests.gpu_util import BF16_HALF_ULP, GEMM_TOL, rel_err, step, tensor_bf16_to_f64, to_oracle, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("M,N,K", [(1, 256, 256), (5, 300, 512), (16, 384, 1024), (17, 1000, 4096),
                                   (37, 640, 2048), (64, 256, 768), (1, 5120, 17408), (2, 34816, 512)])
def test_w4a16_gemm_shapes(orc, M, N, K):
    a = synth.normal_bf16((M, K), 1.0, (820, M, K)).to(DEV)
    w = synth.normal_bf16((N, K), 0.02, (821, N, K)).to(DEV)
    step(f"w4a16 gemm M={M} N={N} K={K}")
    W = nv.nvfp4_quantize(w)
    C = nv.nvfp4_gemm_w4a16(a, W).cpu().numpy()
    R = orc.gemm_w4a16(synth.bits(a.cpu()), to_oracle(W))
    err = rel_err(C, R)
    print(f"w4a16 rel err {err:.3e}")
    assert err <= GEMM_TOL
    Cb = nv.nvfp4_gemm_w4a16(a, W, torch.bfloat16).float().cpu().numpy()
    assert rel_err(Cb, R) <= GEMM_TOL + BF16_HALF_ULP


def test_w4a16_gemm_strided_rows(orc):
    M, N, K, lda = 9, 320, 512, 768
    base = synth.normal_bf16((M, lda), 1.0, (822, 0)).to(DEV)
    a = base[:, 128:128 + K]
    assert a.stride(0) == lda
    W = nv.nvfp4_quantize(synth.normal_bf16((N, K), 0.02, (822, 1)).to(DEV))
    step("w4a16 gemm strided A")
    C = nv.nvfp4_gemm_w4a16(a, W).cpu().numpy()
    R = orc.gemm_w4a16(synth.bits(a.contiguous().cpu()), to_oracle(W))
    assert rel_err(C, R) <= GEMM_TOL


@pytest.mark.parametrize("M,N,K", [(3, 512, 1024), (40, 256, 2048)])
def test_w4a16_pow2_weight_scales(orc, M, N, K):
    """Remapped MXFP4 weights (power-of-two block scales) flagged
    NVFP4_POW2_SCALES fold the scale into the fp4 -> bf16 conversion: the
    product must equal the general path's bit for bit."""
    a = synth.normal_bf16((M, K), 1.0, (823, M, K)).to(DEV)
    p, e = nv.mxfp4_quantize(synth.normal_bf16((N, K), 0.02, (824, N, K)).to(DEV))
    W = nv.mxfp4_to_nvfp4(p, e, N, K, 1)
    assert W.flags == nv._lib.POW2_SCALES
    Wg = nv.NVFP4Tensor(W.packed, W.scales, W.global_, N, K, 1, 0)
    step(f"w4a16 pow2 {M}x{N}x{K}")
    C = nv.nvfp4_gemm_w4a16(a, W)
    assert torch.equal(C, nv.nvfp4_gemm_w4a16(a, Wg))
    assert rel_err(C.cpu().numpy(), orc.gemm_w4a16(synth.bits(a.cpu()), to_oracle(W))) <= GEMM_TOL


def test_w4a16_gemm_unsupported_k():
    W = nv.nvfp4_quantize(synth.normal_bf16((64, 384), 0.02, (825, 0)).to(DEV))
    a = synth.normal_bf16((4, 384), 1.0, (825, 1)).to(DEV)
    with pytest.raises(nv.NVFP4Error) as ei:
        nv.nvfp4_gemm_w4a16(a, W)
    assert ei.value.status == nv._lib.UNSUPPORTED


def _oracle_experts(orc, W, experts, E, H, I):
    """Oracle operands of the listed experts (GPU bytes); others zero-filled
    and never read."""
    w13p = np.zeros((E, 2 * I, H // 2), np.uint8)
    w13s = np.zeros((E, 2 * I, H // 16), np.uint8)
    w13g = np.ones(E, np.float32)
    w2p = np.zeros((E, H, I // 2), np.uint8)
    w2s = np.zeros((E, H, I // 16), np.uint8)
    w2g = np.ones(E, np.float32)
    for e in experts:
        a = workloads.expert_view(W.w13, e)
        b = workloads.expert_view(W.w2, e)
        w13p[e], w13s[e], w13g[e] = u8(a.packed)[0], u8(a.scales)[0], a.global_.item()
        w2p[e], w2s[e], w2g[e] = u8(b.packed)[0], u8(b.scales)[0], b.global_.item()
    return orc.Experts(w13p, w13s, w13g), orc.Experts(w2p, w2s, w2g)


def _check_w4a16_moe(orc, cfg, sample_tokens=None, seed=0):
    step(f"w4a16 moe build E={cfg.E} k={cfg.k} H={cfg.H} I={cfg.I} T={cfg.T} mx={cfg.mx}")
    W = workloads.build_moe_weights(cfg, DEV)
    x = cfg.x(DEV)
    ids, w = workloads.routing(cfg, DEV)
    step("w4a16 moe fused run")
    out = nv.nvfp4_moe_w4a16(x, ids, w, W.w13, W.w2)
    again = nv.nvfp4_moe_w4a16(x, ids, w, W.w13, W.w2)
    torch.cuda.synchronize()
    assert torch.equal(out, again)
    assert nv.nvfp4_get_error() == 0
    T, k, E, H, I = cfg.T, cfg.k, cfg.E, cfg.H, cfg.I
    ids_np, w_np = ids.cpu().numpy(), w.cpu().numpy()
    perm, offsets, inv = orc.moe_route(ids_np, E)
    rng = np.random.default_rng(seed)
    toks = np.arange(T) if sample_tokens is None else np.unique(
        np.r_[rng.choice(T, sample_tokens, replace=False), T - 1])
    rows = inv.reshape(T, k)[toks].ravel()
    experts = sorted(set(int(np.searchsorted(offsets, q, side="right") - 1) for q in rows))
    ex13, ex2 = _oracle_experts(orc, W, experts, E, H, I)
    x_bits = synth.bits(x.cpu())
    h = np.zeros((T * k, I), np.uint16)
    h[rows] = orc.moe_w4a16_gate_up(x_bits, perm, offsets, k, ex13, rows)
    y = np.zeros((T * k, H))
    y[rows] = orc.moe_w4a16_down(h, offsets, ex2, rows)
    ref = orc.moe_combine(y, inv, w_np)[toks]
    err = rel_err(tensor_bf16_to_f64(out)[toks], (ref.astype(np.uint32) << 16).view(np.float32))
    print(f"w4a16 moe out rel err {err:.3e}")
    assert err <= GEMM_TOL + BF16_HALF_ULP
    return out, W, x, ids, w


def test_w4a16_moe_small_every_token(orc):
    _check_w4a16_moe(orc, synth.MoE(seed=40, E=6, k=2, H=512, I=256, T=9))


def test_w4a16_moe_k_split_paths(orc):
    """Two tokens on two experts: both projections split K over streaming
    workgroups (partial planes added in a fixed order)."""
    _check_w4a16_moe(orc, synth.MoE(seed=41, E=2, k=1, H=2048, I=2048, T=2))


def test_w4a16_moe_384_experts_decode_sampled(orc):
    """384 MXFP4-origin experts, top-8, H=7168, I=2048, T=64: power-of-two
    weight scales; the general path on the same bytes gives the same output."""
    out, W, x, ids, w = _check_w4a16_moe(orc, synth.C4_DECODE, sample_tokens=5)
    assert W.w13.flags == nv._lib.POW2_SCALES
    g13 = nv.NVFP4Tensor(W.w13.packed, W.w13.scales, W.w13.global_, W.w13.rows, W.w13.cols, W.w13.batch, 0)
    g2 = nv.NVFP4Tensor(W.w2.packed, W.w2.scales, W.w2.global_, W.w2.rows, W.w2.cols, W.w2.batch, 0)
    step("w4a16 moe general-scale path")
    assert torch.equal(nv.nvfp4_moe_w4a16(x, ids, w, g13, g2), out)


def test_w4a16_moe_empty_deterministic_and_bad_ids():
    """No tokens gives an empty output; two calls give the same bytes; an
    expert id outside [0, E) raises the range error and its pair is dropped
    (the output stays finite)."""
    cfg = synth.MoE(seed=59, E=4, k=2, H=512, I=256, T=24)
    W = workloads.build_moe_weights(cfg, DEV)
    x = cfg.x(DEV)
    ids, w = workloads.routing(cfg, DEV)
    step("w4a16 moe empty / deterministic / bad ids")
    a = nv.nvfp4_moe_w4a16(x, ids, w, W.w13, W.w2)
    b = nv.nvfp4_moe_w4a16(x, ids, w, W.w13, W.w2)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    e = nv.nvfp4_moe_w4a16(x[:0], ids[:0], w[:0], W.w13, W.w2)
    assert e.shape == (0, cfg.H)
    assert nv.nvfp4_get_error() == 0
    bad = ids.clone()
    bad[2, 1] = cfg.E
    bad[7, 0] = -3
    c = nv.nvfp4_moe_w4a16(x, bad, w, W.w13, W.w2)
    torch.cuda.synchronize()
    assert nv.nvfp4_get_error() == 3
    assert torch.isfinite(c.float()).all()
    assert nv.nvfp4_get_error() == 0
