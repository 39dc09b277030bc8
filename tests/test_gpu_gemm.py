"""GPU parity: dense W4A4 GEMM vs the exact (int64) oracle.

Bar: max|C - R| / max|R| <= 1e-3 (fp32 accumulation order) for fp32 output,
1e-3 + 2^-8 for bf16 output; bit-exact in the integer special case (all
scales 1, G = 1, where every partial sum is a small integer).
"""
import numpy as np
import pytest
import torch

import oracle
import precision_moe_gemm_amd as nv
from precision_moe_gemm_amd import synth
from tests.gpu_util import BF16_HALF_ULP, GEMM_TOL, assert_same_nvfp4, elem_rel_err, rel_err, step, to_oracle, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _q(t):
    return nv.nvfp4_quantize(t.to(DEV) if not t.is_cuda else t)


def test_tiny_linear(orc):
    x, w = synth.C1.x(), synth.C1.w()
    step("gemm tiny linear 16x256x512")
    A, W = _q(x), _q(w)
    Ao, Wo = orc.quantize(synth.bits(x)), orc.quantize(synth.bits(w))
    assert_same_nvfp4(A, Ao)
    assert_same_nvfp4(W, Wo)
    C = nv.nvfp4_gemm(A, W).cpu().numpy()
    R = orc.gemm(Ao, Wo)
    err = rel_err(C, R)
    print(f"tiny linear rel err {err:.3e}")
    assert err <= GEMM_TOL
    Cb = nv.nvfp4_gemm(A, W, torch.bfloat16).float().cpu().numpy()
    assert rel_err(Cb, R) <= GEMM_TOL + BF16_HALF_ULP


@pytest.mark.parametrize("M,N,K", [(1, 256, 128), (5, 300, 256), (33, 512, 640), (100, 256, 1152),
                                   (129, 768, 512), (300, 256, 256), (517, 1280, 384)])
def test_random_shapes(orc, M, N, K):
    x = synth.normal_bf16((M, K), 1.0, (300, M, K))
    w = synth.normal_bf16((N, K), 0.02, (301, N, K))
    step(f"gemm random M={M} N={N} K={K}")
    A, W = _q(x), _q(w)
    C = nv.nvfp4_gemm(A, W).cpu().numpy()
    R = orc.gemm(to_oracle(A), to_oracle(W))
    assert rel_err(C, R) <= GEMM_TOL


@pytest.mark.parametrize("M,N,K", [(1, 300, 256), (5, 256, 768), (17, 1000, 4096), (32, 520, 1024),
                                   (1, 5120, 17408), (32, 264, 2560), (2, 34816, 512)])
def test_weight_streaming_shapes(orc, M, N, K):
    """Few-row shapes (<= 32 rows, K % 256 == 0) take the weight-streaming
    kernel, with K split over workgroups when the tiles alone are few."""
    x = synth.normal_bf16((M, K), 1.0, (310, M, K))
    w = synth.normal_bf16((N, K), 0.02, (311, N, K))
    step(f"gemm weight streaming M={M} N={N} K={K}")
    A, W = _q(x), _q(w)
    C = nv.nvfp4_gemm(A, W)
    Cb = nv.nvfp4_gemm(A, W, torch.bfloat16)
    torch.cuda.synchronize()
    Ao, Wo = to_oracle(A), to_oracle(W)
    if N * K <= 1 << 22:
        R = orc.gemm(Ao, Wo)
        got, gotb = C.cpu().numpy(), Cb.float().cpu().numpy()
    else:
        cols = np.unique(np.r_[np.random.default_rng(N).choice(N, 64, replace=False), 0, N - 1])
        R = orc.gemm_rows(Ao, orc.NVFP4(u8(W.packed)[0][cols], u8(W.scales)[0][cols], W.global_.item()))
        got, gotb = C.cpu().numpy()[:, cols], Cb.float().cpu().numpy()[:, cols]
    err = rel_err(got, R)
    print(f"streaming M={M} N={N} K={K} rel err {err:.3e}")
    assert err <= GEMM_TOL
    assert rel_err(gotb, R) <= GEMM_TOL + BF16_HALF_ULP


@pytest.mark.parametrize("M,N,K", [(20, 128 * 500 + 64, 256), (32, 128 * 400 + 1, 512)])
def test_weight_streaming_many_items(orc, M, N, K):
    """More (A tile, W tile) items than the chip holds workgroups, so every
    workgroup walks several items and its load pipeline crosses item
    boundaries (one- and two-stage items, a ragged A tile and a ragged last
    W tile); every output element is checked."""
    x = synth.normal_bf16((M, K), 1.0, (312, M, K))
    w = synth.normal_bf16((N, K), 0.02, (313, N, K))
    step(f"gemm weight streaming, many items M={M} N={N} K={K}")
    A, W = _q(x), _q(w)
    C = nv.nvfp4_gemm(A, W)
    Cb = nv.nvfp4_gemm(A, W, torch.bfloat16)
    torch.cuda.synchronize()
    R = orc.gemm(to_oracle(A), to_oracle(W))
    err = rel_err(C.cpu().numpy(), R)
    print(f"streaming many items M={M} N={N} K={K} rel err {err:.3e}")
    assert err <= GEMM_TOL
    assert rel_err(Cb.float().cpu().numpy(), R) <= GEMM_TOL + BF16_HALF_ULP


def test_split_k_matches_unsplit_and_is_reproducible():
    M, N, K = 3, 1024, 8192
    A = _q(synth.normal_bf16((M, K), 1.0, (320, 0)))
    W = _q(synth.normal_bf16((N, K), 0.02, (321, 0)))
    nbytes = nv.nvfp4_workspace_size(2, M, 0, 0, K, N)
    assert nbytes > 0
    step("gemm split-K vs unsplit")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    a = nv.nvfp4_gemm(A, W, ws=ws)
    b = nv.nvfp4_gemm(A, W, ws=ws)
    c = nv.nvfp4_gemm(A, W, ws=torch.empty(0, dtype=torch.uint8, device=DEV))  # size 0: unsplit
    assert torch.equal(a, b)
    ref = c.double()
    assert ((a.double() - ref).abs().max() / ref.abs().max()).item() <= GEMM_TOL
    with pytest.raises(nv.NVFP4Error) as ei:
        nv.nvfp4_gemm(A, W, ws=ws[: nbytes // 2])
    assert ei.value.status == 4


def test_integer_special_case_is_exact(orc):
    rng = np.random.default_rng(4)
    M, N, K = 64, 512, 1024
    a = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    w = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    one = lambda r: np.full((r, K // 16), 0x38, np.uint8)
    A = nv.NVFP4Tensor(torch.from_numpy(a[None]).to(DEV), torch.from_numpy(one(M)[None]).to(DEV),
                       torch.ones(1, device=DEV), M, K)
    W = nv.NVFP4Tensor(torch.from_numpy(w[None]).to(DEV), torch.from_numpy(one(N)[None]).to(DEV),
                       torch.ones(1, device=DEV), N, K)
    step("gemm integer special case")
    C = nv.nvfp4_gemm(A, W).cpu().numpy().astype(np.float64)
    R = orc.gemm(orc.NVFP4(a, one(M), 1.0), orc.NVFP4(w, one(N), 1.0))
    np.testing.assert_array_equal(C, R)


@pytest.mark.parametrize("M", [1, 32, 8192])
def test_dense_mlp_gate_up_sampled(orc, M):
    """27B-class gate_up projection (34816 x 5120) at its real shape; the oracle
    computes sampled output rows and columns one by one."""
    c = synth.C2
    w = c.w13(DEV)
    W = nv.nvfp4_quantize(w)
    x = c.x(M, DEV)
    A = nv.nvfp4_quantize(x)
    step(f"gemm dense MLP gate_up M={M}")
    C = nv.nvfp4_gemm(A, W)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M)
    rows = np.unique(np.r_[rng.choice(M, min(M, 6), replace=False), M - 1])
    cols = np.unique(np.r_[rng.choice(w.shape[0], 96, replace=False), 0, w.shape[0] - 1])
    Ao = to_oracle(A)
    Wo = orc.NVFP4(u8(W.packed)[0][cols], u8(W.scales)[0][cols], W.global_.item())
    R = orc.gemm_rows(Ao, Wo, a_rows=rows)
    got = C.cpu().numpy()[np.ix_(rows, cols)]
    err = rel_err(got, R)
    print(f"dense MLP M={M} sampled rel err {err:.3e}")
    assert err <= GEMM_TOL
    del w, W, C


def test_k_not_multiple_of_16_is_a_shape_error():
    """The format blocks K by 16: other K are refused before any launch."""
    A = nv.NVFP4Tensor.empty(4, 72, 1, DEV)
    W = nv.NVFP4Tensor.empty(8, 72, 1, DEV)
    with pytest.raises(nv.NVFP4Error) as ei:
        nv.nvfp4_gemm(A, W)
    assert ei.value.status == 2


def test_gemm_deterministic():
    x, w = synth.C1.x(DEV), synth.C1.w(DEV)
    A, W = nv.nvfp4_quantize(x), nv.nvfp4_quantize(w)
    assert torch.equal(nv.nvfp4_gemm(A, W), nv.nvfp4_gemm(A, W))


@pytest.mark.parametrize("M,N,K", [(512, 256, 1024), (200, 256, 1024), (300, 256, 576), (16, 512, 1024)])
def test_pow2_weight_scales(orc, M, N, K):
    """A remapped MXFP4 weight (every block scale a power of two) flagged
    NVFP4_POW2_SCALES takes the conversion-folded scale path: the product
    must equal the general path's bit for bit, and the oracle within the
    GEMM bar.  Shapes cover the 256- and 128-row tiles (K with a partial
    last group) and the weight-streaming kernel."""
    step(f"gemm pow2 weight scales {M}x{N}x{K}")
    x = synth.normal_bf16((M, K), 1.0, (810, M, K))
    w = synth.normal_bf16((N, K), 0.02, (811, N, K))
    A = _q(x)
    p, e = nv.mxfp4_quantize(w.to(DEV))
    W = nv.mxfp4_to_nvfp4(p, e, N, K, 1)
    assert W.flags == nv._lib.POW2_SCALES
    Wg = nv.NVFP4Tensor(W.packed, W.scales, W.global_, N, K, 1, 0)
    C = nv.nvfp4_gemm(A, W)
    Cg = nv.nvfp4_gemm(A, Wg)
    assert torch.equal(C, Cg)
    Ao = orc.quantize(synth.bits(x))
    Wo = orc.mxfp4_to_nvfp4(*orc.mxfp4_encode(synth.bits(w)))
    err = rel_err(C.cpu().numpy(), orc.gemm(Ao, Wo))
    print(f"pow2 scales rel err {err:.3e}")
    assert err <= GEMM_TOL


@pytest.mark.parametrize("M", [40, 100, 300])
def test_down_projection_K17408(orc, M):
    """The 27B-class down projection (W 5120 x 17408; page "Qwen3.8-27B-NVFP4",
    section 2) at M = 40 (64-row register-decode tiles), 100 (a 128-row tile)
    and 300 (a 256-row tile and a partial one): every row of A against 256
    sampled columns, W's sampled rows bit-exact vs the oracle."""
    N, K = 5120, 17408
    x = synth.normal_bf16((M, K), 1.0, (320, M), DEV)
    w = synth.normal_bf16((N, K), 0.02, (321, N), DEV)
    step(f"gemm down projection M={M} N={N} K={K}")
    A, W = nv.nvfp4_quantize(x), nv.nvfp4_quantize(w)
    C = nv.nvfp4_gemm(A, W)
    torch.cuda.synchronize()
    Ao = orc.quantize(synth.bits(x))
    assert_same_nvfp4(A, Ao)
    cols = np.unique(np.r_[np.random.default_rng(M).choice(N, 254, replace=False), 0, N - 1])
    wb = synth.bits(w)
    Gw = orc.global_from_amax(orc.amax_bf16(wb))
    Wo = orc.quantize(np.ascontiguousarray(wb[cols]), static_G=Gw)
    assert np.float32(W.global_.item()) == np.float32(Gw)
    np.testing.assert_array_equal(u8(W.scales)[0][cols], Wo.scales)
    np.testing.assert_array_equal(u8(W.packed)[0][cols], Wo.packed)
    R = orc.gemm(Ao, Wo)
    got = C.cpu().numpy()[:, cols]
    err, eerr = rel_err(got, R), elem_rel_err(got, R)
    print(f"down projection M={M} rel err {err:.3e} (element-wise {eerr:.3e})")
    assert err <= GEMM_TOL
    assert eerr <= GEMM_TOL
