"""GPU parity: MX-native W4A8 (MXFP8 activations x MXFP4 weights on the
scaled FP8 x FP4 MFMA) vs the oracle.

Page "DeepSeek-V4.1-Flash-NVFP4", section 二 (the reference FP8 x FP4 GEMM).
Bar: the activation encode bit-exact (codes and scale bytes); the GEMM
max|C - R| / max|R| <= 1e-3 for fp32 output (the scaled MFMA's internal sum
is not exact fp32: about 6e-5 relative per 64-element step), 1e-3 + 2^-8
for bf16 output; full-size shapes checked on sampled rows.
"""
import numpy as np
import pytest
import torch

import precision_moe_gemm_amd as nv
from precision_moe_gemm_amd import synth
from tests.gpu_util import BF16_HALF_ULP, GEMM_TOL, rel_err, step, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("R,K,outliers", [(7, 256, 0.0), (300, 1024, 0.02), (33, 7168, 0.001), (3, 32, 0.0), (5, 96, 0.1)])
def test_mxfp8_encode_matches_oracle(orc, R, K, outliers):
    x = synth.normal_bf16((R, K), 1.0, (830, R, K))
    if outliers:
        x = synth.with_outliers(x, outliers, 40.0, (831, R, K))
    step(f"mxfp8 encode {R}x{K}")
    q, e8 = nv.mxfp8_quantize(x.to(DEV))
    rq, re8 = orc.mxfp8_encode(synth.bits(x))
    np.testing.assert_array_equal(u8(e8), re8)
    np.testing.assert_array_equal(u8(q), rq)


def test_mxfp8_encode_ranges_zero_blocks_strided(orc):
    rng = np.random.default_rng(832)
    v = rng.standard_normal((16, 384)).astype(np.float32) * np.exp2(rng.integers(-40, 40, (16, 1)))
    v[3, 32:64] = 0.0
    v[5, 64:96] = -0.0
    v[7, :32] = 448.0 * 2.0 ** 5
    base = torch.from_numpy(v).to(torch.bfloat16)
    wide = torch.zeros((16, 512), dtype=torch.bfloat16)
    wide[:, 64:448] = base
    x = wide.to(DEV)[:, 64:448]
    step("mxfp8 encode ranges / zero blocks / strided rows")
    q, e8 = nv.mxfp8_quantize(x)
    rq, re8 = orc.mxfp8_encode(synth.bits(base))
    np.testing.assert_array_equal(u8(e8), re8)
    np.testing.assert_array_equal(u8(q), rq)


def _operands(M, N, K, seed):
    a = synth.normal_bf16((M, K), 1.0, (833, seed, M, K)).to(DEV)
    w = synth.normal_bf16((N, K), 0.02, (834, seed, N, K)).to(DEV)
    q, qe = nv.mxfp8_quantize(a)
    wp, we = nv.mxfp4_quantize(w)
    return q, qe, wp, we


@pytest.mark.parametrize("M,N,K", [(1, 256, 128), (5, 300, 256), (100, 520, 384), (129, 768, 512),
                                   (256, 256, 1024), (300, 264, 640), (517, 1280, 384)])
def test_mx_w4a8_gemm_shapes(orc, M, N, K):
    q, qe, wp, we = _operands(M, N, K, 0)
    step(f"mx w4a8 gemm M={M} N={N} K={K}")
    C = nv.mx_gemm_w4a8(q, qe, wp, we).cpu().numpy()
    R = orc.mx_gemm_w4a8(u8(q), u8(qe), u8(wp), u8(we))
    err = rel_err(C, R)
    print(f"mx w4a8 rel err {err:.3e}")
    assert err <= GEMM_TOL
    Cb = nv.mx_gemm_w4a8(q, qe, wp, we, torch.bfloat16).float().cpu().numpy()
    assert rel_err(Cb, R) <= GEMM_TOL + BF16_HALF_ULP


@pytest.mark.parametrize("M,N,K", [(8192, 4096, 7168), (2048, 34816, 5120)])
def test_mx_w4a8_gemm_full_size_sampled(orc, M, N, K):
    q, qe, wp, we = _operands(M, N, K, 1)
    step(f"mx w4a8 gemm full size M={M} N={N} K={K}")
    C = nv.mx_gemm_w4a8(q, qe, wp, we)
    rng = np.random.default_rng(835)
    rows = np.unique(np.r_[rng.choice(M, 6, replace=False), 0, M - 1])
    cols = np.unique(np.r_[rng.choice(N, 48, replace=False), 0, N - 1])
    R = orc.mx_gemm_w4a8(u8(q), u8(qe), u8(wp), u8(we), a_rows=rows, w_rows=cols)
    got = C.cpu().numpy()[np.ix_(rows, cols)]
    assert rel_err(got, R) <= GEMM_TOL
    assert torch.equal(C, nv.mx_gemm_w4a8(q, qe, wp, we))


def test_mx_w4a8_unsupported_k():
    q, qe, wp, we = _operands(4, 64, 96, 2)
    with pytest.raises(nv.NVFP4Error) as ei:
        nv.mx_gemm_w4a8(q, qe, wp, we)
    assert ei.value.status == nv._lib.UNSUPPORTED
