"""GPU parity of ragged shapes: K a multiple of 16 but not of 64 (the block
axis of the format is 16 elements along the last dimension, page
"Qwen3.8-Flash-Next-NVFP4", section 核心), and MoE layers whose hidden or
intermediate size is off the 64 / 128 grid of the tiled kernels.  These run
the register-decode kernel with block-by-block loads of the last partial
stage and masked columns; every output is compared with the exact oracle."""
import numpy as np
import pytest
import torch

import precision_moe_gemm_amd as nv
from precision_moe_gemm_amd import synth
from tests.gpu_util import BF16_HALF_ULP, GEMM_TOL, elem_rel_err, rel_err, step, to_oracle
from tests.moe_check import check_moe_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("M,N,K", [(1, 64, 16), (5, 300, 48), (16, 256, 80), (40, 300, 80), (100, 520, 272),
                                   (300, 264, 272), (33, 1000, 1040)])
def test_dense_ragged_k(orc, M, N, K):
    x = synth.normal_bf16((M, K), 1.0, (330, M, K), DEV)
    w = synth.normal_bf16((N, K), 0.02, (331, N, K), DEV)
    step(f"gemm ragged K M={M} N={N} K={K}")
    A, W = nv.nvfp4_quantize(x), nv.nvfp4_quantize(w)
    C = nv.nvfp4_gemm(A, W)
    Cb = nv.nvfp4_gemm(A, W, torch.bfloat16)
    torch.cuda.synchronize()
    R = orc.gemm(to_oracle(A), to_oracle(W))
    got = C.cpu().numpy()
    err, eerr = rel_err(got, R), elem_rel_err(got, R)
    print(f"ragged K={K} M={M} N={N} rel err {err:.3e} (element-wise {eerr:.3e})")
    assert err <= GEMM_TOL and eerr <= GEMM_TOL
    assert rel_err(Cb.float().cpu().numpy(), R) <= GEMM_TOL + BF16_HALF_ULP


def test_dense_ragged_k_integer_case(orc):
    """Every 16-element block holds a 6 and the global is 1, so every block
    scale is exactly 1 and the operands are plain E2M1 values: each row sum
    of K = 272 products is a multiple of 1/4 below 2^14, exact in fp32, so
    the kernel (ragged last stage included) must match the oracle bit for
    bit."""
    M, N, K = 7, 40, 272
    rng = np.random.default_rng(5)
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)

    def operand(R):
        v = mags[rng.integers(0, 8, (R, K))] * rng.choice([-1.0, 1.0], (R, K))
        v[:, ::16] = 6.0 * rng.choice([-1.0, 1.0], (R, K // 16))
        return torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).to(DEV)

    g = torch.ones(1, dtype=torch.float32, device=DEV)
    A = nv.nvfp4_quantize(operand(M), static_global=g)
    W = nv.nvfp4_quantize(operand(N), static_global=g)
    assert int(A.scales.min()) == int(A.scales.max()) == 0x38  # E4M3 1.0
    step("gemm ragged K integer case")
    C = nv.nvfp4_gemm(A, W).cpu().numpy().astype(np.float64)
    R = orc.gemm(to_oracle(A), to_oracle(W))
    np.testing.assert_array_equal(C, R)


@pytest.mark.parametrize("cfg", [
    synth.MoE(seed=60, E=4, k=2, H=272, I=80, T=50),        # H and I off the grid: every row ragged
    synth.MoE(seed=61, E=3, k=2, H=512, I=96, T=130),       # gate_up N = 96: masked columns; down K = 96
    synth.MoE(seed=62, E=5, k=3, H=336, I=128, T=90),       # gate_up K = 336 (ragged), down K = 128
], ids=["h272-i80", "h512-i96", "h336-i128"])
def test_moe_ragged_every_row(cfg):
    check_moe_rows(cfg, rows=None, sample_tokens=cfg.T, full_tokens=4)


def test_moe_rejects_h_not_multiple_of_16():
    W = nv.NVFP4Tensor.empty(2 * 32, 40, 2, DEV)
    W2 = nv.NVFP4Tensor.empty(40, 32, 2, DEV)
    x = torch.zeros((4, 40), dtype=torch.bfloat16, device=DEV)
    ids = torch.zeros((4, 1), dtype=torch.int32, device=DEV)
    wt = torch.ones((4, 1), dtype=torch.float32, device=DEV)
    with pytest.raises(nv.NVFP4Error):
        nv.nvfp4_moe_grouped_gemm(x, ids, wt, W, W2)
