"""GPU: weight scale bytes in the 128-row tiled storage order
(NVFP4_TILED_SCALES, written by nvfp4_tile_scales).

The order moves scale bytes and nothing else, so:
* nvfp4_tile_scales writes, byte for byte, the oracle's tile_scales of the
  row-major bytes;
* every GEMM path that takes a tiled weight gives results bit-identical to
  the same weight in row-major order: the weight-streaming kernel (16- and
  32-row tiles, K split, W4A16), the register-decode kernel (33-95 rows and
  the ragged gate_up), the 128- and 256-row tile kernels, and the grouped
  layer over every tile class with general and power-of-two scales.
The row-major results are compared with the oracle by test_gpu_gemm.py,
test_gpu_moe.py and test_gpu_moe_tiles.py, so the equality carries that
parity over to the tiled order.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_moe_gemm_amd as nv
from precision_moe_gemm_amd import _lib, synth, workloads
from tests.gpu_util import step, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _weights(B, R, C, seed, mx=False):
    t = nv.NVFP4Tensor.empty(R, C, B, DEV)
    if mx:
        ps, es = [], []
        for b in range(B):
            p, e = nv.mxfp4_quantize(synth.normal_bf16((R, C), 0.02, (seed, b), DEV))
            ps.append(p)
            es.append(e)
        return nv.mxfp4_to_nvfp4(torch.stack(ps), torch.stack(es), R, C, B)
    for b in range(B):
        nv.nvfp4_quantize(synth.normal_bf16((R, C), 0.02, (seed, b), DEV), out=workloads.expert_view(t, b))
    return t


@pytest.mark.parametrize("B,R,C", [(3, 384, 768), (1, 4096, 7168)])
def test_tile_scales_bytes_equal_oracle(B, R, C):
    step(f"tile scales {B} x {R} x {C}")
    t = _weights(B, R, C, 60)
    tt = nv.nvfp4_tile_scales(t)
    torch.cuda.synchronize()
    assert tt.flags == t.flags | _lib.TILED_SCALES
    assert tt.packed is t.packed and tt.global_ is t.global_
    np.testing.assert_array_equal(u8(tt.scales).ravel(), oracle.tile_scales(u8(t.scales)))


@pytest.mark.parametrize("mx", [False, True], ids=["general", "pow2"])
@pytest.mark.parametrize("M", [1, 16, 20, 32, 48, 80, 100, 200, 300])
def test_dense_gemm_tiled_equals_row_major(M, mx):
    """M picks the path: streaming tiles (<= 32 rows; K split when the tiles
    cannot fill the chip), the register-decode kernel (33-95), the 128-row
    (96-255) and 256-row (>= 256) tile kernels."""
    step(f"dense gemm tiled M={M} mx={mx}")
    N, K = 384, 1024
    W = _weights(1, N, K, 61, mx)
    Wt = nv.nvfp4_tile_scales(W)
    A = nv.nvfp4_quantize(synth.normal_bf16((M, K), 1.0, (62, M), DEV))
    for dtype in (torch.float32, torch.bfloat16):
        assert torch.equal(nv.nvfp4_gemm(A, Wt, dtype), nv.nvfp4_gemm(A, W, dtype))


def test_dense_gemm_k_split_and_w4a16_tiled():
    step("dense gemm tiled: K split, W4A16")
    N, K = 256, 8192
    W = _weights(1, N, K, 63)
    Wt = nv.nvfp4_tile_scales(W)
    x = synth.normal_bf16((4, K), 1.0, (64, 0), DEV)
    A = nv.nvfp4_quantize(x)
    assert torch.equal(nv.nvfp4_gemm(A, Wt), nv.nvfp4_gemm(A, W))
    assert torch.equal(nv.nvfp4_gemm_w4a16(x, Wt), nv.nvfp4_gemm_w4a16(x, W))


MOE_CASES = [
    synth.MoE(seed=50, E=8, k=2, H=1024, I=512, T=1200, zipf=1.1),             # 256/128-row tiles + streaming
    synth.MoE(seed=50, E=8, k=2, H=1024, I=512, T=1200, zipf=1.1, mx=True),
    synth.MoE(seed=38, E=64, k=8, H=256, I=2048, T=64),                        # decode: streaming tiles only
    synth.MoE(seed=37, E=2, k=1, H=2048, I=512, T=12),                         # K-split gate_up
]


@pytest.mark.parametrize("cfg", MOE_CASES, ids=["tiles-general", "tiles-pow2", "decode", "gate-split"])
def test_moe_tiled_equals_row_major(cfg):
    step(f"moe tiled E={cfg.E} H={cfg.H} I={cfg.I} T={cfg.T} mx={cfg.mx}")
    W = workloads.build_moe_weights(cfg, DEV)
    w13t, w2t = nv.nvfp4_tile_scales(W.w13), nv.nvfp4_tile_scales(W.w2)
    x = cfg.x(DEV)
    ids, w = workloads.routing(cfg, DEV)
    ref = nv.nvfp4_moe_grouped_gemm(x, ids, w, W.w13, W.w2)
    assert torch.equal(nv.nvfp4_moe_grouped_gemm(x, ids, w, w13t, w2t), ref)
    # staged entry points
    xq = nv.nvfp4_quantize(x)
    perm, offsets, _ = nv.nvfp4_moe_route(ids, cfg.E)
    h, hmax = nv.nvfp4_moe_gate_up(xq, perm, offsets, cfg.k, W.w13)
    ht, hmaxt = nv.nvfp4_moe_gate_up(xq, perm, offsets, cfg.k, w13t)
    assert torch.equal(ht, h) and torch.equal(hmaxt, hmax)
    hq = nv.nvfp4_quantize(h)
    assert torch.equal(nv.nvfp4_moe_down(hq, offsets, cfg.T, cfg.k, w2t), nv.nvfp4_moe_down(hq, offsets, cfg.T, cfg.k, W.w2))
    if not cfg.mx:
        assert torch.equal(nv.nvfp4_moe_w4a16(x, ids, w, w13t, w2t), nv.nvfp4_moe_w4a16(x, ids, w, W.w13, W.w2))
    assert nv.nvfp4_get_error() == 0


def test_moe_ragged_gate_up_with_tiled_w13():
    """I = 192: the gate_up projection's N is off the 128-column tile, so
    its rows run on the register-decode kernel; w13 (384 rows) can be tiled,
    w2 (I = 192 columns) cannot and stays row-major."""
    cfg = synth.MoE(seed=65, E=4, k=2, H=512, I=192, T=40)
    step("moe ragged gate_up, tiled w13")
    W = workloads.build_moe_weights(cfg, DEV)
    w13t = nv.nvfp4_tile_scales(W.w13)
    with pytest.raises(nv.NVFP4Error):
        nv.nvfp4_tile_scales(W.w2)
    x = cfg.x(DEV)
    ids, w = workloads.routing(cfg, DEV)
    assert torch.equal(nv.nvfp4_moe_grouped_gemm(x, ids, w, w13t, W.w2),
                       nv.nvfp4_moe_grouped_gemm(x, ids, w, W.w13, W.w2))


def test_tiled_tensor_refused_where_not_taken():
    step("tiled tensors refused outside weight operands")
    t = nv.nvfp4_tile_scales(_weights(1, 128, 256, 66))
    with pytest.raises(nv.NVFP4Error) as e:
        nv.nvfp4_dequantize(t)
    assert e.value.status == _lib.UNSUPPORTED
    with pytest.raises(nv.NVFP4Error) as e:
        nv.nvfp4_gemm(t, t)
    assert e.value.status == _lib.UNSUPPORTED
