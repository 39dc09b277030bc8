"""GPU parity: the MX-native W4A8 routed-expert layer (MXFP4 experts, MXFP8
activations on the scaled FP8 x FP4 MFMA) vs the oracle, staged:

  1. x -> MXFP8 bit-exact; route bit-exact;
  2. h (gate_up + SwiGLU) vs the oracle on the same MXFP8 x,
     max|h - R| / max|R| <= 1e-3 + 2^-8 (bf16), and its max word exact;
  3. the MXFP8 encode of the GPU's h bit-exact;
  4. y (down) vs the oracle on that MXFP8 h, <= 1e-3;
  5. out (combine) vs the oracle's combine of the oracle y, <= 1e-3 + 2^-8;
  6. the fused entry point equals the staged one bit for bit.

Pages "DeepSeek-V4.1-Flash-NVFP4" (section 二) and "Qwen3.8-Flash-Next-NVFP4"
(section 核心).
"""
import numpy as np
import pytest
import torch

import precision_moe_gemm_amd as nv
from precision_moe_gemm_amd import synth, workloads
from tests.gpu_util import BF16_HALF_ULP, GEMM_TOL, bf16_to_f64, rel_err, step, tensor_bf16_to_f64, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _mx_experts(cfg, which):
    packed, e8 = [], []
    for e in range(cfg.E):
        wb = cfg.w13(e, DEV) if which == "w13" else cfg.w2(e, DEV)
        p, s = nv.mxfp4_quantize(wb)
        packed.append(p)
        e8.append(s)
    return torch.stack(packed).contiguous(), torch.stack(e8).contiguous()


def _check_mx_moe(orc, cfg, sample_rows=None, sample_tokens=None, seed=0, ids=None, experts=None):
    step(f"mx moe build E={cfg.E} k={cfg.k} H={cfg.H} I={cfg.I} T={cfg.T}")
    if experts is None:
        w13p, w13e = _mx_experts(cfg, "w13")
        w2p, w2e = _mx_experts(cfg, "w2")
    else:
        w13p, w13e, w2p, w2e = experts
    x = cfg.x(DEV)
    rids, w = workloads.routing(cfg, DEV)
    ids = rids if ids is None else ids.to(DEV)
    T, k, E, H, I = cfg.T, cfg.k, cfg.E, cfg.H, cfg.I
    step("mx moe staged run")
    xq, xe = nv.mxfp8_quantize(x)
    perm, offsets, inv = nv.nvfp4_moe_route(ids, E)
    h, hmax = nv.mx_moe_gate_up(xq, xe, perm, offsets, k, w13p, w13e)
    hq, he = nv.mxfp8_quantize(h)
    y = nv.mx_moe_down(hq, he, offsets, T, k, w2p, w2e)
    out = nv.nvfp4_moe_combine(y, inv, w)
    torch.cuda.synchronize()
    # 1. x encode and route
    rq, re8 = orc.mxfp8_encode(synth.bits(x))
    np.testing.assert_array_equal(u8(xq), rq)
    np.testing.assert_array_equal(u8(xe), re8)
    ids_np, w_np = ids.cpu().numpy(), w.cpu().numpy()
    operm, ooff, oinv = orc.moe_route(ids_np, E)
    np.testing.assert_array_equal(perm.cpu().numpy(), operm)
    np.testing.assert_array_equal(offsets.cpu().numpy(), ooff)
    np.testing.assert_array_equal(inv.cpu().numpy(), oinv)
    rng = np.random.default_rng(seed)
    npairs = T * k
    rows = np.arange(npairs) if sample_rows is None else np.unique(
        np.r_[rng.choice(npairs, sample_rows, replace=False), 0, npairs - 1])
    w13p_np, w13e_np = u8(w13p), u8(w13e)
    w2p_np, w2e_np = u8(w2p), u8(w2e)
    # 2. h
    h_ref = orc.mx_moe_gate_up(rq, re8, operm, ooff, k, w13p_np, w13e_np, rows)
    h_bits = synth.bits(h.cpu())
    err_h = rel_err(bf16_to_f64(h_bits[rows]), bf16_to_f64(h_ref))
    print(f"mx h rel err {err_h:.3e}")
    assert err_h <= GEMM_TOL + BF16_HALF_ULP
    amax_h = np.abs(bf16_to_f64(h_bits)).max()
    assert np.uint32(hmax.item()) == np.float32(amax_h).view(np.uint32)
    # 3. h encode
    hq_ref, he_ref = orc.mxfp8_encode(h_bits)
    np.testing.assert_array_equal(u8(hq), hq_ref)
    np.testing.assert_array_equal(u8(he), he_ref)
    # 4. y from the GPU's MXFP8 h
    y_ref = orc.mx_moe_down(hq_ref, he_ref, ooff, w2p_np, w2e_np, rows)
    err_y = rel_err(y.cpu().numpy()[rows], y_ref)
    print(f"mx y rel err {err_y:.3e}")
    assert err_y <= GEMM_TOL
    # 5. combine on sampled tokens (all k slots of each)
    toks = np.arange(T) if sample_tokens is None else np.unique(
        np.r_[rng.choice(T, sample_tokens, replace=False), T - 1])
    slot_rows = oinv.reshape(T, k)[toks].ravel()
    y_full = np.zeros((npairs, H))
    y_full[slot_rows] = orc.mx_moe_down(hq_ref, he_ref, ooff, w2p_np, w2e_np, slot_rows)
    out_ref = orc.moe_combine(y_full, oinv, w_np)[toks]
    err_o = rel_err(tensor_bf16_to_f64(out)[toks], bf16_to_f64(out_ref))
    print(f"mx out rel err {err_o:.3e}")
    assert err_o <= GEMM_TOL + BF16_HALF_ULP
    # 6. fused == staged
    step("mx moe fused run")
    fused = nv.mx_moe_w4a8(x, ids, w, w13p, w13e, w2p, w2e)
    torch.cuda.synchronize()
    assert torch.equal(fused, out)
    assert nv.nvfp4_get_error() == 0


def test_mx_moe_small_every_row(orc):
    """Few rows per expert: 64-row and 128-row tiles, every row checked."""
    _check_mx_moe(orc, synth.MoE(seed=50, E=8, k=2, H=256, I=128, T=77))


def test_mx_moe_all_tile_classes_sampled(orc):
    """About 175 rows per expert: 256-row tiles with 128- and 64-row
    remainders; sampled rows and tokens."""
    _check_mx_moe(orc, synth.MoE(seed=51, E=12, k=3, H=512, I=256, T=700), sample_rows=300, sample_tokens=48)


def test_mx_moe_decode_batch(orc):
    """A decode-sized batch over many experts: every row in 32-row
    weight-streaming tiles (mx_stream_kernel)."""
    _check_mx_moe(orc, synth.MoE(seed=52, E=64, k=8, H=512, I=256, T=16))


@pytest.mark.parametrize("cfg", [
    synth.MoE(seed=54, E=16, k=4, H=2048, I=512, T=48, zipf=1.1),  # 8 / 2 stages, experts of 1-45 rows
    synth.MoE(seed=55, E=8, k=2, H=512, I=256, T=1),               # one token
    synth.MoE(seed=57, E=8, k=2, H=1024, I=1024, T=40),            # K % 1024 == 0 in both projections
], ids=["skewed-many-stages", "one-token", "four-stage-scale-chunks"])
def test_mx_moe_streaming_every_row(orc, cfg):
    """The streaming class with several 256-element stages per item (the
    register pipeline crosses items), experts holding more than one 32-row
    tile, a single token, and K a multiple of 1024 in both projections (the
    scale bytes of four stages per request); every row checked."""
    _check_mx_moe(orc, cfg)


def test_mx_moe_streaming_repeated_ids(orc):
    """All 120 pairs to one expert with I = 256: four 32-row streaming tiles
    of one expert, every row checked."""
    cfg = synth.MoE(seed=56, E=4, k=3, H=256, I=256, T=40)
    ids = torch.full((cfg.T, cfg.k), 1, dtype=torch.int32)
    _check_mx_moe(orc, cfg, ids=ids)


def test_mx_moe_decode_full_size_sampled(orc):
    """The 384-expert top-8 decode batch (T = 64) at its real shapes, H = 7168
    and I = 2048 (page "DeepSeek-V4.1-Flash-NVFP4", sections 一 and 二: the
    routed experts as stored in MXFP4), as the bench times it: every row in
    32-row streaming tiles, both K multiples of 1024 (scale bytes of four
    stages per request); sampled rows and tokens."""
    cfg = synth.C4_DECODE
    W = workloads.build_moe_weights(cfg, DEV, keep_mx=True)
    experts = (W.mx13[0], W.mx13[1], W.mx2[0], W.mx2[1])
    del W.w13, W.w2
    _check_mx_moe(orc, cfg, sample_rows=48, sample_tokens=6, experts=experts)


def test_mx_moe_repeated_ids_decode_batch(orc):
    """A small batch whose pairs all go to one expert (ids repeated within a
    token): 120 rows of one expert in 64-row tiles (I = 128 is not a whole
    streaming stage), every row checked."""
    cfg = synth.MoE(seed=53, E=4, k=3, H=256, I=128, T=40)
    ids = torch.full((cfg.T, cfg.k), 2, dtype=torch.int32)
    _check_mx_moe(orc, cfg, ids=ids)


def test_mx_moe_unsupported_shapes():
    x = torch.zeros((4, 384), dtype=torch.bfloat16, device=DEV)
    ids = torch.zeros((4, 1), dtype=torch.int32, device=DEV)
    w = torch.ones((4, 1), dtype=torch.float32, device=DEV)
    w13 = torch.zeros((1, 256, 192), dtype=torch.uint8, device=DEV)
    w13e = torch.zeros((1, 256, 12), dtype=torch.uint8, device=DEV)
    w2 = torch.zeros((1, 384, 64), dtype=torch.uint8, device=DEV)
    w2e = torch.zeros((1, 384, 4), dtype=torch.uint8, device=DEV)
    with pytest.raises(nv.NVFP4Error) as ei:  # H % 256 != 0
        nv.mx_moe_w4a8(x, ids, w, w13, w13e, w2, w2e)
    assert ei.value.status == 6


def test_mx_moe_empty_deterministic_and_bad_ids():
    """No tokens gives an empty output; two calls give the same bytes; an
    expert id outside [0, E) raises the range error and its pair is dropped
    (the output stays finite)."""
    cfg = synth.MoE(seed=58, E=4, k=2, H=512, I=256, T=24)
    w13p, w13e = _mx_experts(cfg, "w13")
    w2p, w2e = _mx_experts(cfg, "w2")
    x = cfg.x(DEV)
    ids, w = workloads.routing(cfg, DEV)
    step("mx moe empty / deterministic / bad ids")
    a = nv.mx_moe_w4a8(x, ids, w, w13p, w13e, w2p, w2e)
    b = nv.mx_moe_w4a8(x, ids, w, w13p, w13e, w2p, w2e)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    e = nv.mx_moe_w4a8(x[:0], ids[:0], w[:0], w13p, w13e, w2p, w2e)
    assert e.shape == (0, cfg.H)
    assert nv.nvfp4_get_error() == 0
    bad = ids.clone()
    bad[2, 1] = cfg.E
    bad[7, 0] = -3
    c = nv.mx_moe_w4a8(x, bad, w, w13p, w13e, w2p, w2e)
    torch.cuda.synchronize()
    assert nv.nvfp4_get_error() == 3
    assert torch.isfinite(c.float()).all()
    assert nv.nvfp4_get_error() == 0
