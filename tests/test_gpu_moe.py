"""GPU parity: routed-expert MoE (route, gate_up + SwiGLU, h quantize, down,
combine) vs the oracle, following the staged protocol:

  1. x and every weight: GPU bytes bit-exact vs oracle Q (then the oracle uses
     its own, identical, quantized operands);
  2. route: perm / offsets / inv bit-exact;
  3. h: GPU gate_up output vs the oracle's h on the same quantized operands,
     max|h - R| / max|R| <= 1e-3 + 2^-8 (bf16 output);
  4. G_h == amax(h_gpu) / 2688 exactly, oracle Q(h_gpu) == GPU hq bit-exact;
  5. y: GPU down output vs the oracle on GPU hq, <= 1e-3;
  6. out: GPU combine vs the oracle's combine of the oracle y, <= 1e-3 + 2^-8;
  7. the fused entry point equals the staged one bit for bit.
End-to-end oracle error (h re-quantization amplifies fp32 order
differences) is printed, gated only loosely.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_moe_gemm_amd as nv
from precision_moe_gemm_amd import synth, workloads
from tests.gpu_util import (BF16_HALF_ULP, GEMM_TOL, bf16_to_f64, rel_err, step, tensor_bf16_to_f64,
                            to_oracle, u8)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _oracle_expert_checked(orc, W, cfg, e, which):
    """Oracle Q of expert e's bf16 weights, checked bit-exact against the GPU copy."""
    if which == "w13":
        src = synth.bits(cfg.w13(e, DEV))
        gt = workloads.expert_view(W.w13, e)
    else:
        src = synth.bits(cfg.w2(e, DEV))
        gt = workloads.expert_view(W.w2, e)
    if cfg.mx:
        ref = orc.mxfp4_to_nvfp4(*orc.mxfp4_encode(src))
    else:
        ref = orc.quantize(src)
    np.testing.assert_array_equal(u8(gt.scales)[0], ref.scales)
    np.testing.assert_array_equal(u8(gt.packed)[0], ref.packed)
    assert np.float32(gt.global_.item()) == ref.G
    return ref


def _run_staged(x, ids, w, W, cfg):
    T, k, E = cfg.T, cfg.k, cfg.E
    xq = nv.nvfp4_quantize(x)
    perm, offsets, inv = nv.nvfp4_moe_route(ids, E)
    h, hmax = nv.nvfp4_moe_gate_up(xq, perm, offsets, k, W.w13)
    hq = nv.nvfp4_quantize(h)
    y = nv.nvfp4_moe_down(hq, offsets, T, k, W.w2)
    out = nv.nvfp4_moe_combine(y, inv, w)
    torch.cuda.synchronize()
    return dict(xq=xq, perm=perm, offsets=offsets, inv=inv, h=h, hmax=hmax, hq=hq, y=y, out=out)


def _check_moe(orc, cfg, sample_rows=None, sample_tokens=None, seed=0, fused_exact=True):
    step(f"moe build E={cfg.E} k={cfg.k} H={cfg.H} I={cfg.I} T={cfg.T} mx={cfg.mx}")
    W = workloads.build_moe_weights(cfg, DEV)
    x = cfg.x(DEV)
    ids, w = workloads.routing(cfg, DEV)
    step("moe staged run")
    g = _run_staged(x, ids, w, W, cfg)
    T, k, E = cfg.T, cfg.k, cfg.E
    ids_np = ids.cpu().numpy()
    w_np = w.cpu().numpy()
    # 1. x bit-exact
    xo = orc.quantize(synth.bits(x))
    np.testing.assert_array_equal(u8(g["xq"].scales)[0], xo.scales)
    np.testing.assert_array_equal(u8(g["xq"].packed)[0], xo.packed)
    assert np.float32(g["xq"].global_.item()) == xo.G
    # 2. route bit-exact
    perm, offsets, inv = orc.moe_route(ids_np, E)
    np.testing.assert_array_equal(g["perm"].cpu().numpy(), perm)
    np.testing.assert_array_equal(g["offsets"].cpu().numpy(), offsets)
    np.testing.assert_array_equal(g["inv"].cpu().numpy(), inv)
    rng = np.random.default_rng(seed)
    npairs = T * k
    if sample_rows is None:
        rows = np.arange(npairs)
    else:
        rows = np.unique(np.r_[rng.choice(npairs, sample_rows, replace=False), 0, npairs - 1])
    experts_needed = sorted(set(int(np.searchsorted(offsets, q, side="right") - 1) for q in rows))
    # oracle expert operands (bit-exact vs GPU), others zero-filled (never read)
    H, I = cfg.H, cfg.I
    w13p = np.zeros((E, 2 * I, H // 2), np.uint8)
    w13s = np.zeros((E, 2 * I, H // 16), np.uint8)
    w13g = np.ones(E, np.float32)
    w2p = np.zeros((E, H, I // 2), np.uint8)
    w2s = np.zeros((E, H, I // 16), np.uint8)
    w2g = np.ones(E, np.float32)
    for e in experts_needed:
        r13 = _oracle_expert_checked(orc, W, cfg, e, "w13")
        w13p[e], w13s[e], w13g[e] = r13.packed, r13.scales, r13.G
        r2 = _oracle_expert_checked(orc, W, cfg, e, "w2")
        w2p[e], w2s[e], w2g[e] = r2.packed, r2.scales, r2.G
    ex13 = orc.Experts(w13p, w13s, w13g)
    ex2 = orc.Experts(w2p, w2s, w2g)
    # 3. h on sampled list positions
    h_ref = orc.moe_gate_up(xo, perm, offsets, k, ex13, rows)
    h_gpu = g["h"].cpu()
    h_bits = synth.bits(h_gpu)
    err_h = rel_err(bf16_to_f64(h_bits[rows]), bf16_to_f64(h_ref))
    print(f"h rel err {err_h:.3e}")
    assert err_h <= GEMM_TOL + BF16_HALF_ULP
    # 4. G_h and hq bit-exact vs oracle Q(h_gpu)
    amax_h = np.abs(bf16_to_f64(h_bits)).max()
    assert np.uint32(g["hmax"].item()) == np.float32(amax_h).view(np.uint32)
    hq_ref = orc.quantize(np.ascontiguousarray(h_bits[rows]), static_G=orc.global_from_amax(amax_h))
    assert np.float32(g["hq"].global_.item()) == np.float32(orc.global_from_amax(amax_h))
    np.testing.assert_array_equal(u8(g["hq"].scales)[0][rows], hq_ref.scales)
    np.testing.assert_array_equal(u8(g["hq"].packed)[0][rows], hq_ref.packed)
    # 5. y from the GPU's hq
    hq_full = to_oracle(g["hq"])
    y_ref = orc.moe_down(hq_full, offsets, ex2, rows)
    err_y = rel_err(g["y"].cpu().numpy()[rows], y_ref)
    print(f"y rel err {err_y:.3e}")
    assert err_y <= GEMM_TOL
    # 6. combine on sampled tokens (all k slots of each)
    if sample_tokens is None:
        toks = np.arange(T)
    else:
        toks = np.unique(np.r_[rng.choice(T, sample_tokens, replace=False), T - 1])
    slot_rows = inv.reshape(T, k)[toks].ravel()
    for e in sorted(set(int(np.searchsorted(offsets, q, side="right") - 1) for q in slot_rows)):
        if e not in experts_needed:
            r2 = _oracle_expert_checked(orc, W, cfg, e, "w2")
            w2p[e], w2s[e], w2g[e] = r2.packed, r2.scales, r2.G
    ex2 = orc.Experts(w2p, w2s, w2g)
    y_tok = orc.moe_down(hq_full, offsets, ex2, slot_rows)
    y_full = np.zeros((T * k, H))
    y_full[slot_rows] = y_tok
    out_ref = orc.moe_combine(y_full, inv, w_np)[toks]
    err_o = rel_err(tensor_bf16_to_f64(g["out"])[toks], bf16_to_f64(out_ref))
    print(f"out rel err {err_o:.3e}")
    assert err_o <= GEMM_TOL + BF16_HALF_ULP
    # 7. fused == staged
    step("moe fused run")
    fused = nv.nvfp4_moe_grouped_gemm(x, ids, w, W.w13, W.w2)
    torch.cuda.synchronize()
    if fused_exact:
        assert torch.equal(fused, g["out"])
    else:
        # the fused down projection splits K (fp32 partial planes added in a
        # fixed order), so only the summation order differs from the staged run
        err_f = rel_err(tensor_bf16_to_f64(fused), tensor_bf16_to_f64(g["out"]))
        print(f"fused vs staged rel err {err_f:.3e}")
        assert err_f <= GEMM_TOL + BF16_HALF_ULP
        again = nv.nvfp4_moe_grouped_gemm(x, ids, w, W.w13, W.w2)
        assert torch.equal(again, fused)
    assert nv.nvfp4_get_error() == 0
    return g, W


def test_small_moe_every_row(orc):
    cfg = synth.MoE(seed=30, E=8, k=3, H=512, I=256, T=77)
    _check_moe(orc, cfg)


def test_small_moe_mx_experts_every_row(orc):
    cfg = synth.MoE(seed=31, E=5, k=2, H=384, I=256, T=50, zipf=1.1, mx=True)
    _check_moe(orc, cfg)


def test_moe_many_items_per_workgroup(orc):
    """A decode-sized batch (every tile a 16-row streaming tile) whose gate_up
    projection has more (tile, column tile) items than resident workgroups,
    each one stage long (H = 256): the streaming pipeline crosses an item
    boundary at every stage; every row checked."""
    cfg = synth.MoE(seed=38, E=64, k=8, H=256, I=2048, T=64)
    _check_moe(orc, cfg)


def test_fused_down_k_split_small(orc):
    """A batch of 12 tokens over 2 experts with I = 2048: the fused layer splits
    the down projection's K over two streaming workgroups."""
    cfg = synth.MoE(seed=35, E=2, k=1, H=512, I=2048, T=12)
    assert nv.nvfp4_workspace_size(3, cfg.T, cfg.k, cfg.E, cfg.H, cfg.I) >= 2 * cfg.T * cfg.H * 4
    _check_moe(orc, cfg, fused_exact=False)


def test_fused_gate_up_k_split_small(orc):
    """12 tokens over 2 experts with H = 2048: the fused layer splits the
    gate_up projection's K over two streaming workgroups (partial gate and
    up planes, SwiGLU after the ordered sum)."""
    cfg = synth.MoE(seed=37, E=2, k=1, H=2048, I=512, T=12)
    _check_moe(orc, cfg, fused_exact=False)


@pytest.mark.parametrize("T", [1, 32])
def test_dense_mlp_as_one_expert_sampled(orc, T):
    """The 27B-class MLP (H=5120, I=17408) as a one-expert layer at decode
    batch sizes: streaming tiles, K-split down projection."""
    cfg = synth.MoE(seed=36, E=1, k=1, H=5120, I=17408, T=T)
    _check_moe(orc, cfg, sample_rows=min(T, 6), sample_tokens=min(T, 3), fused_exact=False)


def test_single_expert_is_dense_mlp(orc):
    """E=1, k=1, w=1: the MoE path equals the dense MLP built from nvfp4_gemm."""
    T, H, I = 40, 512, 384
    x = synth.normal_bf16((T, H), 1.0, (32, 0), DEV)
    w13 = nv.nvfp4_quantize(synth.normal_bf16((2 * I, H), 0.02, (32, 1), DEV))
    w2 = nv.nvfp4_quantize(synth.normal_bf16((H, I), 0.02, (32, 2), DEV))
    ids = torch.zeros((T, 1), dtype=torch.int32, device=DEV)
    wt = torch.ones((T, 1), dtype=torch.float32, device=DEV)
    step("moe E=1 vs dense")
    out = nv.nvfp4_moe_grouped_gemm(x, ids, wt, w13, w2)
    xq = nv.nvfp4_quantize(x)
    gu = nv.nvfp4_gemm(xq, w13)
    h = (torch.nn.functional.silu(gu[:, :I]) * gu[:, I:]).to(torch.bfloat16)
    ref = nv.nvfp4_gemm(nv.nvfp4_quantize(h), w2, torch.bfloat16)
    err = rel_err(out.float().cpu().numpy(), ref.float().cpu().numpy())
    print(f"E=1 MoE vs dense rel err {err:.3e}")
    assert err <= 2e-2  # h re-quantization can flip codes between the two fp32 orders


def test_invalid_expert_ids_raise_and_are_dropped(orc):
    T, k, E = 20, 2, 4
    ids = torch.randint(0, E, (T, k), dtype=torch.int32, device=DEV)
    ids[3, 1] = 7
    ids[5, 0] = -1
    step("route with invalid ids")
    perm, offsets, inv = nv.nvfp4_moe_route(ids, E)
    assert nv.nvfp4_get_error() == 3
    inv = inv.cpu().numpy()
    assert inv[3 * k + 1] == -1 and inv[5 * k + 0] == -1
    assert offsets.cpu().numpy()[E] == T * k - 2
    assert nv.nvfp4_get_error() == 0


def test_moe_empty_and_deterministic():
    cfg = synth.MoE(seed=33, E=4, k=2, H=256, I=128, T=16)
    W = workloads.build_moe_weights(cfg, DEV)
    x = cfg.x(DEV)
    ids, w = workloads.routing(cfg, DEV)
    a = nv.nvfp4_moe_grouped_gemm(x, ids, w, W.w13, W.w2)
    b = nv.nvfp4_moe_grouped_gemm(x, ids, w, W.w13, W.w2)
    assert torch.equal(a, b)
    e = nv.nvfp4_moe_grouped_gemm(x[:0], ids[:0], w[:0], W.w13, W.w2)
    assert e.shape == (0, cfg.H)


@pytest.mark.parametrize("cfg", [synth.MoE(seed=34, E=4, k=2, H=256, I=128, T=33),
                                 synth.MoE(seed=37, E=2, k=1, H=2048, I=512, T=12),
                                 synth.MoE(seed=41, E=3, k=2, H=512, I=256, T=300, mx=True)],
                         ids=["small", "gate-split", "tiles-mx"])
def test_static_globals_equal_dynamic(cfg):
    """Static globals equal to the dynamic ones give the same output; with a
    static G_h the gate_up epilogue encodes h itself (tile, streaming and
    K-split paths), so this also pins that encode to the quantize kernel."""
    step(f"moe static globals E={cfg.E} H={cfg.H} I={cfg.I} T={cfg.T}")
    W = workloads.build_moe_weights(cfg, DEV)
    x = cfg.x(DEV)
    ids, w = workloads.routing(cfg, DEV)
    g = _run_staged(x, ids, w, W, cfg)
    sg = torch.stack([g["xq"].global_[0], g["hq"].global_[0]]).contiguous()
    out = nv.nvfp4_moe_grouped_gemm(x, ids, w, W.w13, W.w2, static_in_globals=sg)
    assert torch.equal(out, g["out"])


@pytest.mark.parametrize("cfg,scale", [
    (synth.MoE(seed=42, E=4, k=2, H=512, I=256, T=300), 1.0),     # 256/128-row tiles + streaming
    (synth.MoE(seed=43, E=4, k=2, H=576, I=256, T=40), 1.0),      # K % 256 != 0: 32-row tiles
    (synth.MoE(seed=44, E=8, k=2, H=1024, I=256, T=48, mx=True), 0.25),  # streaming, saturating G_h
])
def test_gate_up_q_equals_quantize_of_h(orc, cfg, scale):
    """nvfp4_moe_gate_up_q (h encoded in the epilogue with a static G_h)
    gives, byte for byte, nvfp4_quantize(h, static G_h) of the h that
    nvfp4_moe_gate_up writes, and the oracle's quantization of that h."""
    step(f"gate_up_q E={cfg.E} H={cfg.H} I={cfg.I} T={cfg.T} scale={scale}")
    W = workloads.build_moe_weights(cfg, DEV)
    x = cfg.x(DEV)
    ids, _ = workloads.routing(cfg, DEV)
    xq = nv.nvfp4_quantize(x)
    perm, offsets, _ = nv.nvfp4_moe_route(ids, cfg.E)
    h, hmax = nv.nvfp4_moe_gate_up(xq, perm, offsets, cfg.k, W.w13)
    amax = float(np.uint32(hmax.item()).view(np.float32))
    Gh = np.float32(orc.global_from_amax(amax) * scale)
    g = torch.tensor([Gh], dtype=torch.float32, device=DEV)
    hq = nv.nvfp4_moe_gate_up_q(xq, perm, offsets, cfg.k, W.w13, g)
    ref = nv.nvfp4_quantize(h, static_global=g)
    assert torch.equal(hq.packed, ref.packed)
    assert torch.equal(hq.scales, ref.scales)
    ho = orc.quantize(synth.bits(h.cpu()), static_G=Gh)
    np.testing.assert_array_equal(u8(hq.packed)[0], ho.packed)
    np.testing.assert_array_equal(u8(hq.scales)[0], ho.scales)
