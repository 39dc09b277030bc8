"""GPU parity: NVFP4 quantize / dequantize / scale audit vs the CPU oracle.

Bar: bit-exact packed codes, scale bytes and global scale.  Inputs are the
seeded synthetic tensors of the workloads plus a sweep of every finite bf16
bit pattern under a grid of static globals.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_moe_gemm_amd as nv
from precision_moe_gemm_amd import synth
from tests.gpu_util import assert_same_nvfp4, step, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _all_finite_bf16():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = (b & 0x7F80) != 0x7F80
    return b[finite]


def _gpu_q(xb, static_G=None):
    x = synth.from_bits(xb, DEV)
    g = None if static_G is None else torch.tensor([static_G], dtype=torch.float32, device=DEV)
    return nv.nvfp4_quantize(x, static_global=g)


@pytest.mark.parametrize("G", [1.0, 2.0 ** -20, 1e-3, 0.37, 3.0e5, 1e-30, 1e30])
def test_every_finite_bf16_under_static_globals(orc, G):
    vals = _all_finite_bf16()
    vals = vals[: (vals.size // 16) * 16]
    for order in ("sorted", "shuffled"):
        v = vals if order == "sorted" else np.random.default_rng(1).permutation(vals)
        xb = np.ascontiguousarray(v.reshape(-1, 64))
        step(f"quantize sweep G={G} {order} shape={xb.shape}")
        q = _gpu_q(xb, G)
        ref = orc.quantize(xb, static_G=G)
        assert_same_nvfp4(q, ref)


def test_every_finite_bf16_dynamic(orc):
    vals = _all_finite_bf16()
    vals = vals[: (vals.size // 16) * 16]
    xb = np.ascontiguousarray(np.random.default_rng(2).permutation(vals).reshape(-1, 16))
    step("quantize sweep dynamic")
    assert_same_nvfp4(_gpu_q(xb), orc.quantize(xb))


def test_tiny_linear_operands(orc):
    for name, t in (("x", synth.C1.x()), ("w", synth.C1.w())):
        xb = synth.bits(t)
        step(f"quantize tiny linear {name}")
        q = _gpu_q(xb)
        ref = orc.quantize(xb)
        assert_same_nvfp4(q, ref)
        counts = nv.nvfp4_audit_scales(q).cpu().numpy()
        a = orc.audit_scales(ref)
        assert list(counts) == [a["total"], a["nonfinite"], a["nonpositive"], a["at_max"]]
        assert counts[1] == 0 and counts[2] == 0 and counts[3] >= 1


@pytest.mark.parametrize("shape", [(1, 16), (3, 48), (7, 1040), (257, 272), (1000, 512)])
def test_ragged_shapes(orc, shape):
    xb = synth.bits(synth.normal_bf16(shape, 1.0, (200, *shape)))
    step(f"quantize ragged {shape}")
    assert_same_nvfp4(_gpu_q(xb), orc.quantize(xb))


def test_strided_rows(orc):
    full = synth.normal_bf16((64, 384), 1.0, (201, 0), DEV)
    view = full[:, 64:320]  # row stride 384 elements, 256 columns
    step("quantize strided view")
    q = nv.nvfp4_quantize(view)
    ref = orc.quantize(np.ascontiguousarray(synth.bits(view)))
    assert_same_nvfp4(q, ref)


def test_degenerate_values(orc):
    rows = []
    rows.append(np.zeros(64, np.float32))                     # zero row
    rows.append(np.r_[np.full(16, -0.0), np.full(48, 1.0)])   # negative zeros
    rows.append(np.r_[np.full(16, 1000.0), np.linspace(-1e-2, 1e-2, 48)])  # subnormal scales
    rows.append(np.r_[np.full(16, 3e38), np.full(48, 1e-38)])  # extreme spread
    x = torch.tensor(np.stack(rows), dtype=torch.float32).to(torch.bfloat16)
    xb = synth.bits(x)
    for G in (None, 1e-37, 1.0):
        step(f"quantize degenerate G={G}")
        assert_same_nvfp4(_gpu_q(xb, G), orc.quantize(xb, static_G=G))


def test_tiny_magnitudes_underflow_path(orc):
    """Tensors of bf16 subnormals: s*G underflows, the reciprocal is inf."""
    b = np.arange(1, 0x80, dtype=np.uint16)       # positive bf16 subnormals
    v = np.concatenate([b, b | 0x8000, np.zeros(2, np.uint16)])
    v = v[: (v.size // 16) * 16].reshape(-1, 16)
    step("quantize subnormal tensor")
    assert_same_nvfp4(_gpu_q(v), orc.quantize(v))


def test_all_zero_tensor_and_empty(orc):
    xb = np.zeros((4, 32), np.uint16)
    step("quantize zeros")
    q = _gpu_q(xb)
    assert_same_nvfp4(q, orc.quantize(xb))
    assert q.global_.item() == 1.0
    x0 = torch.empty((0, 32), dtype=torch.bfloat16, device=DEV)
    q0 = nv.nvfp4_quantize(x0)
    torch.cuda.synchronize()
    assert q0.global_.item() == 1.0


def test_dense_mlp_weights_sampled(orc):
    """27B-class MLP weights (34816x5120, 5120x17408): exact global, sampled rows bit-exact."""
    c = synth.C2
    for name, gen in (("w13", c.w13), ("w2", c.w2)):
        w = gen(DEV)
        step(f"quantize dense MLP {name} {tuple(w.shape)}")
        q = nv.nvfp4_quantize(w)
        torch.cuda.synchronize()
        amax = w.float().abs().max().item()
        G = orc.global_from_amax(amax)
        assert np.float32(q.global_.item()) == np.float32(G)
        rows = np.random.default_rng(3).choice(w.shape[0], 48, replace=False)
        rows = np.concatenate([rows, [0, w.shape[0] - 1]])
        xb = synth.bits(w[torch.from_numpy(rows).to(DEV)])
        ref = orc.quantize(np.ascontiguousarray(xb), static_G=G)
        assert_same_nvfp4(q, ref, rows=rows)
        del w, q


def test_dequantize_matches_oracle(orc):
    xb = synth.bits(synth.C1.x())
    q = _gpu_q(xb)
    ref = orc.quantize(xb)
    f_ref, b_ref = orc.dequantize(ref, want_bf16=True)
    step("dequantize f32/bf16")
    f = nv.nvfp4_dequantize(q, torch.float32).cpu().numpy()
    b = synth.bits(nv.nvfp4_dequantize(q, torch.bfloat16))
    np.testing.assert_array_equal(f.view(np.uint32), f_ref.view(np.uint32))
    np.testing.assert_array_equal(b, b_ref)


def test_dequantize_batched_globals(orc):
    ts = [orc.quantize(synth.bits(synth.normal_bf16((32, 64), 10.0 ** i, (202, i)))) for i in range(3)]
    ex = orc.Experts.stack(ts)
    t = nv.NVFP4Tensor(torch.from_numpy(ex.packed).to(DEV), torch.from_numpy(ex.scales).to(DEV),
                       torch.from_numpy(ex.G).to(DEV), 32, 64, 3)
    step("dequantize batched")
    f = nv.nvfp4_dequantize(t).cpu().numpy()
    ref = np.concatenate([orc.dequantize(x) for x in ts])
    np.testing.assert_array_equal(f.view(np.uint32), ref.view(np.uint32))


def test_deterministic(orc):
    x = synth.C1.x(DEV)
    a = nv.nvfp4_quantize(x)
    b = nv.nvfp4_quantize(x)
    assert torch.equal(a.packed, b.packed) and torch.equal(a.scales, b.scales)
    assert torch.equal(a.global_, b.global_)


def test_host_errors():
    x = torch.zeros((4, 24), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(nv.NVFP4Error) as ei:
        nv.nvfp4_quantize(x, out=nv.NVFP4Tensor.empty(4, 16, 1, DEV))
    assert ei.value.status == 2


@pytest.mark.parametrize("R,D,n", [(1000, 2560, 700), (37, 64, 5), (513, 16, 1031), (200, 96, 333), (50, 48, 77)])
def test_gather_dequantize_matches_oracle(orc, R, D, n):
    """Row gather-dequantize of an NVFP4 embedding table (rows of 2560 as in
    the n-gram table, plus small and ragged shapes): bit-exact against the
    oracle for fp32 and bf16, repeated and unsorted ids."""
    step(f"gather dequant R={R} D={D} n={n}")
    xb = synth.bits(synth.normal_bf16((R, D), 0.05, (730, R, D)))
    t = _gpu_q(xb)
    ref = orc.quantize(xb)
    ids = np.random.default_rng(R + n).integers(0, R, n).astype(np.int32)
    gi = torch.from_numpy(ids).to(DEV)
    f_ref, b_ref = orc.gather_dequantize(ref, ids, want_bf16=True)
    f = nv.nvfp4_gather_dequantize(t, gi, torch.float32).cpu().numpy()
    b = synth.bits(nv.nvfp4_gather_dequantize(t, gi, torch.bfloat16))
    np.testing.assert_array_equal(f.view(np.uint32), f_ref.view(np.uint32))
    np.testing.assert_array_equal(b, b_ref)


def test_gather_dequantize_bad_ids_and_empty(orc):
    xb = synth.bits(synth.normal_bf16((40, 128), 1.0, (731,)))
    t = _gpu_q(xb)
    ref = orc.quantize(xb)
    ids = np.array([3, -1, 40, 39, 0, 1 << 30], np.int32)
    nv.nvfp4_get_error()  # clear
    f = nv.nvfp4_gather_dequantize(t, torch.from_numpy(ids).to(DEV), torch.float32).cpu().numpy()
    assert nv.nvfp4_get_error() == 3  # NVFP4_ERR_RANGE
    np.testing.assert_array_equal(f.view(np.uint32), orc.gather_dequantize(ref, ids).view(np.uint32))
    e = nv.nvfp4_gather_dequantize(t, torch.zeros(0, dtype=torch.int32, device=DEV))
    assert e.shape == (0, 128)


def test_audit_counts_planted_bytes(orc):
    """NaN-pattern, zero, negative-zero, negative and 448 scale bytes planted
    in a tensor: the device audit gives the hand counts and the oracle's."""
    from tests.test_oracle_quant import AUDIT_EXPECT, audit_planted_scales
    s = audit_planted_scales()
    t = nv.NVFP4Tensor(torch.zeros((1, 3, 96), dtype=torch.uint8, device=DEV),
                       torch.from_numpy(s).reshape(1, 3, 12).to(DEV),
                       torch.ones(1, dtype=torch.float32, device=DEV), 3, 192, 1)
    step("audit planted scale bytes")
    counts = nv.nvfp4_audit_scales(t).cpu().numpy().tolist()
    want = [AUDIT_EXPECT[k] for k in ("total", "nonfinite", "nonpositive", "at_max")]
    assert counts == want
    a = orc.audit_scales(orc.NVFP4(np.zeros((3, 96), np.uint8), s, 1.0))
    assert counts == [a["total"], a["nonfinite"], a["nonpositive"], a["at_max"]]
