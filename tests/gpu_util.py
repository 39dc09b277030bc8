"""Helpers shared by the GPU parity tests (marshalling and error metrics only)."""
import sys

import numpy as np
import torch

import oracle
from precision_moe_gemm_amd import synth


def step(msg):
    """Name the case before a GPU step, so a failure can be traced."""
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def u8(t):
    return t.detach().contiguous().cpu().numpy()


def to_oracle(t, batch_index=None):
    """An NVFP4Tensor from the device as an oracle NVFP4 (or Experts)."""
    p, s, g = u8(t.packed), u8(t.scales), t.global_.detach().cpu().numpy()
    if batch_index is not None:
        return oracle.NVFP4(np.ascontiguousarray(p[batch_index]), np.ascontiguousarray(s[batch_index]),
                            g[batch_index])
    if t.batch == 1:
        return oracle.NVFP4(np.ascontiguousarray(p[0]), np.ascontiguousarray(s[0]), g[0])
    return oracle.Experts(p, s, g)


def assert_same_nvfp4(gpu, orc_t, rows=None):
    """Bit-exact comparison of codes, scale bytes and global."""
    p = u8(gpu.packed).reshape(-1, gpu.cols // 2)
    s = u8(gpu.scales).reshape(-1, gpu.cols // 16)
    if rows is not None:
        p, s = p[rows], s[rows]
    np.testing.assert_array_equal(s, orc_t.scales, err_msg="scale bytes differ")
    np.testing.assert_array_equal(p, orc_t.packed, err_msg="packed codes differ")
    g = float(gpu.global_[0].item())
    assert np.float32(g).view(np.uint32) == np.float32(orc_t.G).view(np.uint32), (g, orc_t.G)


def rel_err(got, ref):
    """max |got - ref| / max |ref| (the GEMM error metric)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    if den == 0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max() / den)


def elem_rel_err(got, ref, floor=1e-2):
    """Element-wise companion of rel_err: max |got - ref| / |ref| over the
    elements with |ref| >= floor * max |ref| (the floor keeps outputs that
    cancel to near zero, where fp32 summation order dominates, out of it)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    if den == 0:
        return float(np.abs(got).max())
    sel = np.abs(ref) >= floor * den
    return float((np.abs(got[sel] - ref[sel]) / np.abs(ref[sel])).max())


def bf16_to_f64(b):
    return (np.asarray(b).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def tensor_bf16_to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


BF16_HALF_ULP = 2.0 ** -8
# one bf16 ulp relative to the value (7 stored mantissa bits): the element-wise
# bound of a bf16 output whose fp32 source is within the GEMM tolerance
BF16_ULP = 2.0 ** -7
GEMM_TOL = 1e-3
