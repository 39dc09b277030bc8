"""precision_moe_gemm_amd -- Python binding of libnvfp4 (NVFP4 W4A4 on MI355X).

Thin marshalling over the C ABI in include/nvfp4.h: torch tensors supply
device memory and the current HIP stream, every computation runs in the
library's gfx950 kernels.  Functions carry the C names.  A non-OK status
raises :class:`NVFP4Error`.

NVFP4 (page "Qwen3.8-Flash-Next-NVFP4", section 核心): E2M1 codes two per
byte, one E4M3 scale per 16 elements along the last dimension, one FP32
scale per tensor -- 4.5 bits per element.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib

__all__ = [
    "NVFP4Error", "NVFP4Tensor", "nvfp4_workspace_size", "nvfp4_quantize", "nvfp4_dequantize",
    "mxfp4_quantize", "mxfp4_to_nvfp4", "nvfp4_gemm", "nvfp4_moe_grouped_gemm", "nvfp4_moe_grouped_gemm_noalloc",
    "nvfp4_moe_route", "nvfp4_moe_gate_up", "nvfp4_moe_gate_up_q", "nvfp4_moe_down", "nvfp4_moe_combine",
    "nvfp4_gather_dequantize", "nvfp4_tile_scales", "nvfp4_gemm_w4a16", "nvfp4_moe_w4a16", "mxfp8_quantize", "mx_gemm_w4a8", "mx_moe_w4a8", "mx_moe_gate_up", "mx_moe_down",
    "nvfp4_kv_quant", "nvfp4_kv_dequant", "nvfp4_audit_scales", "nvfp4_get_error", "nvfp4_set_checks",
    "nvfp4_recipe", "status_string",
]


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


def status_string(status: int) -> str:
    return _lib.load().nvfp4_status_string(status).decode()


def _check(status: int, what: str):
    if status != _lib.OK:
        raise NVFP4Error(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libnvfp4 operates on device tensors")


@dataclass
class NVFP4Tensor:
    """`batch` stacked NVFP4 matrices of rows x cols on one device.

    packed uint8 [batch, rows, cols/2], scales uint8 (E4M3 bytes)
    [batch, rows, cols/16], global float32 [batch]."""
    packed: torch.Tensor
    scales: torch.Tensor
    global_: torch.Tensor
    rows: int
    cols: int
    batch: int = 1
    flags: int = 0  # _lib.POW2_SCALES when every block scale is a power of two

    @staticmethod
    def empty(rows: int, cols: int, batch: int = 1, device="cuda") -> "NVFP4Tensor":
        return NVFP4Tensor(
            torch.empty((batch, rows, cols // 2), dtype=torch.uint8, device=device),
            torch.empty((batch, rows, cols // 16), dtype=torch.uint8, device=device),
            torch.empty((batch,), dtype=torch.float32, device=device),
            rows, cols, batch)

    def c(self) -> _lib.NVFP4TensorC:
        return _lib.NVFP4TensorC(self.packed.data_ptr(), self.scales.data_ptr(),
                                 self.global_.data_ptr(), self.rows, self.cols, self.batch, self.flags)

    @property
    def device(self):
        return self.packed.device

    def nbytes(self) -> int:
        return self.packed.numel() + self.scales.numel() + 4 * self.global_.numel()


def nvfp4_workspace_size(op: int, T: int = 0, k: int = 0, E: int = 0, H: int = 0, I: int = 0) -> int:
    return int(_lib.load().nvfp4_workspace_size(op, T, k, E, H, I))


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def nvfp4_recipe() -> list:
    out = (ctypes.c_int32 * 6)()
    _lib.load().nvfp4_recipe(out)
    return list(out)


def nvfp4_quantize(x: torch.Tensor, static_global: torch.Tensor | None = None,
                   out: NVFP4Tensor | None = None, ws: torch.Tensor | None = None) -> NVFP4Tensor:
    """bf16 [rows, cols] (row stride x.stride(0)) -> NVFP4."""
    _need_cuda(x, static_global)
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    rows, cols = x.shape
    if out is None:
        out = NVFP4Tensor.empty(rows, cols, 1, x.device)
    if static_global is None and ws is None:
        ws = _workspace(nvfp4_workspace_size(_lib.OP_QUANTIZE), x.device)
    oc = out.c()
    st = _lib.load().nvfp4_quantize(_ptr(x), rows, cols, x.stride(0), _ptr(static_global),
                                   ctypes.byref(oc), _ptr(ws), 0 if ws is None else ws.numel(),
                                   _stream(x.device))
    _check(st, "nvfp4_quantize")
    out.flags = 0
    return out


def nvfp4_dequantize(t: NVFP4Tensor, dtype=torch.float32) -> torch.Tensor:
    out = torch.empty((t.batch * t.rows, t.cols), dtype=dtype, device=t.device)
    code = _lib.BF16 if dtype == torch.bfloat16 else _lib.F32
    tc = t.c()
    _check(_lib.load().nvfp4_dequantize(ctypes.byref(tc), _ptr(out), code, _stream(t.device)),
           "nvfp4_dequantize")
    return out


def nvfp4_gather_dequantize(table: NVFP4Tensor, ids: torch.Tensor, dtype=torch.bfloat16) -> torch.Tensor:
    """Rows ids (int32 [n]) of an NVFP4 table, dequantized: [n, cols]."""
    _need_cuda(ids)
    assert ids.dtype == torch.int32 and ids.dim() == 1 and ids.is_contiguous()
    n = ids.numel()
    out = torch.empty((n, table.cols), dtype=dtype, device=table.device)
    code = _lib.BF16 if dtype == torch.bfloat16 else _lib.F32
    tc = table.c()
    _check(_lib.load().nvfp4_gather_dequantize(ctypes.byref(tc), _ptr(ids), n, _ptr(out), code,
                                               _stream(table.device)), "nvfp4_gather_dequantize")
    return out


def nvfp4_tile_scales(t: NVFP4Tensor) -> NVFP4Tensor:
    """The same tensor with its scale bytes in the 128-row tiled order
    (NVFP4_TILED_SCALES): a new scales buffer; packed and global are shared."""
    scales = torch.empty_like(t.scales)
    tc = t.c()
    _check(_lib.load().nvfp4_tile_scales(ctypes.byref(tc), _ptr(scales), _stream(t.device)), "nvfp4_tile_scales")
    return NVFP4Tensor(t.packed, scales, t.global_, t.rows, t.cols, t.batch, t.flags | _lib.TILED_SCALES)


def mxfp4_quantize(x: torch.Tensor):
    """bf16 [rows, cols] -> (packed uint8 [rows, cols/2], e8m0 uint8 [rows, cols/32])."""
    _need_cuda(x)
    rows, cols = x.shape
    packed = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
    e8 = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    _check(_lib.load().mxfp4_quantize(_ptr(x), rows, cols, x.stride(0), _ptr(packed), _ptr(e8),
                                      _stream(x.device)), "mxfp4_quantize")
    return packed, e8


def mxfp8_quantize(x: torch.Tensor):
    """bf16 [rows, cols] -> (E4M3 uint8 [rows, cols], e8m0 uint8 [rows, cols/32])."""
    _need_cuda(x)
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    e8 = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    _check(_lib.load().mxfp8_quantize(_ptr(x), rows, cols, x.stride(0), _ptr(q), _ptr(e8), _stream(x.device)),
           "mxfp8_quantize")
    return q, e8


def mx_gemm_w4a8(a: torch.Tensor, a_e8m0: torch.Tensor, w_packed: torch.Tensor, w_e8m0: torch.Tensor,
                 dtype=torch.float32, out: torch.Tensor | None = None):
    """C[M, N] = a W^T with MXFP8 activations (E4M3 [M, K], e8m0 [M, K/32])
    and MXFP4 weights (codes [N, K/2], e8m0 [N, K/32])."""
    _need_cuda(a, a_e8m0, w_packed, w_e8m0)
    for t in (a, a_e8m0, w_packed, w_e8m0):
        if t.dtype != torch.uint8 or not t.is_contiguous():
            raise ValueError("MX operands are contiguous uint8 tensors")
    M, K = a.shape
    N = w_packed.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=dtype, device=a.device)
    code = _lib.BF16 if out.dtype == torch.bfloat16 else _lib.F32
    _check(_lib.load().mx_gemm_w4a8(_ptr(a), _ptr(a_e8m0), M, K, _ptr(w_packed), _ptr(w_e8m0), N, _ptr(out),
                                    code, _stream(a.device)), "mx_gemm_w4a8")
    return out


def mx_moe_w4a8(x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor, w13: torch.Tensor,
                w13_e8m0: torch.Tensor, w2: torch.Tensor, w2_e8m0: torch.Tensor, out: torch.Tensor | None = None,
                ws: torch.Tensor | None = None):
    """MX-native W4A8 routed-expert MoE forward: bf16 x [T, H] -> bf16 [T, H]
    with MXFP4 experts (w13 codes [E, 2I, H/2], e8m0 [E, 2I, H/32]; w2 codes
    [E, H, I/2], e8m0 [E, H, I/32]) and MXFP8 activations."""
    _need_cuda(x, topk_ids, topk_w, w13, w13_e8m0, w2, w2_e8m0)
    for t in (w13, w13_e8m0, w2, w2_e8m0):
        if t.dtype != torch.uint8 or not t.is_contiguous():
            raise ValueError("MX expert operands are contiguous uint8 tensors")
    T, H = x.shape
    k = topk_ids.shape[1]
    E, I2 = w13.shape[0], w13.shape[1]
    I = I2 // 2
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if ws is None:
        ws = _workspace(nvfp4_workspace_size(_lib.OP_MX_MOE, T, k, E, H, I), x.device)
    _check(_lib.load().mx_moe_w4a8(
        _ptr(x), _ptr(topk_ids), _ptr(topk_w), T, k, E, H, I, _ptr(w13), _ptr(w13_e8m0), _ptr(w2), _ptr(w2_e8m0),
        _ptr(out), _ptr(ws), ws.numel(), _stream(x.device)), "mx_moe_w4a8")
    return out


def mx_moe_gate_up(xq: torch.Tensor, xe: torch.Tensor, perm: torch.Tensor, offsets: torch.Tensor, k: int,
                   w13: torch.Tensor, w13_e8m0: torch.Tensor, ws: torch.Tensor | None = None):
    """MX gate_up + SwiGLU: MXFP8 x (codes [T, H], e8m0 [T, H/32]) -> (h bf16
    [T*k, I] in list order, max |h| as float bits)."""
    T, H = xq.shape
    E, I = w13.shape[0], w13.shape[1] // 2
    dev = xq.device
    h = torch.empty((T * k, I), dtype=torch.bfloat16, device=dev)
    hmax = torch.zeros(1, dtype=torch.int32, device=dev)
    if ws is None:
        ws = _workspace(nvfp4_workspace_size(_lib.OP_MOE_ROUTE, T, k, E), dev)
    _check(_lib.load().mx_moe_gate_up(_ptr(xq), _ptr(xe), _ptr(perm), _ptr(offsets), T, k, E, H, I, _ptr(w13),
                                      _ptr(w13_e8m0), _ptr(h), _ptr(hmax), _ptr(ws), ws.numel(), _stream(dev)),
           "mx_moe_gate_up")
    return h, hmax


def mx_moe_down(hq: torch.Tensor, he: torch.Tensor, offsets: torch.Tensor, T: int, k: int, w2: torch.Tensor,
                w2_e8m0: torch.Tensor, ws: torch.Tensor | None = None):
    """MX down: MXFP8 h (codes [T*k, I], e8m0 [T*k, I/32], list order) -> y
    fp32 [T*k, H]."""
    E, H = w2.shape[0], w2.shape[1]
    I = hq.shape[1]
    dev = hq.device
    y = torch.empty((T * k, H), dtype=torch.float32, device=dev)
    if ws is None:
        ws = _workspace(nvfp4_workspace_size(_lib.OP_MOE_ROUTE, T, k, E), dev)
    _check(_lib.load().mx_moe_down(_ptr(hq), _ptr(he), _ptr(offsets), T, k, E, H, I, _ptr(w2), _ptr(w2_e8m0),
                                   _ptr(y), _ptr(ws), ws.numel(), _stream(dev)), "mx_moe_down")
    return y


def mxfp4_to_nvfp4(packed: torch.Tensor, e8m0: torch.Tensor, rows: int, cols: int, batch: int = 1,
                   out: NVFP4Tensor | None = None, ws: torch.Tensor | None = None,
                   in_place: bool = False) -> NVFP4Tensor:
    """Lossless remap of `batch` stacked MXFP4 matrices.  in_place=True makes
    the result's codes alias `packed` (no copy)."""
    _need_cuda(packed, e8m0)
    dev = packed.device
    if out is None:
        if in_place:
            out = NVFP4Tensor(packed.view(batch, rows, cols // 2),
                              torch.empty((batch, rows, cols // 16), dtype=torch.uint8, device=dev),
                              torch.empty((batch,), dtype=torch.float32, device=dev), rows, cols, batch)
        else:
            out = NVFP4Tensor.empty(rows, cols, batch, dev)
    if ws is None:
        ws = _workspace(nvfp4_workspace_size(_lib.OP_REMAP, batch, 0, 0, rows, cols), dev)
    oc = out.c()
    _check(_lib.load().mxfp4_to_nvfp4(_ptr(packed), _ptr(e8m0), rows, cols, batch, ctypes.byref(oc),
                                      _ptr(ws), ws.numel(), _stream(dev)), "mxfp4_to_nvfp4")
    out.flags = _lib.POW2_SCALES  # remapped scales are 2^k or zero
    return out


def nvfp4_gemm(A: NVFP4Tensor, W: NVFP4Tensor, dtype=torch.float32, out: torch.Tensor | None = None,
               ws: torch.Tensor | None = None):
    """C[M, N] = A W^T with both operands NVFP4.  `ws` (uint8, 256-byte
    aligned) holds split-K partials of few-row shapes; allocated if omitted."""
    if out is None:
        out = torch.empty((A.rows, W.rows), dtype=dtype, device=A.device)
    code = _lib.BF16 if out.dtype == torch.bfloat16 else _lib.F32
    if ws is None:
        n = nvfp4_workspace_size(_lib.OP_GEMM, A.rows, 0, 0, A.cols, W.rows)
        ws = _workspace(n, A.device) if n else None
    ac, wc = A.c(), W.c()
    _check(_lib.load().nvfp4_gemm(ctypes.byref(ac), ctypes.byref(wc), _ptr(out), code, _ptr(ws),
                                  0 if ws is None else ws.numel(), _stream(A.device)), "nvfp4_gemm")
    return out


def nvfp4_moe_grouped_gemm(x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor,
                           w13: NVFP4Tensor, w2: NVFP4Tensor, static_in_globals: torch.Tensor | None = None,
                           out: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """Routed-expert MoE forward: bf16 x [T, H] -> bf16 [T, H]."""
    _need_cuda(x, topk_ids, topk_w)
    T, H = x.shape
    k = topk_ids.shape[1]
    E = w13.batch
    I = w13.rows // 2
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if ws is None:
        ws = _workspace(nvfp4_workspace_size(_lib.OP_MOE, T, k, E, H, I), x.device)
    c13, c2 = w13.c(), w2.c()
    _check(_lib.load().nvfp4_moe_grouped_gemm(
        _ptr(x), _ptr(topk_ids), _ptr(topk_w), T, k, E, ctypes.byref(c13), ctypes.byref(c2),
        _ptr(static_in_globals), _ptr(out), _ptr(ws), ws.numel(), _stream(x.device)),
        "nvfp4_moe_grouped_gemm")
    return out


def nvfp4_moe_grouped_gemm_noalloc(x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor,
                                   w13: NVFP4Tensor, w2: NVFP4Tensor, static_in_globals: torch.Tensor | None = None,
                                   out: torch.Tensor | None = None):
    """nvfp4_moe_grouped_gemm on the library's own device scratch (no
    workspace; for callers that cannot allocate, pass `out`)."""
    _need_cuda(x, topk_ids, topk_w)
    T, H = x.shape
    k = topk_ids.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    c13, c2 = w13.c(), w2.c()
    _check(_lib.load().nvfp4_moe_grouped_gemm_noalloc(
        _ptr(x), _ptr(topk_ids), _ptr(topk_w), T, k, w13.batch, ctypes.byref(c13), ctypes.byref(c2),
        _ptr(static_in_globals), _ptr(out), _stream(x.device)), "nvfp4_moe_grouped_gemm_noalloc")
    return out


def nvfp4_gemm_w4a16(a: torch.Tensor, W: NVFP4Tensor, dtype=torch.float32, out: torch.Tensor | None = None,
                     ws: torch.Tensor | None = None):
    """C[M, N] = a W^T with bf16 activations a [M, K] (row stride a.stride(0))
    and NVFP4 weights W [N, K]."""
    _need_cuda(a)
    if a.dtype != torch.bfloat16 or a.dim() != 2 or a.stride(1) != 1:
        raise ValueError("a must be a 2-D bf16 tensor with unit column stride")
    M, K = a.shape
    if out is None:
        out = torch.empty((M, W.rows), dtype=dtype, device=a.device)
    code = _lib.BF16 if out.dtype == torch.bfloat16 else _lib.F32
    if ws is None:
        n = nvfp4_workspace_size(_lib.OP_GEMM, M, 0, 0, K, W.rows)
        ws = _workspace(n, a.device) if n else None
    wc = W.c()
    _check(_lib.load().nvfp4_gemm_w4a16(_ptr(a), M, K, a.stride(0), ctypes.byref(wc), _ptr(out), code, _ptr(ws),
                                        0 if ws is None else ws.numel(), _stream(a.device)), "nvfp4_gemm_w4a16")
    return out


def nvfp4_moe_w4a16(x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor, w13: NVFP4Tensor,
                    w2: NVFP4Tensor, out: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """W4A16 routed-expert MoE forward: bf16 x [T, H] -> bf16 [T, H], no
    activation quantization."""
    _need_cuda(x, topk_ids, topk_w)
    T, H = x.shape
    k = topk_ids.shape[1]
    E = w13.batch
    I = w13.rows // 2
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if ws is None:
        ws = _workspace(nvfp4_workspace_size(_lib.OP_MOE, T, k, E, H, I), x.device)
    c13, c2 = w13.c(), w2.c()
    _check(_lib.load().nvfp4_moe_w4a16(
        _ptr(x), _ptr(topk_ids), _ptr(topk_w), T, k, E, ctypes.byref(c13), ctypes.byref(c2),
        _ptr(out), _ptr(ws), ws.numel(), _stream(x.device)), "nvfp4_moe_w4a16")
    return out


def nvfp4_moe_route(topk_ids: torch.Tensor, E: int, ws: torch.Tensor | None = None):
    T, k = topk_ids.shape
    dev = topk_ids.device
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    if ws is None:
        ws = _workspace(nvfp4_workspace_size(_lib.OP_MOE_ROUTE, T, k, E), dev)
    _check(_lib.load().nvfp4_moe_route(_ptr(topk_ids), T, k, E, _ptr(perm), _ptr(offsets), _ptr(inv),
                                       _ptr(ws), ws.numel(), _stream(dev)), "nvfp4_moe_route")
    return perm, offsets, inv


def nvfp4_moe_gate_up(xq: NVFP4Tensor, perm: torch.Tensor, offsets: torch.Tensor, k: int,
                      w13: NVFP4Tensor, ws: torch.Tensor | None = None):
    """h bf16 [T*k, I] (list order) and the uint32 max-|h| word."""
    T = xq.rows
    E = w13.batch
    I = w13.rows // 2
    dev = xq.device
    h = torch.empty((T * k, I), dtype=torch.bfloat16, device=dev)
    hmax = torch.zeros(1, dtype=torch.int32, device=dev)
    if ws is None:
        ws = _workspace(nvfp4_workspace_size(_lib.OP_MOE_ROUTE, T, k, E), dev)
    xc, wc = xq.c(), w13.c()
    _check(_lib.load().nvfp4_moe_gate_up(ctypes.byref(xc), _ptr(perm), _ptr(offsets), T, k, E,
                                         ctypes.byref(wc), _ptr(h), _ptr(hmax), _ptr(ws), ws.numel(),
                                         _stream(dev)), "nvfp4_moe_gate_up")
    return h, hmax


def nvfp4_moe_gate_up_q(xq: NVFP4Tensor, perm: torch.Tensor, offsets: torch.Tensor, k: int,
                        w13: NVFP4Tensor, h_global: torch.Tensor, ws: torch.Tensor | None = None) -> NVFP4Tensor:
    """gate_up + SwiGLU with h encoded to NVFP4 in the epilogue under the
    static global h_global (float32 [1] on the device): the NVFP4 h [T*k, I]
    (list order) whose global is h_global."""
    T = xq.rows
    E = w13.batch
    I = w13.rows // 2
    dev = xq.device
    _need_cuda(h_global)
    hq = NVFP4Tensor(torch.empty((1, T * k, I // 2), dtype=torch.uint8, device=dev),
                     torch.empty((1, T * k, I // 16), dtype=torch.uint8, device=dev),
                     h_global.reshape(1), T * k, I, 1)
    if ws is None:
        ws = _workspace(nvfp4_workspace_size(_lib.OP_MOE_ROUTE, T, k, E), dev)
    xc, wc, hc = xq.c(), w13.c(), hq.c()
    _check(_lib.load().nvfp4_moe_gate_up_q(ctypes.byref(xc), _ptr(perm), _ptr(offsets), T, k, E,
                                           ctypes.byref(wc), _ptr(h_global), ctypes.byref(hc), _ptr(ws),
                                           ws.numel(), _stream(dev)), "nvfp4_moe_gate_up_q")
    return hq


def nvfp4_moe_down(hq: NVFP4Tensor, offsets: torch.Tensor, T: int, k: int, w2: NVFP4Tensor,
                   ws: torch.Tensor | None = None):
    """y fp32 [T*k, H] (list order)."""
    E = w2.batch
    H = w2.rows
    dev = hq.device
    y = torch.empty((T * k, H), dtype=torch.float32, device=dev)
    if ws is None:
        ws = _workspace(nvfp4_workspace_size(_lib.OP_MOE_ROUTE, T, k, E), dev)
    hc, wc = hq.c(), w2.c()
    _check(_lib.load().nvfp4_moe_down(ctypes.byref(hc), _ptr(offsets), T, k, E, ctypes.byref(wc),
                                      _ptr(y), _ptr(ws), ws.numel(), _stream(dev)), "nvfp4_moe_down")
    return y


def nvfp4_moe_combine(y: torch.Tensor, inv: torch.Tensor, topk_w: torch.Tensor):
    T, k = topk_w.shape
    H = y.shape[1]
    out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    _check(_lib.load().nvfp4_moe_combine(_ptr(y), _ptr(inv), _ptr(topk_w), T, k, H, _ptr(out),
                                         _stream(y.device)), "nvfp4_moe_combine")
    return out


def nvfp4_kv_quant(k: torch.Tensor | None, v: torch.Tensor | None, tok_offset: int,
                   k_cache: NVFP4Tensor, v_cache: NVFP4Tensor, heads: int):
    """Quantize bf16 [n, heads, head_dim] chunks into the caches at tok_offset."""
    ref = k if k is not None else v
    n = ref.shape[0]
    kc, vc = k_cache.c(), v_cache.c()
    _check(_lib.load().nvfp4_kv_quant(_ptr(k), _ptr(v), n, heads, tok_offset, ctypes.byref(kc),
                                      ctypes.byref(vc), _stream(ref.device)), "nvfp4_kv_quant")


def nvfp4_kv_dequant(k_cache: NVFP4Tensor, v_cache: NVFP4Tensor, heads: int, tok_begin: int, n: int,
                     dtype=torch.bfloat16, want_k=True, want_v=True, k_out=None, v_out=None):
    D = k_cache.cols
    dev = k_cache.device
    ko = vo = None
    if want_k:
        ko = k_out if k_out is not None else torch.empty((n, heads, D), dtype=dtype, device=dev)
    if want_v:
        vo = v_out if v_out is not None else torch.empty((n, heads, D), dtype=dtype, device=dev)
    code = _lib.BF16 if dtype == torch.bfloat16 else _lib.F32
    kc, vc = k_cache.c(), v_cache.c()
    _check(_lib.load().nvfp4_kv_dequant(ctypes.byref(kc), ctypes.byref(vc), heads, tok_begin, n,
                                        _ptr(ko), _ptr(vo), code, _stream(dev)), "nvfp4_kv_dequant")
    return ko, vo


def nvfp4_audit_scales(t: NVFP4Tensor) -> torch.Tensor:
    """int64 [4] = {scale bytes, non-finite, non-positive, equal to 448}."""
    counts = torch.empty(4, dtype=torch.int64, device=t.device)
    tc = t.c()
    _check(_lib.load().nvfp4_audit_scales(ctypes.byref(tc), _ptr(counts), _stream(t.device)),
           "nvfp4_audit_scales")
    return counts


def nvfp4_set_checks(on: bool) -> bool:
    """Switch the operand data checks on or off for the process (see
    include/nvfp4.h); returns the previous setting."""
    return bool(_lib.load().nvfp4_set_checks(1 if on else 0))


def nvfp4_get_error(device=None) -> int:
    """Synchronize the current stream; return and clear the sticky device error."""
    return int(_lib.load().nvfp4_get_error(_stream(device)))
