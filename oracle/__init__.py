"""CPU oracle for the NVFP4 W4A4 hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (``libnvfp4`` and the
``precision_moe_gemm_amd`` binding) never imports, links or calls it; the two
share no code.

The arithmetic lives in ``nvfp4_oracle.c`` (plain C, IEEE binary32 step by
step, brute-force codecs, exact int64 GEMM); this module is argument
marshalling over ctypes plus a few compositions (KV cache, MoE forward,
audit) that only call the C functions.  bf16 tensors are passed as numpy
``uint16`` arrays of raw bf16 bits.

Sources: the pages "Qwen3.8-Flash-Next-NVFP4" (section 核心: two-level scaling,
4.5 bits, dynamic activations; section 证据链: scale audit),
"DeepSeek-V4.1-Flash-NVFP4" (section 二: E2M1 table, packing, MXFP4 vs NVFP4;
sections 一/四/六: lossless remap), "Qwen3.8-2.4T-A95B-NVFP4" (NVFP4 KV cache),
"Qwen3.8-27B-NVFP4" (section 2: NVFP4 MLP shapes) and
"Qwen3.8-Flash-Next-FP4-Local" (section 2.1: NVFP4 n-gram table; section 3.2:
W4A16 NVFP4 MTP experts).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
# NVFP4_ORACLE_LIB selects another build of nvfp4_oracle.c (the sanitizer
# build used by the CPU tests)
_LIB_PATH = os.environ.get("NVFP4_ORACLE_LIB") or os.path.join(_HERE, "libnvfp4_oracle.so")
_lock = threading.Lock()
_lib = None

OK, INVALID, SHAPE, RANGE = 0, 1, 2, 3


class OracleError(RuntimeError):
    def __init__(self, code, what):
        super().__init__(f"oracle {what} failed with code {code}")
        self.code = code


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no FMA contraction, no fast-math)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_sanitized(out: str) -> str:
    """The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
    (gcc; load it with gcc's libasan preloaded, see sanitizer_runtime)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def sanitizer_runtime() -> str:
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        i32 = ctypes.c_int32
        f32 = ctypes.c_float
        sig = {
            "orc_e2m1_value": (ctypes.c_double, [ctypes.c_uint8]),
            "orc_e4m3_value": (ctypes.c_double, [ctypes.c_uint8]),
            "orc_e8m0_value": (ctypes.c_double, [ctypes.c_uint8]),
            "orc_e4m3_encode": (ctypes.c_uint8, [f32]),
            "orc_e2m1_encode": (ctypes.c_uint8, [f32]),
            "orc_bf16_from_double": (ctypes.c_uint16, [ctypes.c_double]),
            "orc_global_from_amax": (f32, [f32]),
            "orc_amax_bf16": (f32, [P, i64, i64, i64]),
            "orc_quantize": (ctypes.c_int, [P, i64, i64, i64, P, P, P, P]),
            "orc_dequantize": (ctypes.c_int, [P, P, f32, i64, i64, P, P]),
            "orc_gemm_rows": (ctypes.c_int, [P, P, f32, P, i64, P, P, f32, P, i64, i64, P]),
            "orc_mxfp4_encode": (ctypes.c_int, [P, i64, i64, i64, P, P]),
            "orc_mxfp4_dequantize": (ctypes.c_int, [P, P, i64, i64, P]),
            "orc_mxfp4_to_nvfp4": (ctypes.c_int, [P, P, i64, i64, P, P, P]),
            "orc_moe_route": (ctypes.c_int, [P, i64, i32, i32, P, P, P]),
            "orc_moe_gate_up": (ctypes.c_int, [P, P, f32, P, P, i32, i32, P, P, P, i64, i64, P, i64, P]),
            "orc_moe_down": (ctypes.c_int, [P, P, f32, P, i32, P, P, P, i64, i64, P, i64, P]),
            "orc_moe_combine": (ctypes.c_int, [P, P, P, i64, i32, i64, P]),
            "orc_gemm_w4a16_rows": (ctypes.c_int, [P, i64, P, i64, P, P, f32, P, i64, i64, P]),
            "orc_moe_w4a16_gate_up": (ctypes.c_int, [P, P, P, i32, i32, P, P, P, i64, i64, P, i64, P]),
            "orc_moe_w4a16_down": (ctypes.c_int, [P, P, i32, P, P, P, i64, i64, P, i64, P]),
            "orc_mxfp8_encode": (ctypes.c_int, [P, i64, i64, i64, P, P]),
            "orc_mx_gemm_w4a8_rows": (ctypes.c_int, [P, P, P, i64, P, P, P, i64, i64, P]),
            "orc_mx_moe_gate_up": (ctypes.c_int, [P, P, P, P, i32, i32, P, P, i64, i64, P, i64, P]),
            "orc_mx_moe_down": (ctypes.c_int, [P, P, P, i32, P, P, i64, i64, P, i64, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != OK:
        raise OracleError(rc, what)


def _u16(x):
    x = np.ascontiguousarray(x)
    assert x.dtype == np.uint16, "bf16 inputs are uint16 bit arrays"
    return x


# --------------------------------------------------------------------------
# scalar codecs
# --------------------------------------------------------------------------

def e2m1_value(nibble: int) -> float:
    return _load().orc_e2m1_value(nibble)


def e4m3_value(byte: int) -> float:
    return _load().orc_e4m3_value(byte)


def e8m0_value(byte: int) -> float:
    return _load().orc_e8m0_value(byte)


def e4m3_encode(s: float) -> int:
    return _load().orc_e4m3_encode(s)


def e2m1_encode(a: float) -> int:
    return _load().orc_e2m1_encode(a)


def bf16_from_double(v: float) -> int:
    return _load().orc_bf16_from_double(v)


def bf16_round_array(v: np.ndarray) -> np.ndarray:
    """Element-wise nearest-even bf16 of a float64 array (bits as uint16)."""
    f = _load().orc_bf16_from_double
    flat = np.asarray(v, dtype=np.float64).ravel()
    out = np.fromiter((f(float(t)) for t in flat), dtype=np.uint16, count=flat.size)
    return out.reshape(np.shape(v))


def global_from_amax(amax: float) -> float:
    return _load().orc_global_from_amax(amax)


def amax_bf16(x: np.ndarray) -> float:
    x = _u16(x)
    R, K = x.shape
    return _load().orc_amax_bf16(_p(x), R, K, K)


# --------------------------------------------------------------------------
# NVFP4 tensors
# --------------------------------------------------------------------------

class NVFP4:
    """packed u8 [R, K/2], scales u8 (E4M3 bytes) [R, K/16], global fp32."""

    def __init__(self, packed, scales, G):
        self.packed = packed
        self.scales = scales
        self.G = np.float32(G)

    @property
    def shape(self):
        return (self.packed.shape[0], self.packed.shape[1] * 2)

    def rows(self, r0, r1):
        return NVFP4(np.ascontiguousarray(self.packed[r0:r1]),
                     np.ascontiguousarray(self.scales[r0:r1]), self.G)


def quantize(x: np.ndarray, static_G: float | None = None) -> NVFP4:
    """NVFP4 quantization of a bf16 [R, K] matrix (see orc_quantize)."""
    x = _u16(x)
    R, K = x.shape
    packed = np.zeros((R, K // 2), np.uint8)
    scales = np.zeros((R, K // 16), np.uint8)
    G = np.zeros(1, np.float32)
    sg = None
    if static_G is not None:
        sg = np.array([static_G], np.float32)
    rc = _load().orc_quantize(_p(x), R, K, K, _p(sg) if sg is not None else None,
                              _p(packed), _p(scales), _p(G))
    _check(rc, "quantize")
    return NVFP4(packed, scales, G[0])


def dequantize(t: NVFP4, want_bf16: bool = False):
    R, K = t.shape
    out = np.zeros((R, K), np.float32)
    outb = np.zeros((R, K), np.uint16) if want_bf16 else None
    rc = _load().orc_dequantize(_p(t.packed), _p(t.scales), float(t.G), R, K, _p(out),
                                _p(outb) if outb is not None else None)
    _check(rc, "dequantize")
    return (out, outb) if want_bf16 else out


def gather_dequantize(t: NVFP4, ids, want_bf16: bool = False):
    """Row gather of an NVFP4 embedding table, then dequantize (page
    "Qwen3.8-Flash-Next-FP4-Local", section 2.1: rows of an NVFP4 n-gram
    table looked up per token).  An id outside [0, rows) gives a zero row.
    This is the definition written out: select the rows, dequantize them."""
    ids = np.asarray(ids, dtype=np.int64)
    R, K = t.shape
    ok = (ids >= 0) & (ids < R)
    src = np.where(ok, ids, 0)
    sub = NVFP4(np.ascontiguousarray(t.packed[src]), np.ascontiguousarray(t.scales[src]), t.G)
    res = dequantize(sub, want_bf16)
    for a in (res if want_bf16 else (res,)):
        a[~ok] = 0
    return res


def gemm_rows(A: NVFP4, W: NVFP4, a_rows=None, w_rows=None) -> np.ndarray:
    """Exact C = Ga*Gw*deq0(A[a_rows]) @ deq0(W[w_rows])^T as float64."""
    M, K = A.shape
    N, K2 = W.shape
    assert K == K2
    a_rows = np.arange(M, dtype=np.int64) if a_rows is None else np.ascontiguousarray(a_rows, np.int64)
    w_rows = np.arange(N, dtype=np.int64) if w_rows is None else np.ascontiguousarray(w_rows, np.int64)
    C = np.zeros((a_rows.size, w_rows.size), np.float64)
    rc = _load().orc_gemm_rows(_p(A.packed), _p(A.scales), float(A.G), _p(a_rows), a_rows.size,
                               _p(W.packed), _p(W.scales), float(W.G), _p(w_rows), w_rows.size,
                               K, _p(C))
    _check(rc, "gemm")
    return C


def gemm(A: NVFP4, W: NVFP4) -> np.ndarray:
    return gemm_rows(A, W)


def gemm_w4a16(a: np.ndarray, W: NVFP4, a_rows=None, w_rows=None) -> np.ndarray:
    """W4A16 C = Gw * a[a_rows] @ deq0(W[w_rows])^T as float64 (a: bf16 bits
    [M, K]; see orc_gemm_w4a16_rows)."""
    a = np.ascontiguousarray(_u16(a))
    M, K = a.shape
    N, K2 = W.shape
    assert K == K2
    a_rows = np.arange(M, dtype=np.int64) if a_rows is None else np.ascontiguousarray(a_rows, np.int64)
    w_rows = np.arange(N, dtype=np.int64) if w_rows is None else np.ascontiguousarray(w_rows, np.int64)
    C = np.zeros((a_rows.size, w_rows.size), np.float64)
    rc = _load().orc_gemm_w4a16_rows(_p(a), K, _p(a_rows), a_rows.size, _p(W.packed), _p(W.scales),
                                     float(W.G), _p(w_rows), w_rows.size, K, _p(C))
    _check(rc, "gemm_w4a16")
    return C


# --------------------------------------------------------------------------
# MXFP4
# --------------------------------------------------------------------------

def mxfp4_encode(x: np.ndarray):
    """OCP MXFP4 encode of a bf16 [R, K] matrix -> (packed [R,K/2], e8m0 [R,K/32])."""
    x = _u16(x)
    R, K = x.shape
    packed = np.zeros((R, K // 2), np.uint8)
    e8 = np.zeros((R, K // 32), np.uint8)
    _check(_load().orc_mxfp4_encode(_p(x), R, K, K, _p(packed), _p(e8)), "mxfp4_encode")
    return packed, e8


def mxfp4_dequantize(packed: np.ndarray, e8: np.ndarray) -> np.ndarray:
    packed = np.ascontiguousarray(packed)
    e8 = np.ascontiguousarray(e8)
    R = packed.shape[0]
    K = packed.shape[1] * 2
    out = np.zeros((R, K), np.float32)
    _check(_load().orc_mxfp4_dequantize(_p(packed), _p(e8), R, K, _p(out)), "mxfp4_dequantize")
    return out


def mxfp4_to_nvfp4(packed: np.ndarray, e8: np.ndarray) -> NVFP4:
    """Lossless remap of one MXFP4 tensor (raises OracleError(RANGE) past 17 octaves)."""
    packed = np.ascontiguousarray(packed)
    e8 = np.ascontiguousarray(e8)
    R = packed.shape[0]
    K = packed.shape[1] * 2
    out_p = np.zeros_like(packed)
    out_s = np.zeros((R, K // 16), np.uint8)
    G = np.zeros(1, np.float32)
    _check(_load().orc_mxfp4_to_nvfp4(_p(packed), _p(e8), R, K, _p(out_p), _p(out_s), _p(G)),
           "mxfp4_to_nvfp4")
    return NVFP4(out_p, out_s, G[0])


def mxfp8_encode(x: np.ndarray):
    """MXFP8 (E4M3, UE8M0 per 32) of bf16 bits [R, K] -> (codes [R, K], e8m0
    [R, K/32]) (see orc_mxfp8_encode)."""
    x = np.ascontiguousarray(_u16(x))
    R, K = x.shape
    q = np.zeros((R, K), np.uint8)
    e8 = np.zeros((R, K // 32), np.uint8)
    _check(_load().orc_mxfp8_encode(_p(x), R, K, K, _p(q), _p(e8)), "mxfp8_encode")
    return q, e8


def mx_gemm_w4a8(a: np.ndarray, a_e8: np.ndarray, w_packed: np.ndarray, w_e8: np.ndarray,
                 a_rows=None, w_rows=None) -> np.ndarray:
    """MX W4A8 C = A_mxfp8 @ W_mxfp4^T as float64 (see orc_mx_gemm_w4a8_rows)."""
    a, a_e8 = np.ascontiguousarray(a, np.uint8), np.ascontiguousarray(a_e8, np.uint8)
    w_packed, w_e8 = np.ascontiguousarray(w_packed, np.uint8), np.ascontiguousarray(w_e8, np.uint8)
    M, K = a.shape
    N = w_packed.shape[0]
    assert w_packed.shape[1] * 2 == K
    a_rows = np.arange(M, dtype=np.int64) if a_rows is None else np.ascontiguousarray(a_rows, np.int64)
    w_rows = np.arange(N, dtype=np.int64) if w_rows is None else np.ascontiguousarray(w_rows, np.int64)
    C = np.zeros((a_rows.size, w_rows.size), np.float64)
    _check(_load().orc_mx_gemm_w4a8_rows(_p(a), _p(a_e8), _p(a_rows), a_rows.size, _p(w_packed), _p(w_e8),
                                         _p(w_rows), w_rows.size, K, _p(C)), "mx_gemm_w4a8")
    return C


# --------------------------------------------------------------------------
# MoE routed experts
# --------------------------------------------------------------------------

def moe_route(ids: np.ndarray, E: int):
    ids = np.ascontiguousarray(ids, np.int32)
    T, k = ids.shape
    perm = np.zeros(T * k, np.int32)
    inv = np.zeros(T * k, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    _check(_load().orc_moe_route(_p(ids), T, k, E, _p(perm), _p(offsets), _p(inv)), "moe_route")
    return perm, offsets, inv


class Experts:
    """E stacked NVFP4 matrices: packed [E, R, K/2], scales [E, R, K/16], G [E]."""

    def __init__(self, packed, scales, G):
        self.packed = np.ascontiguousarray(packed)
        self.scales = np.ascontiguousarray(scales)
        self.G = np.ascontiguousarray(G, np.float32)

    @staticmethod
    def stack(tensors):
        return Experts(np.stack([t.packed for t in tensors]),
                       np.stack([t.scales for t in tensors]),
                       np.array([t.G for t in tensors], np.float32))

    def expert(self, e) -> NVFP4:
        return NVFP4(self.packed[e], self.scales[e], self.G[e])


def moe_gate_up(xq: NVFP4, perm, offsets, k: int, w13: Experts, rows) -> np.ndarray:
    """h (bf16 bits) [len(rows), I] for list positions ``rows`` (see orc_moe_gate_up)."""
    E = w13.G.size
    twoI, H = w13.packed.shape[1], w13.packed.shape[2] * 2
    I = twoI // 2
    rows = np.ascontiguousarray(rows, np.int64)
    h = np.zeros((rows.size, I), np.uint16)
    perm = np.ascontiguousarray(perm, np.int32)
    offsets = np.ascontiguousarray(offsets, np.int32)
    _check(_load().orc_moe_gate_up(_p(xq.packed), _p(xq.scales), float(xq.G), _p(perm),
                                   _p(offsets), k, E, _p(w13.packed), _p(w13.scales),
                                   _p(w13.G), H, I, _p(rows), rows.size, _p(h)), "moe_gate_up")
    return h


def moe_down(hq: NVFP4, offsets, w2: Experts, rows) -> np.ndarray:
    """y (float64) [len(rows), H] for list positions ``rows`` (see orc_moe_down)."""
    E = w2.G.size
    H, I = w2.packed.shape[1], w2.packed.shape[2] * 2
    rows = np.ascontiguousarray(rows, np.int64)
    y = np.zeros((rows.size, H), np.float64)
    offsets = np.ascontiguousarray(offsets, np.int32)
    _check(_load().orc_moe_down(_p(hq.packed), _p(hq.scales), float(hq.G), _p(offsets), E,
                                _p(w2.packed), _p(w2.scales), _p(w2.G), H, I, _p(rows),
                                rows.size, _p(y)), "moe_down")
    return y


def moe_combine(y: np.ndarray, inv, w: np.ndarray) -> np.ndarray:
    y = np.ascontiguousarray(y, np.float64)
    inv = np.ascontiguousarray(inv, np.int32)
    w = np.ascontiguousarray(w, np.float32)
    T, k = w.shape
    H = y.shape[1]
    out = np.zeros((T, H), np.uint16)
    _check(_load().orc_moe_combine(_p(y), _p(inv), _p(w), T, k, H, _p(out)), "moe_combine")
    return out


def moe_forward(x: np.ndarray, ids: np.ndarray, w: np.ndarray, w13: Experts, w2: Experts,
                static_in_globals=None):
    """Whole routed-expert MoE forward on bf16 x [T, H] (every step in order):
    route -> quantize x once -> gate_up + SwiGLU -> quantize h over all T*k
    rows -> down -> router-weighted combine.  Returns a dict of every
    intermediate (xq, perm, offsets, inv, h, hq, y, out)."""
    E = w13.G.size
    T, k = ids.shape
    perm, offsets, inv = moe_route(ids, E)
    gx = None if static_in_globals is None else static_in_globals[0]
    gh = None if static_in_globals is None else static_in_globals[1]
    xq = quantize(x, gx)
    rows = np.arange(T * k, dtype=np.int64)
    h = moe_gate_up(xq, perm, offsets, k, w13, rows)
    hq = quantize(h, gh)
    y = moe_down(hq, offsets, w2, rows)
    out = moe_combine(y, inv, w)
    return dict(xq=xq, perm=perm, offsets=offsets, inv=inv, h=h, hq=hq, y=y, out=out)


def moe_w4a16_gate_up(x: np.ndarray, perm, offsets, k: int, w13: Experts, rows) -> np.ndarray:
    """W4A16 h (bf16 bits) [len(rows), I] from the bf16 rows of x (see
    orc_moe_w4a16_gate_up)."""
    x = np.ascontiguousarray(_u16(x))
    E = w13.G.size
    twoI, H = w13.packed.shape[1], w13.packed.shape[2] * 2
    I = twoI // 2
    rows = np.ascontiguousarray(rows, np.int64)
    h = np.zeros((rows.size, I), np.uint16)
    _check(_load().orc_moe_w4a16_gate_up(_p(x), _p(np.ascontiguousarray(perm, np.int32)),
                                         _p(np.ascontiguousarray(offsets, np.int32)), k, E, _p(w13.packed),
                                         _p(w13.scales), _p(w13.G), H, I, _p(rows), rows.size, _p(h)),
           "moe_w4a16_gate_up")
    return h


def moe_w4a16_down(h: np.ndarray, offsets, w2: Experts, rows) -> np.ndarray:
    """W4A16 y (float64) [len(rows), H] from bf16 h rows in list order."""
    h = np.ascontiguousarray(_u16(h))
    E = w2.G.size
    H, I = w2.packed.shape[1], w2.packed.shape[2] * 2
    rows = np.ascontiguousarray(rows, np.int64)
    y = np.zeros((rows.size, H), np.float64)
    _check(_load().orc_moe_w4a16_down(_p(h), _p(np.ascontiguousarray(offsets, np.int32)), E, _p(w2.packed),
                                      _p(w2.scales), _p(w2.G), H, I, _p(rows), rows.size, _p(y)),
           "moe_w4a16_down")
    return y


def moe_w4a16_forward(x: np.ndarray, ids: np.ndarray, w: np.ndarray, w13: Experts, w2: Experts):
    """W4A16 routed-expert MoE forward on bf16 x [T, H] ("Qwen3.8-Flash-Next-
    FP4-Local", section 3.2): route -> gate_up + SwiGLU from the bf16 x rows
    -> down from the bf16 h rows -> router-weighted combine.  No activation
    is quantized.  Returns a dict of the intermediates (perm, offsets, inv,
    h, y, out)."""
    E = w13.G.size
    T, k = ids.shape
    perm, offsets, inv = moe_route(ids, E)
    rows = np.arange(T * k, dtype=np.int64)
    h = moe_w4a16_gate_up(x, perm, offsets, k, w13, rows)
    y = moe_w4a16_down(h, offsets, w2, rows)
    out = moe_combine(y, inv, w)
    return dict(perm=perm, offsets=offsets, inv=inv, h=h, y=y, out=out)


# --------------------------------------------------------------------------
# NVFP4 KV cache
# --------------------------------------------------------------------------

def kv_write(cache: NVFP4, chunk: np.ndarray, tok_offset: int, G: float):
    """Quantize a bf16 chunk [n, Hkv, D] with the static global G and store its
    rows (token, head) at token offset tok_offset of a cache whose rows are
    (token, head) pairs, D columns."""
    n, Hkv, D = chunk.shape
    q = quantize(np.ascontiguousarray(chunk.reshape(n * Hkv, D)), G)
    r0 = tok_offset * Hkv
    cache.packed[r0:r0 + n * Hkv] = q.packed
    cache.scales[r0:r0 + n * Hkv] = q.scales
    cache.G = np.float32(G)


def kv_empty(tokens: int, Hkv: int, D: int) -> NVFP4:
    return NVFP4(np.zeros((tokens * Hkv, D // 2), np.uint8),
                 np.zeros((tokens * Hkv, D // 16), np.uint8), 1.0)


# --------------------------------------------------------------------------
# scale audit
# --------------------------------------------------------------------------

def audit_scales(t: NVFP4) -> dict:
    """Counts over the E4M3 scale bytes: total, non-finite (NaN pattern),
    non-positive (zero or sign set), at the maximum 448 (0x7E)."""
    s = t.scales.ravel()
    nan = int(np.count_nonzero((s & 0x7F) == 0x7F))
    nonpos = int(np.count_nonzero((s == 0) | ((s & 0x80) != 0)))
    return dict(total=int(s.size), nonfinite=nan, nonpositive=nonpos,
                at_max=int(np.count_nonzero(s == 0x7E)))


# --------------------------------------------------------------------------
# 128-row tiled storage order of the scale bytes (a storage order of the
# library's own, not a page's: the pages fix one E4M3 scale per 16 elements
# along the last dimension, not where the bytes live)
# --------------------------------------------------------------------------

def tile_scales(scales: np.ndarray) -> np.ndarray:
    """Scale bytes [batch, rows, cols/16] (row-major) -> the flat tiled
    order: byte b of row r of matrix m goes to
    m*rows*cols/16 + ((r//128 * cols/256 + b//16) * 128 + r%128) * 16 + b%16."""
    s = np.asarray(scales, np.uint8)
    if s.ndim == 2:
        s = s[None]
    B, R, NB = s.shape
    if R % 128 or NB % 16:
        raise OracleError(SHAPE, "tile_scales")
    # [m, tile, rr, chunk, j] -> [m, tile, chunk, rr, j]
    t = s.reshape(B, R // 128, 128, NB // 16, 16).transpose(0, 1, 3, 2, 4)
    return np.ascontiguousarray(t).reshape(-1)


# --------------------------------------------------------------------------
# MX-native W4A8 routed experts (MXFP4 experts, MXFP8 activations)
# --------------------------------------------------------------------------

def mx_moe_gate_up(xq, xe, perm, offsets, k: int, w13p, w13e, rows) -> np.ndarray:
    """h (bf16 bits) [len(rows), I] for list positions ``rows``: x MXFP8
    (codes [T, H], e8m0 [T, H/32]), w13 MXFP4 (codes [E, 2I, H/2], e8m0
    [E, 2I, H/32]) (see orc_mx_moe_gate_up)."""
    xq, xe = np.ascontiguousarray(xq, np.uint8), np.ascontiguousarray(xe, np.uint8)
    w13p, w13e = np.ascontiguousarray(w13p, np.uint8), np.ascontiguousarray(w13e, np.uint8)
    E, twoI, H = w13p.shape[0], w13p.shape[1], w13p.shape[2] * 2
    I = twoI // 2
    rows = np.ascontiguousarray(rows, np.int64)
    h = np.zeros((rows.size, I), np.uint16)
    _check(_load().orc_mx_moe_gate_up(_p(xq), _p(xe), _p(np.ascontiguousarray(perm, np.int32)),
                                      _p(np.ascontiguousarray(offsets, np.int32)), k, E, _p(w13p), _p(w13e),
                                      H, I, _p(rows), rows.size, _p(h)), "mx_moe_gate_up")
    return h


def mx_moe_down(hq, he, offsets, w2p, w2e, rows) -> np.ndarray:
    """y (float64) [len(rows), H] for list positions ``rows``: h MXFP8 in list
    order (codes [T*k, I], e8m0 [T*k, I/32]), w2 MXFP4 (codes [E, H, I/2],
    e8m0 [E, H, I/32]) (see orc_mx_moe_down)."""
    hq, he = np.ascontiguousarray(hq, np.uint8), np.ascontiguousarray(he, np.uint8)
    w2p, w2e = np.ascontiguousarray(w2p, np.uint8), np.ascontiguousarray(w2e, np.uint8)
    E, H, I = w2p.shape[0], w2p.shape[1], w2p.shape[2] * 2
    rows = np.ascontiguousarray(rows, np.int64)
    y = np.zeros((rows.size, H), np.float64)
    _check(_load().orc_mx_moe_down(_p(hq), _p(he), _p(np.ascontiguousarray(offsets, np.int32)), E, _p(w2p),
                                   _p(w2e), H, I, _p(rows), rows.size, _p(y)), "mx_moe_down")
    return y


def mx_moe_forward(x: np.ndarray, ids: np.ndarray, w: np.ndarray, w13p, w13e, w2p, w2e):
    """Whole MX W4A8 routed-expert forward on bf16 x [T, H]: route -> x to
    MXFP8 -> gate_up + SwiGLU -> h to MXFP8 (list order) -> down -> combine.
    Returns every intermediate (xq, xe, perm, offsets, inv, h, hq, he, y, out)."""
    E = w13p.shape[0]
    T, k = ids.shape
    perm, offsets, inv = moe_route(ids, E)
    xq, xe = mxfp8_encode(x)
    rows = np.arange(T * k, dtype=np.int64)
    h = mx_moe_gate_up(xq, xe, perm, offsets, k, w13p, w13e, rows)
    hq, he = mxfp8_encode(h)
    y = mx_moe_down(hq, he, offsets, w2p, w2e, rows)
    out = moe_combine(y, inv, w)
    return dict(xq=xq, xe=xe, perm=perm, offsets=offsets, inv=inv, h=h, hq=hq, he=he, y=y, out=out)
