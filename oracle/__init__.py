"""CPU oracle for the scaled FP8 down-projection path (ctypes over oracle.c).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with ``scaled_quantization_amd`` and never imports it.

Every function here is a thin numpy wrapper around the plain single-threaded C
definitions in ``oracle.c``; the page and section each rule follows is cited
there.  Parity status of each function is listed in ``PINNED`` below: each is
pinned by a test under ``tests/`` against values the pages print, closed
forms, library routines or brute force.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

E4M3, E5M2 = 0, 1
ACT_IDENTITY, ACT_RELU2 = 0, 1
PER_TENSOR, PER_GROUP128 = 0, 1
GROUP = 128
MAX_HIST = 16
FMT_MAX = {E4M3: 448.0, E5M2: 57344.0}

# Which oracle function is pinned by which independent check (see tests/).
PINNED = {
    "fp8_decode": "page format facts + closed form + torch float8 decode (all 256 codes)",
    "fp8_encode": "nearest-neighbour search over the decode table at every rounding boundary "
                  "+ torch float8 cast on clamped inputs",
    "fp8_saturates": "torch non-saturating float8 cast returns non-finite",
    "bf16_rne": "torch bfloat16 cast (boundaries + random) + the 1/3 worked example",
    "scale_from_amax": "amax 3.2 -> 140 and amax 0.8 -> 560 worked examples; Python float32 division",
    "quantize": "worked outlier experiment (16.24% zeroed, 12.78% / 3.41% RMSE); numpy brute force",
    "state/history": "closed-form delayed recurrence on the tiny workload",
    "quantize_weight_blocks": "brute force composition per block (numpy + nearest-code search)",
    "gemm_f64": "exact rational arithmetic (fractions) on small cases; identity and constant cases",
    "relu2_backward": "chain rule against torch autograd of relu(h)^2 in float64 within the "
                      "formats' error bound (BF16 and FP8 caches); exact squares; signed zeros; "
                      "E5M2 codes by nearest-code search; amax and saturation by numpy/torch",
    "mx_exponent": "closed form from the BF16 exponent and fraction bits at every BF16 magnitude; "
                   "minimality and no-overflow invariants",
    "quantize_mx": "nearest-code search over the decode table of b / 2^k with an independently "
                   "computed k (pure Python); block locality; zero, infinity and NaN blocks",
    "gemm_mx_f64": "float64 matmul of the dequantized operands; exact rational arithmetic on a "
                   "small case; error bound against the unquantized product",
}

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB names another build of oracle.c (the mutation test loads copies
# with planted mistakes this way, each in a process of its own).
_LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_u64p = ctypes.POINTER(ctypes.c_uint64)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


class _State(ctypes.Structure):
    _fields_ = [
        ("scale", ctypes.c_float),
        ("scale_inv", ctypes.c_float),
        ("scale_inv_used", ctypes.c_float),
        ("amax_acc", ctypes.c_uint32),
        ("sat_acc", ctypes.c_uint64),
        ("sat_last", ctypes.c_uint64),
        ("overflow", ctypes.c_uint32),
        ("margin", ctypes.c_float),
        ("hist_len", ctypes.c_int32),
        ("hist_pos", ctypes.c_int32),
        ("steps", ctypes.c_uint32),
        ("fmt", ctypes.c_int32),
        ("history", ctypes.c_float * MAX_HIST),
    ]


def lib() -> ctypes.CDLL:
    """Load liboracle.so, compiling it first only if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    L = ctypes.CDLL(_LIB_PATH)
    L.oracle_fp8_decode.restype = ctypes.c_double
    L.oracle_fp8_decode.argtypes = [ctypes.c_uint8, ctypes.c_int]
    L.oracle_fp8_encode.restype = ctypes.c_uint8
    L.oracle_fp8_encode.argtypes = [ctypes.c_float, ctypes.c_int]
    L.oracle_bf16_rne.restype = ctypes.c_uint16
    L.oracle_bf16_rne.argtypes = [ctypes.c_float]
    L.oracle_scale_from_amax.restype = ctypes.c_float
    L.oracle_scale_from_amax.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_int]
    L.oracle_recip_f32.restype = ctypes.c_float
    L.oracle_recip_f32.argtypes = [ctypes.c_float]
    L.oracle_quantize.restype = None
    L.oracle_quantize.argtypes = [_u16p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_float, _u16p, _u8p, _f32p, _f32p, _u32p,
                                  _u64p]
    L.oracle_state_size.restype = ctypes.c_int64
    L.oracle_state_init.restype = ctypes.c_int
    L.oracle_state_init.argtypes = [ctypes.POINTER(_State), ctypes.c_int, ctypes.c_int,
                                    ctypes.c_float, ctypes.c_float]
    L.oracle_history_update.restype = None
    L.oracle_history_update.argtypes = [ctypes.POINTER(_State)]
    L.oracle_state_accumulate.restype = None
    L.oracle_state_accumulate.argtypes = [ctypes.POINTER(_State), ctypes.c_uint32, ctypes.c_uint64]
    L.oracle_gemm_f64.restype = None
    L.oracle_gemm_f64.argtypes = [_u8p, ctypes.c_int, _u8p, ctypes.c_int, ctypes.c_int64,
                                  ctypes.c_int64, ctypes.c_int64, ctypes.c_int, _f32p, _f32p,
                                  _i64p, ctypes.c_int64, _f64p, _f64p]
    L.oracle_gemm_bf16_f64.restype = None
    L.oracle_gemm_bf16_f64.argtypes = [_u16p, _u16p, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, _i64p, ctypes.c_int64, _f64p, _f64p]
    L.oracle_fp8_encode_batch.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int, _u8p]
    L.oracle_fp8_saturates_batch.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int, _u8p]
    L.oracle_bf16_rne_batch.argtypes = [_f32p, ctypes.c_int64, _u16p]
    L.oracle_scale_batch.argtypes = [_f32p, ctypes.c_int64, ctypes.c_float, ctypes.c_int, _f32p,
                                     _f32p]
    L.oracle_quantize_weight_blocks.restype = None
    L.oracle_quantize_weight_blocks.argtypes = [_u16p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                                _u8p, _f32p, _f32p]
    L.oracle_fp8_encode_range.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int, _u8p]
    L.oracle_bf16_rne_range.argtypes = [ctypes.c_uint64, ctypes.c_uint64, _u16p]
    L.oracle_relu2_backward.argtypes = [_u16p, ctypes.c_void_p, ctypes.c_int, ctypes.c_float,
                                        ctypes.c_int64, ctypes.c_int, ctypes.c_float, _u16p, _u8p,
                                        _u32p, _u64p]
    L.oracle_mx_exponent.argtypes = [ctypes.c_double, ctypes.c_int, ctypes.c_int]
    L.oracle_mx_exponent.restype = ctypes.c_int
    L.oracle_quantize_mx.argtypes = [_u16p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                     ctypes.c_int, _u16p, _u8p, _u8p]
    L.oracle_gemm_mx_f64.argtypes = [_u8p, ctypes.c_int, _u8p, _u8p, ctypes.c_int, _u8p,
                                     ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _i64p,
                                     ctypes.c_int64, _f64p, _f64p]
    if L.oracle_state_size() != ctypes.sizeof(_State):
        raise RuntimeError("oracle_state layout mismatch between oracle.c and its wrapper")
    _lib = L
    return L


def _ptr(a: Optional[np.ndarray], typ):
    if a is None:
        return ctypes.cast(None, typ)
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(typ)


# --------------------------------------------------------------------------- formats
def fp8_decode_table(fmt: int) -> np.ndarray:
    """Float64 value of each of the 256 codes of ``fmt`` (NaN for NaN codes)."""
    L = lib()
    return np.array([L.oracle_fp8_decode(c, fmt) for c in range(256)], dtype=np.float64)


def fp8_encode(x, fmt: int) -> np.ndarray:
    """Saturating round-to-nearest-even cast of float32 values to FP8 codes."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(x.shape, dtype=np.uint8)
    lib().oracle_fp8_encode_batch(_ptr(x, _f32p), x.size, fmt, _ptr(out, _u8p))
    return out


def fp8_saturates(x, fmt: int) -> np.ndarray:
    """True where a non-saturating cast of the float32 value would overflow."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(x.shape, dtype=np.uint8)
    lib().oracle_fp8_saturates_batch(_ptr(x, _f32p), x.size, fmt, _ptr(out, _u8p))
    return out.astype(bool)


def bf16_rne(x) -> np.ndarray:
    """Round float32 values to BF16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_bf16_rne_batch(_ptr(x, _f32p), x.size, _ptr(out, _u16p))
    return out


def bf16_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def scale_from_amax(amax, margin: float, fmt: int):
    """(scale, scale_inv) in float32 for each amax: scale = max / (amax * margin)."""
    a = np.ascontiguousarray(np.atleast_1d(np.asarray(amax, dtype=np.float32)))
    s = np.empty_like(a)
    si = np.empty_like(a)
    lib().oracle_scale_batch(_ptr(a, _f32p), a.size, margin, fmt, _ptr(s, _f32p), _ptr(si, _f32p))
    return s, si


def fp8_encode_range(lo: int, hi: int, fmt: int) -> np.ndarray:
    """Codes for every float32 bit pattern u in [lo, hi)."""
    out = np.empty(hi - lo, dtype=np.uint8)
    lib().oracle_fp8_encode_range(lo, hi, fmt, _ptr(out, _u8p))
    return out


def bf16_rne_range(lo: int, hi: int) -> np.ndarray:
    out = np.empty(hi - lo, dtype=np.uint16)
    lib().oracle_bf16_rne_range(lo, hi, _ptr(out, _u16p))
    return out


# --------------------------------------------------------------------------- quantize
@dataclass
class QuantResult:
    bf16: Optional[np.ndarray]        # uint16 [rows, cols] (activation copy) or None
    fp8: Optional[np.ndarray]         # uint8 [rows, cols] or None
    group_scale_inv: Optional[np.ndarray]  # float32 [rows, cols/128] (group mode) or None
    amax_bits: int                    # binary32 bits of max |b|
    sat: int                          # saturating element count
    group_scale: Optional[np.ndarray] = None  # the multipliers s_g themselves (group mode)

    @property
    def amax(self) -> float:
        return float(np.array([self.amax_bits], dtype=np.uint32).view(np.float32)[0])


def quantize(h: np.ndarray, act: int, fmt: int, mode: int, scale: float = 1.0,
             want_bf16: bool = True, want_fp8: bool = True) -> QuantResult:
    """One quantization call over a row-major uint16 (BF16 bits) [rows, cols] array."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    if h.ndim == 1:
        h = h.reshape(1, -1)
    rows, cols = h.shape
    if mode == PER_GROUP128 and cols % GROUP:
        raise ValueError("group mode needs cols % 128 == 0")
    bf = np.empty_like(h) if want_bf16 else None
    q = np.empty(h.shape, dtype=np.uint8) if want_fp8 else None
    gsi = np.empty((rows, cols // GROUP), dtype=np.float32) if mode == PER_GROUP128 else None
    gs = np.empty((rows, cols // GROUP), dtype=np.float32) if mode == PER_GROUP128 else None
    amax = ctypes.c_uint32(0)
    sat = ctypes.c_uint64(0)
    lib().oracle_quantize(_ptr(h, _u16p), rows, cols, act, fmt, mode, scale, _ptr(bf, _u16p),
                          _ptr(q, _u8p), _ptr(gsi, _f32p), _ptr(gs, _f32p), ctypes.byref(amax),
                          ctypes.byref(sat))
    return QuantResult(bf, q, gsi, int(amax.value), int(sat.value), gs)


def quantize_weight_blocks(w: np.ndarray, fmt: int, with_scale: bool = False):
    """128 x 128-block current-scaled cast of a BF16 [N, K] weight: (codes, scale_inv)
    or, with_scale=True, (codes, scale_inv, scale)."""
    w = np.ascontiguousarray(w, dtype=np.uint16)
    N, K = w.shape
    if N % GROUP or K % GROUP:
        raise ValueError("weight blocks need N % 128 == 0 and K % 128 == 0")
    q = np.empty_like(w, dtype=np.uint8)
    si = np.empty((N // GROUP, K // GROUP), dtype=np.float32)
    sc = np.empty((N // GROUP, K // GROUP), dtype=np.float32)
    lib().oracle_quantize_weight_blocks(_ptr(w, _u16p), N, K, fmt, _ptr(q, _u8p), _ptr(si, _f32p),
                                        _ptr(sc, _f32p))
    return (q, si, sc) if with_scale else (q, si)


def quantize_weight_tensor(w: np.ndarray, fmt: int):
    """Per-tensor current-scaled cast of a BF16 weight: (codes, scale, scale_inv)."""
    amax = quantize(w, ACT_IDENTITY, fmt, PER_TENSOR, 1.0, want_bf16=False, want_fp8=False).amax
    s, si = scale_from_amax(amax, 1.0, fmt)
    r = quantize(w, ACT_IDENTITY, fmt, PER_TENSOR, float(s[0]), want_bf16=False)
    return r.fp8, float(s[0]), float(si[0])


# --------------------------------------------------------------------------- activation backward
CACHE_BF16 = 2


def relu2_backward(dA: np.ndarray, cache: np.ndarray, cache_kind: int, a_scale_inv: float,
                   fmt: int, scale: float) -> QuantResult:
    """dH = bf16(dA * 2 sqrt(a)) from the cached activation (BF16 bits when
    cache_kind == CACHE_BF16, else FP8 codes of format cache_kind with their
    inverse scale), cast to `fmt` with `scale`.  Returns a QuantResult
    (bf16 = dH copy, fp8 = codes, amax_bits, sat)."""
    dA = np.ascontiguousarray(dA, dtype=np.uint16)
    shape = dA.shape
    if cache_kind == CACHE_BF16:
        cache = np.ascontiguousarray(cache, dtype=np.uint16)
    else:
        cache = np.ascontiguousarray(cache, dtype=np.uint8)
    assert cache.shape == shape
    n = dA.size
    bf = np.empty(shape, dtype=np.uint16)
    q = np.empty(shape, dtype=np.uint8)
    amax = ctypes.c_uint32(0)
    sat = ctypes.c_uint64(0)
    lib().oracle_relu2_backward(_ptr(dA, _u16p), cache.ctypes.data, cache_kind, a_scale_inv, n,
                                fmt, scale, _ptr(bf, _u16p), _ptr(q, _u8p), ctypes.byref(amax),
                                ctypes.byref(sat))
    return QuantResult(bf, q, None, int(amax.value), int(sat.value))


# --------------------------------------------------------------------------- MXFP8
MX_BLOCK = 32


def mx_exponent(amax: float, nonfinite: bool, fmt: int) -> int:
    """Exponent k of an MXFP8 block's decode scale 2^k (E8M0 byte k + 127)."""
    return int(lib().oracle_mx_exponent(float(amax), int(bool(nonfinite)), fmt))


@dataclass
class MXResult:
    bf16: Optional[np.ndarray]    # uint16 [rows, cols] activation copy or None
    fp8: Optional[np.ndarray]     # uint8 [rows, cols] codes or None
    scale: np.ndarray             # uint8 [rows, cols/32] E8M0 bytes (decode scale 2^(e - 127))


def quantize_mx(h: np.ndarray, act: int, fmt: int, want_bf16: bool = True,
                want_fp8: bool = True) -> MXResult:
    """MXFP8 cast of a row-major uint16 (BF16 bits) [rows, cols] array, cols % 32 == 0."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    if h.ndim == 1:
        h = h.reshape(1, -1)
    rows, cols = h.shape
    if cols % MX_BLOCK:
        raise ValueError("MXFP8 needs cols % 32 == 0")
    bf = np.empty_like(h) if want_bf16 else None
    q = np.empty(h.shape, dtype=np.uint8) if want_fp8 else None
    e = np.empty((rows, cols // MX_BLOCK), dtype=np.uint8)
    lib().oracle_quantize_mx(_ptr(h, _u16p), rows, cols, act, fmt, _ptr(bf, _u16p),
                             _ptr(q, _u8p), _ptr(e, _u8p))
    return MXResult(bf, q, e)


def gemm_mx_f64(a: np.ndarray, fa: int, ea: np.ndarray, b: np.ndarray, fb: int, eb: np.ndarray,
                rows: Optional[Sequence[int]] = None):
    """Float64 reference of the MXFP8 GEMM y = a b^T with E8M0 block scales ea [M, K/32],
    eb [N, K/32].  Returns (ref, absref), each float64 [len(rows) or M, N]."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    ea = np.ascontiguousarray(ea, dtype=np.uint8)
    eb = np.ascontiguousarray(eb, dtype=np.uint8)
    M, K = a.shape
    N, K2 = b.shape
    assert K == K2 and K % MX_BLOCK == 0
    assert ea.size == M * (K // MX_BLOCK) and eb.size == N * (K // MX_BLOCK)
    r = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    cnt = M if r is None else r.size
    ref = np.empty((cnt, N), dtype=np.float64)
    absref = np.empty((cnt, N), dtype=np.float64)
    lib().oracle_gemm_mx_f64(_ptr(a, _u8p), fa, _ptr(ea, _u8p), _ptr(b, _u8p), fb, _ptr(eb, _u8p),
                             M, N, K, _ptr(r, _i64p), 0 if r is None else r.size,
                             _ptr(ref, _f64p), _ptr(absref, _f64p))
    return ref, absref


class State:
    """Delayed-scaling state (history ring, next scale, accumulators)."""

    def __init__(self, fmt: int, hist_len: int = 1, margin: float = 1.25,
                 initial_amax: float = 1.0):
        self._s = _State()
        rc = lib().oracle_state_init(ctypes.byref(self._s), fmt, hist_len, margin, initial_amax)
        if rc != 0:
            raise ValueError("hist_len out of range")

    def accumulate(self, amax_bits: int, sat: int) -> None:
        lib().oracle_state_accumulate(ctypes.byref(self._s), amax_bits, sat)

    def update(self) -> None:
        lib().oracle_history_update(ctypes.byref(self._s))

    def __getattr__(self, name):
        if name.startswith("_"):
            raise AttributeError(name)
        v = getattr(self._s, name)
        if name == "history":
            return np.array(list(v)[: self._s.hist_len], dtype=np.float32)
        return v

    def as_dict(self) -> dict:
        d = {f: getattr(self, f) for f, _ in _State._fields_}
        return d


# --------------------------------------------------------------------------- GEMM
def gemm_bf16_f64(x: np.ndarray, w: np.ndarray, rows: Optional[Sequence[int]] = None):
    """Float64 reference of Y = X W^T over BF16 inputs (bit patterns, uint16):
    x [M, K], w [N, K].  Returns (ref, absref), each float64 [len(rows) or M, N]."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.uint16)
    M, K = x.shape
    N, K2 = w.shape
    assert K == K2
    r = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    cnt = M if r is None else r.size
    ref = np.empty((cnt, N), dtype=np.float64)
    absref = np.empty((cnt, N), dtype=np.float64)
    lib().oracle_gemm_bf16_f64(_ptr(x, _u16p), _ptr(w, _u16p), M, N, K, _ptr(r, _i64p),
                               0 if r is None else r.size, _ptr(ref, _f64p), _ptr(absref, _f64p))
    return ref, absref


def gemm_f64(a: np.ndarray, fa: int, b: np.ndarray, fb: int, mode: int, sa, sb,
             rows: Optional[Sequence[int]] = None):
    """Float64 reference of the scaled FP8 GEMM.

    a: uint8 [M, K]; b: uint8 [N, K]; sa/sb are the cast MULTIPLIERS (scales),
    scalars for PER_TENSOR, [M, K/128] and [N/128, K/128] for PER_GROUP128.
    Returns (ref, absref), each float64 [len(rows) or M, N].
    """
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    M, K = a.shape
    N, K2 = b.shape
    assert K == K2
    sa = np.ascontiguousarray(np.atleast_1d(np.asarray(sa, dtype=np.float32)))
    sb = np.ascontiguousarray(np.atleast_1d(np.asarray(sb, dtype=np.float32)))
    if mode == PER_GROUP128:
        assert sa.size == M * (K // GROUP) and sb.size == (N // GROUP) * (K // GROUP)
    r = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    cnt = M if r is None else r.size
    ref = np.empty((cnt, N), dtype=np.float64)
    absref = np.empty((cnt, N), dtype=np.float64)
    lib().oracle_gemm_f64(_ptr(a, _u8p), fa, _ptr(b, _u8p), fb, M, N, K, mode, _ptr(sa, _f32p),
                          _ptr(sb, _f32p), _ptr(r, _i64p), 0 if r is None else r.size,
                          _ptr(ref, _f64p), _ptr(absref, _f64p))
    return ref, absref
