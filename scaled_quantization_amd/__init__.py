"""scaled_quantization_amd -- scaled FP8 quantization for an MLP down-projection on MI355X.

A thin ctypes binding over ``libfp8dp.so`` (C ABI declared in
``include/fp8dp.h``).  Every step of the path runs in the library's HIP
kernels; this module only marshals torch device tensors into pointers, sizes
and the current HIP stream, and turns nonzero return codes into exceptions.
It raises if the library has not been built; there is no CPU fallback.

Entry points (same names as the C ABI):
    fp8dp_state_init, quantize_fused, amax_history_update, quantize_fused_update,
    fp8_gemm_scaled, quantize_weight, gemm_bf16_quantize_fused, fp8_gemm_scaled_splitk,
    fp8_gemm_scaled_splitk_noalloc, fp8_transpose, quantize_fused_transposed,
    quantize_mx, quantize_mx_transposed, fp8_gemm_mx, fp8_gemm_mx_splitk, and the
    comparison / diagnostic calls fp8dp_bench_*, fp8dp_convert_f32, fp8dp_scale_rule,
    fp8dp_set_grid_limit, fp8dp_set_codec.
"""
from __future__ import annotations

import ctypes
import math
import os
import struct
from typing import Optional, Union

import torch

E4M3, E5M2 = 0, 1
ACT_IDENTITY, ACT_RELU2 = 0, 1
PER_TENSOR, PER_GROUP128 = 0, 1
ACCUM_MFMA_FP8, ACCUM_EXACT = 0, 1
MAX_HIST = 16
ACC_SLOTS = 64
STATE_BYTES = 4288

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8dp.so")
_lib: Optional[ctypes.CDLL] = None

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_f32 = ctypes.c_float

_SIGS = {
    "fp8dp_state_size": ([], _i64),
    "fp8dp_state_init": ([_vp, _i32, _i32, _f32, _f32, _vp], ctypes.c_int),
    "quantize_fused": ([_vp, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "amax_history_update": ([_vp, _vp], ctypes.c_int),
    "quantize_fused_update": ([_vp, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _vp], ctypes.c_int),
    "fp8_gemm_scaled": ([_vp, _i32, _vp, _i32, _i64, _i64, _i64, _i32, _i32, _vp, _vp, _vp,
                         _vp], ctypes.c_int),
    "quantize_weight": ([_vp, _i64, _i64, _i32, _i32, _vp, _vp, _vp], ctypes.c_int),
    "fp8_gemm_scaled_splitk": ([_vp, _i32, _vp, _i32, _i64, _i64, _i64, _i32, _i32, _vp, _vp,
                                _vp, _vp, _vp], ctypes.c_int),
    "fp8_gemm_scaled_splitk_noalloc": ([_vp, _i32, _vp, _i32, _i64, _i64, _i64, _i32, _i32,
                                        _vp, _vp, _vp, _vp], ctypes.c_int),
    "fp8_transpose": ([_vp, _i64, _i64, _vp, _vp], ctypes.c_int),
    "quantize_fused_transposed": ([_vp, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp],
                                  ctypes.c_int),
    "quantize_mx_transposed": ([_vp, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _vp], ctypes.c_int),
    "fp8_gemm_mx_splitk": ([_vp, _i32, _vp, _vp, _i32, _vp, _i64, _i64, _i64, _i32, _i32, _vp,
                            _vp, _vp], ctypes.c_int),
    "relu2_backward_quantize": ([_vp, _vp, _i32, _vp, _i64, _i64, _i32, _vp, _vp, _vp, _vp],
                                ctypes.c_int),
    "fp8_gemm_relu2_backward": ([_vp, _i32, _vp, _i32, _i64, _i64, _i64, _i32, _vp, _vp, _vp,
                                 _i32, _vp, _i32, _vp, _vp, _vp], ctypes.c_int),
    "quantize_recompute": ([_vp, _i64, _i64, _i32, _i32, _vp, _vp, _vp], ctypes.c_int),
    "fp8_gemm_scaled_if": ([_vp, _i32, _vp, _i32, _i64, _i64, _i64, _i32, _vp, _vp, _vp, _vp,
                            _vp], ctypes.c_int),
    "quantize_mx": ([_vp, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _vp], ctypes.c_int),
    "fp8_gemm_mx": ([_vp, _i32, _vp, _vp, _i32, _vp, _i64, _i64, _i64, _i32, _vp, _vp],
                    ctypes.c_int),
    "gemm_bf16_quantize_fused": ([_vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _vp,
                                  _vp], ctypes.c_int),
    "fp8dp_last_error": ([], ctypes.c_char_p),
    "fp8dp_bench_act_bf16": ([_vp, _i64, _i32, _vp, _vp], ctypes.c_int),
    "fp8dp_bench_amax": ([_vp, _i64, _vp, _vp], ctypes.c_int),
    "fp8dp_bench_cast": ([_vp, _i64, _i32, _vp, _vp, _vp], ctypes.c_int),
    "fp8dp_bench_copy": ([_vp, _vp, _i64, _vp], ctypes.c_int),
    "fp8dp_convert_f32": ([_vp, _i64, _i32, _vp, _vp], ctypes.c_int),
    "fp8dp_scale_rule": ([_vp, _i64, _f32, _i32, _vp, _vp, _vp], ctypes.c_int),
    "fp8dp_set_grid_limit": ([_i32], _i32),
    "fp8dp_set_codec": ([_i32], _i32),
}


class Fp8dpError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """Load libfp8dp.so.  Raises if it has not been built (no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise Fp8dpError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH)
    for name, (args, res) in _SIGS.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    if L.fp8dp_state_size() != STATE_BYTES:
        raise Fp8dpError("fp8dp_tensor_state size differs from the binding's layout")
    _lib = L
    return L


def _check(rc: int, name: str) -> None:
    if rc != 0:
        msg = lib().fp8dp_last_error().decode(errors="replace")
        raise Fp8dpError(f"{name} failed ({rc}): {msg}")


# The current device and its current stream's raw handle without building a
# torch.cuda.Stream object (that object costs about 3 us per call, half of a
# call's host time).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_current_device = getattr(torch._C, "_cuda_getDevice", None) or torch.cuda.current_device


def _stream(stream) -> int:
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(_current_device())
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


Ptr = Union[torch.Tensor, int, None]


def _p(t: Ptr) -> Optional[int]:
    """Device address of a tensor (must be on a GPU and contiguous) or a raw int."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise Fp8dpError("expected a device tensor")
    if not t.is_contiguous():
        raise Fp8dpError("expected a contiguous tensor")
    # the kernels run on the current device's stream: a tensor elsewhere would
    # be read or written across devices
    if t.get_device() != _current_device():
        raise Fp8dpError(f"tensor on device {t.get_device()}, the current device is "
                         f"{_current_device()}: make its device current first")
    return t.data_ptr()


# --------------------------------------------------------------------------- state
# Field offsets of fp8dp_tensor_state (include/fp8dp.h).
_HDR = struct.Struct("<fffIQffiiIi16f")          # 112 bytes of header fields
_SLOT = struct.Struct("<IIQ48x")                 # 64-byte accumulator slot
_OFF = {"scale": 0, "scale_inv": 4, "scale_inv_used": 8, "overflow": 12, "ticket": 112,
        "acc": 192}


class TensorState:
    """Device-resident delayed-scaling state (a uint8 tensor of STATE_BYTES)."""

    def __init__(self, fmt: int = E4M3, hist_len: int = 1, margin: float = 1.25,
                 initial_amax: float = 1.0, device="cuda", stream=None):
        self.buf = torch.empty(STATE_BYTES, dtype=torch.uint8, device=device)
        self.fmt = fmt
        fp8dp_state_init(self, fmt, hist_len, margin, initial_amax, stream)

    @property
    def ptr(self) -> int:
        return self.buf.data_ptr()

    def field_ptr(self, name: str) -> int:
        return self.ptr + _OFF[name]

    def read(self) -> dict:
        """Copy the state to the host and decode it (synchronizes the stream)."""
        raw = self.buf.cpu().numpy().tobytes()
        f = _HDR.unpack_from(raw, 0)
        d = dict(scale=f[0], scale_inv=f[1], scale_inv_used=f[2], overflow=f[3], sat_last=f[4],
                 amax_last=f[5], margin=f[6], hist_len=f[7], hist_pos=f[8], steps=f[9],
                 fmt=f[10], history=list(f[11:11 + MAX_HIST]))
        amax_acc, sat_acc, tickets = 0, 0, 0
        for i in range(ACC_SLOTS):
            a, t, s = _SLOT.unpack_from(raw, _OFF["acc"] + 64 * i)
            amax_acc = max(amax_acc, a)
            sat_acc += s
            tickets += t
        d["amax_acc"] = amax_acc
        d["sat_acc"] = sat_acc
        d["ticket"] = struct.unpack_from("<I", raw, _OFF["ticket"])[0]
        d["slot_tickets"] = tickets
        return d

    def raw(self) -> bytes:
        return self.buf.cpu().numpy().tobytes()


def _rows_cols(t) -> tuple:
    """(rows, cols) of a tensor read as rows of its trailing elements (1-D: one
    row), without building a view (t[0] costs a microsecond per call)."""
    if t.dim() == 1:
        return 1, t.numel()
    r = t.shape[0]
    return r, (t.numel() // r if r else math.prod(t.shape[1:]))


def _room(t, nbytes: int, what: str) -> None:
    """Refuse a tensor argument smaller than the nbytes the call writes or reads."""
    if isinstance(t, torch.Tensor) and t.numel() * t.element_size() < nbytes:
        raise Fp8dpError(f"{what}: needs {nbytes} bytes, got {t.numel() * t.element_size()}")


def _elem(t, sizes, what: str) -> None:
    """Refuse a tensor whose element size is not one the kernel reads or writes
    (e.g. a uint8 tensor passed as a BF16 output would be written past its end)."""
    if isinstance(t, torch.Tensor) and t.element_size() not in sizes:
        raise Fp8dpError(f"{what}: expected {'/'.join(str(x) for x in sizes)}-byte elements, "
                         f"got {t.dtype}")


def _codes(t, what: str) -> None:
    if isinstance(t, torch.Tensor) and t.dtype not in (torch.uint8, torch.int8) and \
            not str(t.dtype).startswith("torch.float8"):
        raise Fp8dpError(f"{what}: expected 8-bit codes (uint8), got {t.dtype}")


def _gemm_operands(name: str, a, b, y=None) -> tuple:
    """Shapes (M, N, K) of a GEMM's code operands a [M, K], b [N, K] and its
    16-bit output y [M, N], with their element sizes checked."""
    _codes(a, f"{name}: a")
    _codes(b, f"{name}: b")
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K or (y is not None and tuple(y.shape) != (M, N)):
        raise Fp8dpError(f"{name}: shape mismatch")
    if y is not None:
        _elem(y, (2,), f"{name}: y")
    return M, N, K


def _state_ptr(st) -> Optional[int]:
    if st is None:
        return None
    if isinstance(st, TensorState):
        return _p(st.buf)
    return _p(st)


# --------------------------------------------------------------------------- entry points
def fp8dp_state_init(st, fmt: int, hist_len: int, margin: float, initial_amax: float,
                     stream=None) -> None:
    _check(lib().fp8dp_state_init(_state_ptr(st), fmt, hist_len, margin, initial_amax,
                                  _stream(stream)), "fp8dp_state_init")


def quantize_fused(h: torch.Tensor, act: int, fmt: int, mode: int, st=None,
                   bf16_out: Ptr = None, fp8_out: Ptr = None, group_scale_inv: Ptr = None,
                   stream=None) -> None:
    """h: BF16 (or 16-bit) device tensor [rows, cols] (1-D counts as one row)."""
    _elem(h, (2,), "quantize_fused: h")
    _elem(bf16_out, (2,), "quantize_fused: bf16_out")
    _codes(fp8_out, "quantize_fused: fp8_out")
    rows, cols = _rows_cols(h)
    _room(bf16_out, rows * cols * 2, "quantize_fused: bf16_out")
    _room(fp8_out, rows * cols, "quantize_fused: fp8_out")
    if mode == PER_GROUP128:
        _room(group_scale_inv, rows * (cols // 128) * 4, "quantize_fused: group_scale_inv")
    _check(lib().quantize_fused(_p(h), rows, cols, act, fmt, mode, _state_ptr(st), _p(bf16_out),
                                _p(fp8_out), _p(group_scale_inv), _stream(stream)),
           "quantize_fused")


def amax_history_update(st, stream=None) -> None:
    _check(lib().amax_history_update(_state_ptr(st), _stream(stream)), "amax_history_update")


def quantize_fused_update(h: torch.Tensor, act: int, fmt: int, st, bf16_out: Ptr = None,
                          fp8_out: Ptr = None, stream=None) -> None:
    """quantize_fused (PER_TENSOR) followed by amax_history_update, in one launch."""
    _elem(h, (2,), "quantize_fused_update: h")
    _elem(bf16_out, (2,), "quantize_fused_update: bf16_out")
    _codes(fp8_out, "quantize_fused_update: fp8_out")
    rows, cols = _rows_cols(h)
    _room(bf16_out, rows * cols * 2, "quantize_fused_update: bf16_out")
    _room(fp8_out, rows * cols, "quantize_fused_update: fp8_out")
    _check(lib().quantize_fused_update(_p(h), rows, cols, act, fmt, _state_ptr(st), _p(bf16_out),
                                       _p(fp8_out), _stream(stream)), "quantize_fused_update")


def fp8_gemm_scaled(a: torch.Tensor, fa: int, b: torch.Tensor, fb: int, mode: int,
                    a_scale_inv: Ptr, b_scale_inv: Ptr, y: torch.Tensor,
                    accum: int = ACCUM_EXACT, stream=None) -> None:
    """a [M, K] codes, b [N, K] codes, y [M, N] BF16; scales are device pointers/tensors;
    accum: ACCUM_EXACT (FP16 widening, FP32-accurate sums; the default) or
    ACCUM_MFMA_FP8 (the FP8 matrix instructions, which truncate small products)."""
    M, N, K = _gemm_operands("fp8_gemm_scaled", a, b, y)
    group = mode == PER_GROUP128
    _room(a_scale_inv, (M * (K // 128) if group else 1) * 4, "fp8_gemm_scaled: a_scale_inv")
    _room(b_scale_inv, ((N // 128) * (K // 128) if group else 1) * 4,
          "fp8_gemm_scaled: b_scale_inv")
    _check(lib().fp8_gemm_scaled(_p(a), fa, _p(b), fb, M, N, K, mode, accum, _p(a_scale_inv),
                                 _p(b_scale_inv), _p(y), _stream(stream)), "fp8_gemm_scaled")


def fp8_gemm_scaled_splitk(a: torch.Tensor, fa: int, b: torch.Tensor, fb: int, splits: int,
                           a_scale_inv: Ptr, b_scale_inv: Ptr, workspace: torch.Tensor,
                           y: torch.Tensor, accum: int = ACCUM_EXACT, stream=None) -> None:
    """Per-tensor FP8 GEMM with K split `splits` ways; workspace: float32 device
    tensor of at least splits * M * N elements."""
    M, N, K = _gemm_operands("fp8_gemm_scaled_splitk", a, b, y)
    if workspace.dtype != torch.float32 or workspace.numel() < splits * M * N:
        raise Fp8dpError("fp8_gemm_scaled_splitk: workspace needs splits * M * N float32")
    _check(lib().fp8_gemm_scaled_splitk(_p(a), fa, _p(b), fb, M, N, K, splits, accum,
                                        _p(a_scale_inv),
                                        _p(b_scale_inv), _p(workspace), _p(y), _stream(stream)),
           "fp8_gemm_scaled_splitk")


def fp8_gemm_scaled_splitk_noalloc(a: torch.Tensor, fa: int, b: torch.Tensor, fb: int,
                                   splits: int, a_scale_inv: Ptr, b_scale_inv: Ptr,
                                   y: torch.Tensor, accum: int = ACCUM_EXACT,
                                   stream=None) -> None:
    """fp8_gemm_scaled_splitk with the library's own per-GPU scratch array
    (splits * M * N <= 16 Mi floats) instead of a workspace: allocates nothing.
    Calls that overlap on one GPU race."""
    M, N, K = _gemm_operands("fp8_gemm_scaled_splitk_noalloc", a, b, y)
    _check(lib().fp8_gemm_scaled_splitk_noalloc(_p(a), fa, _p(b), fb, M, N, K, splits, accum,
                                                _p(a_scale_inv), _p(b_scale_inv), _p(y),
                                                _stream(stream)),
           "fp8_gemm_scaled_splitk_noalloc")


def quantize_fused_transposed(h: torch.Tensor, act: int, fmt: int, st, fp8_t_out: torch.Tensor,
                              bf16_out: Ptr = None, fp8_out: Ptr = None, stream=None) -> None:
    """Per-tensor quantize_fused of h [rows, cols] that also writes the codes
    transposed to fp8_t_out [cols, rows] (uint8)."""
    if h.dim() != 2:
        raise Fp8dpError("quantize_fused_transposed: h must be [rows, cols]")
    _elem(h, (2,), "quantize_fused_transposed: h")
    rows, cols = h.shape
    _codes(fp8_t_out, "quantize_fused_transposed: fp8_t_out")
    if fp8_t_out.numel() != rows * cols:
        raise Fp8dpError("quantize_fused_transposed: fp8_t_out needs cols x rows codes")
    _room(bf16_out, rows * cols * 2, "quantize_fused_transposed: bf16_out")
    _room(fp8_out, rows * cols, "quantize_fused_transposed: fp8_out")
    _check(lib().quantize_fused_transposed(_p(h), rows, cols, act, fmt, _state_ptr(st),
                                           _p(bf16_out), _p(fp8_out), _p(fp8_t_out),
                                           _stream(stream)), "quantize_fused_transposed")


def fp8_transpose(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """dst [cols, rows] = src [rows, cols]^T (uint8 codes)."""
    _codes(src, "fp8_transpose: src")
    _codes(dst, "fp8_transpose: dst")
    rows, cols = src.shape
    if tuple(dst.shape) != (cols, rows):
        raise Fp8dpError("fp8_transpose: shape mismatch")
    _check(lib().fp8_transpose(_p(src), rows, cols, _p(dst), _stream(stream)), "fp8_transpose")


CACHE_E4M3, CACHE_E5M2, CACHE_BF16 = 0, 1, 2


def relu2_backward_quantize(dA: torch.Tensor, a_cache: torch.Tensor, cache: int,
                            a_scale_inv: Ptr, fmt: int, st, fp8_out: torch.Tensor,
                            bf16_out: Ptr = None, stream=None) -> None:
    """dH = dA * 2 sqrt(A) from the cached activation (FP8 codes + inverse scale, or
    BF16), cast to fmt with st's delayed scale (amax / saturation folded into st)."""
    _elem(dA, (2,), "relu2_backward_quantize: dA")
    if cache == CACHE_BF16:
        _elem(a_cache, (2,), "relu2_backward_quantize: a_cache")
    else:
        _codes(a_cache, "relu2_backward_quantize: a_cache")
    _codes(fp8_out, "relu2_backward_quantize: fp8_out")
    _elem(bf16_out, (2,), "relu2_backward_quantize: bf16_out")
    rows, cols = _rows_cols(dA)
    if a_cache.numel() != dA.numel() or fp8_out.numel() != dA.numel():
        raise Fp8dpError("relu2_backward_quantize: size mismatch")
    _room(bf16_out, rows * cols * 2, "relu2_backward_quantize: bf16_out")
    _check(lib().relu2_backward_quantize(_p(dA), _p(a_cache), cache, _p(a_scale_inv), rows, cols,
                                         fmt, _state_ptr(st), _p(bf16_out), _p(fp8_out),
                                         _stream(stream)), "relu2_backward_quantize")


def fp8_gemm_relu2_backward(a: torch.Tensor, fa: int, b: torch.Tensor, fb: int, a_scale_inv: Ptr,
                            b_scale_inv: Ptr, act_cache: torch.Tensor, cache: int,
                            act_scale_inv: Ptr, fmt: int, st, dh_out: torch.Tensor,
                            accum: int = ACCUM_EXACT, stream=None) -> None:
    """dgrad a [M, K] x b [N, K]^T with the squared ReLU's backward in the epilogue:
    dh_out [M, N] gradient codes from the cached activation codes act_cache [M, N]."""
    M, N, K = _gemm_operands("fp8_gemm_relu2_backward", a, b)
    _codes(act_cache, "fp8_gemm_relu2_backward: act_cache")
    _codes(dh_out, "fp8_gemm_relu2_backward: dh_out")
    if tuple(act_cache.shape) != (M, N) or tuple(dh_out.shape) != (M, N):
        raise Fp8dpError("fp8_gemm_relu2_backward: shape mismatch")
    _check(lib().fp8_gemm_relu2_backward(_p(a), fa, _p(b), fb, M, N, K, accum, _p(a_scale_inv),
                                         _p(b_scale_inv), _p(act_cache), cache, _p(act_scale_inv),
                                         fmt, _state_ptr(st), _p(dh_out), _stream(stream)),
           "fp8_gemm_relu2_backward")


def quantize_recompute(h: torch.Tensor, act: int, fmt: int, st, fp8_out: torch.Tensor,
                       stream=None) -> None:
    """Re-cast h with st's corrected scale when st's last update flagged an overflow
    (decided on the GPU; otherwise nothing is written)."""
    _elem(h, (2,), "quantize_recompute: h")
    _codes(fp8_out, "quantize_recompute: fp8_out")
    rows, cols = _rows_cols(h)
    _room(fp8_out, rows * cols, "quantize_recompute: fp8_out")
    _check(lib().quantize_recompute(_p(h), rows, cols, act, fmt, _state_ptr(st), _p(fp8_out),
                                    _stream(stream)), "quantize_recompute")


def fp8_gemm_scaled_if(a: torch.Tensor, fa: int, b: torch.Tensor, fb: int, a_scale_inv: Ptr,
                       b_scale_inv: Ptr, y: torch.Tensor, run_flag: Ptr,
                       accum: int = ACCUM_EXACT, stream=None) -> None:
    """Per-tensor FP8 GEMM that runs only when the device word *run_flag is nonzero."""
    M, N, K = _gemm_operands("fp8_gemm_scaled_if", a, b, y)
    _room(a_scale_inv, 4, "fp8_gemm_scaled_if: a_scale_inv")
    _room(b_scale_inv, 4, "fp8_gemm_scaled_if: b_scale_inv")
    _room(run_flag, 4, "fp8_gemm_scaled_if: run_flag")
    _check(lib().fp8_gemm_scaled_if(_p(a), fa, _p(b), fb, M, N, K, accum, _p(a_scale_inv),
                                    _p(b_scale_inv), _p(y), _p(run_flag), _stream(stream)),
           "fp8_gemm_scaled_if")


def quantize_mx(h: torch.Tensor, act: int, fmt: int, fp8_out: torch.Tensor,
                scale_out: torch.Tensor, bf16_out: Ptr = None, stream=None) -> None:
    """MXFP8 cast: h [rows, cols] BF16 (cols % 32 == 0) -> fp8_out [rows, cols] codes and
    scale_out [rows, cols/32] E8M0 block exponents (uint8)."""
    _elem(h, (2,), "quantize_mx: h")
    _codes(fp8_out, "quantize_mx: fp8_out")
    _codes(scale_out, "quantize_mx: scale_out")
    _elem(bf16_out, (2,), "quantize_mx: bf16_out")
    rows, cols = _rows_cols(h)
    if fp8_out.numel() != rows * cols or scale_out.numel() * 32 != rows * cols:
        raise Fp8dpError("quantize_mx: output sizes do not match the input")
    _room(bf16_out, rows * cols * 2, "quantize_mx: bf16_out")
    _check(lib().quantize_mx(_p(h), rows, cols, act, fmt, _p(bf16_out), _p(fp8_out),
                             _p(scale_out), _stream(stream)), "quantize_mx")


def quantize_mx_transposed(h: torch.Tensor, act: int, fmt: int, fp8_t_out: torch.Tensor,
                           scale_t_out: torch.Tensor, bf16_out: Ptr = None,
                           stream=None) -> None:
    """MXFP8 cast of h [rows, cols] BF16 with the blocks of 32 down the columns:
    fp8_t_out [cols, rows] codes, scale_t_out [cols, rows/32] E8M0 exponents
    (quantize_mx of act(h) transposed); bf16_out [rows, cols] optional."""
    if h.dim() != 2:
        raise Fp8dpError("quantize_mx_transposed: h must be [rows, cols]")
    _elem(h, (2,), "quantize_mx_transposed: h")
    _codes(fp8_t_out, "quantize_mx_transposed: fp8_t_out")
    _codes(scale_t_out, "quantize_mx_transposed: scale_t_out")
    _elem(bf16_out, (2,), "quantize_mx_transposed: bf16_out")
    rows, cols = h.shape
    if fp8_t_out.numel() != rows * cols or scale_t_out.numel() * 32 != rows * cols:
        raise Fp8dpError("quantize_mx_transposed: outputs need cols x rows codes and "
                         "cols x rows/32 exponents")
    _room(bf16_out, rows * cols * 2, "quantize_mx_transposed: bf16_out")
    _check(lib().quantize_mx_transposed(_p(h), rows, cols, act, fmt, _p(bf16_out), _p(fp8_t_out),
                                        _p(scale_t_out), _stream(stream)),
           "quantize_mx_transposed")


def fp8_gemm_mx(a: torch.Tensor, fa: int, a_scale: torch.Tensor, b: torch.Tensor, fb: int,
                b_scale: torch.Tensor, y: torch.Tensor, accum: int = ACCUM_EXACT,
                stream=None) -> None:
    """MXFP8 GEMM y [M, N] = a [M, K] b [N, K]^T with E8M0 block exponents
    a_scale [M, K/32] and b_scale [N, K/32] (uint8); accum as for fp8_gemm_scaled."""
    M, N, K = _gemm_operands("fp8_gemm_mx", a, b, y)
    for name, e, rows in (("a_scale", a_scale, M), ("b_scale", b_scale, N)):
        if e.element_size() != 1 or e.numel() * 32 != rows * K:
            raise Fp8dpError(f"fp8_gemm_mx: {name} needs {rows * K // 32} uint8 exponents")
    _check(lib().fp8_gemm_mx(_p(a), fa, _p(a_scale), _p(b), fb, _p(b_scale), M, N, K, accum,
                             _p(y), _stream(stream)), "fp8_gemm_mx")


def fp8_gemm_mx_splitk(a: torch.Tensor, fa: int, a_scale: torch.Tensor, b: torch.Tensor,
                       fb: int, b_scale: torch.Tensor, splits: int, workspace: torch.Tensor,
                       y: torch.Tensor, accum: int = ACCUM_EXACT, stream=None) -> None:
    """fp8_gemm_mx with K split `splits` ways; workspace: float32 device tensor of
    at least splits * M * N elements."""
    M, N, K = _gemm_operands("fp8_gemm_mx_splitk", a, b, y)
    for name, e, rows in (("a_scale", a_scale, M), ("b_scale", b_scale, N)):
        if e.element_size() != 1 or e.numel() * 32 != rows * K:
            raise Fp8dpError(f"fp8_gemm_mx_splitk: {name} needs {rows * K // 32} uint8 exponents")
    if workspace.dtype != torch.float32 or workspace.numel() < splits * M * N:
        raise Fp8dpError("fp8_gemm_mx_splitk: workspace needs splits * M * N float32")
    _check(lib().fp8_gemm_mx_splitk(_p(a), fa, _p(a_scale), _p(b), fb, _p(b_scale), M, N, K,
                                    splits, accum, _p(workspace), _p(y), _stream(stream)),
           "fp8_gemm_mx_splitk")


def quantize_weight(w: torch.Tensor, fmt: int, mode: int, w8: torch.Tensor, scale_out: Ptr,
                    stream=None) -> None:
    """w [N, K] BF16 -> w8 [N, K] codes; scale_out: per tensor [1/s, s], per group
    one inverse scale per 128 x 128 block."""
    if w.dim() != 2:
        raise Fp8dpError("quantize_weight: w must be [N, K]")
    _elem(w, (2,), "quantize_weight: w")
    _codes(w8, "quantize_weight: w8")
    N, K = w.shape
    _room(w8, N * K, "quantize_weight: w8")
    if isinstance(scale_out, torch.Tensor):
        need = 2 if mode == PER_TENSOR else (N // 128) * (K // 128)
        if scale_out.dtype != torch.float32 or scale_out.numel() < need:
            raise Fp8dpError(f"quantize_weight: scale_out needs {need} float32 values "
                             "(per tensor: [1/s, s]; per group: one per 128 x 128 block)")
    _check(lib().quantize_weight(_p(w), N, K, fmt, mode, _p(w8), _p(scale_out), _stream(stream)),
           "quantize_weight")


def gemm_bf16_quantize_fused(x: torch.Tensor, w: torch.Tensor, act: int = ACT_RELU2,
                             fmt: int = E4M3, st=None, h_out: Ptr = None, bf16_out: Ptr = None,
                             fp8_out: Ptr = None, stream=None) -> None:
    """x [M, K] BF16, w [N, K] BF16 device tensors; outputs [M, N] (see the C header)."""
    _elem(x, (2,), "gemm_bf16_quantize_fused: x")
    _elem(w, (2,), "gemm_bf16_quantize_fused: w")
    _elem(h_out, (2,), "gemm_bf16_quantize_fused: h_out")
    _elem(bf16_out, (2,), "gemm_bf16_quantize_fused: bf16_out")
    _codes(fp8_out, "gemm_bf16_quantize_fused: fp8_out")
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise Fp8dpError("gemm_bf16_quantize_fused: shape mismatch")
    _room(h_out, M * N * 2, "gemm_bf16_quantize_fused: h_out")
    _room(bf16_out, M * N * 2, "gemm_bf16_quantize_fused: bf16_out")
    _room(fp8_out, M * N, "gemm_bf16_quantize_fused: fp8_out")
    _check(lib().gemm_bf16_quantize_fused(_p(x), _p(w), M, N, K, act, fmt, _state_ptr(st),
                                          _p(h_out), _p(bf16_out), _p(fp8_out), _stream(stream)),
           "gemm_bf16_quantize_fused")


def fp8dp_bench_act_bf16(h: torch.Tensor, act: int, out: torch.Tensor, stream=None) -> None:
    _elem(h, (2,), "fp8dp_bench_act_bf16: h")
    _elem(out, (2,), "fp8dp_bench_act_bf16: out")
    _room(out, h.numel() * 2, "fp8dp_bench_act_bf16: out")
    _check(lib().fp8dp_bench_act_bf16(_p(h), h.numel(), act, _p(out), _stream(stream)),
           "fp8dp_bench_act_bf16")


def fp8dp_bench_amax(x: torch.Tensor, st, stream=None) -> None:
    _elem(x, (2,), "fp8dp_bench_amax: x")
    _check(lib().fp8dp_bench_amax(_p(x), x.numel(), _state_ptr(st), _stream(stream)),
           "fp8dp_bench_amax")


def fp8dp_bench_cast(x: torch.Tensor, fmt: int, st, out: torch.Tensor, stream=None) -> None:
    _elem(x, (2,), "fp8dp_bench_cast: x")
    _codes(out, "fp8dp_bench_cast: out")
    _room(out, x.numel(), "fp8dp_bench_cast: out")
    _check(lib().fp8dp_bench_cast(_p(x), x.numel(), fmt, _state_ptr(st), _p(out),
                                  _stream(stream)), "fp8dp_bench_cast")


def fp8dp_bench_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    nbytes = src.numel() * src.element_size()
    _room(dst, nbytes, "fp8dp_bench_copy: dst")
    _check(lib().fp8dp_bench_copy(_p(src), _p(dst), nbytes, _stream(stream)), "fp8dp_bench_copy")


def fp8dp_convert_f32(x: torch.Tensor, target: int, out: torch.Tensor, stream=None) -> None:
    """target 0/1: E4M3/E5M2 codes, 2: BF16, 3/4: saturation predicates (bytes),
    5: binary32 square root (float)."""
    _elem(x, (4,), "fp8dp_convert_f32: x")
    _room(out, x.numel() * {2: 2, 5: 4}.get(target, 1), "fp8dp_convert_f32: out")
    _check(lib().fp8dp_convert_f32(_p(x), x.numel(), target, _p(out), _stream(stream)),
           "fp8dp_convert_f32")


def fp8dp_scale_rule(amax: torch.Tensor, margin: float, fmt: int, scale: torch.Tensor,
                     scale_inv: Ptr = None, stream=None) -> None:
    _elem(amax, (4,), "fp8dp_scale_rule: amax")
    _room(scale, amax.numel() * 4, "fp8dp_scale_rule: scale")
    _room(scale_inv, amax.numel() * 4, "fp8dp_scale_rule: scale_inv")
    _check(lib().fp8dp_scale_rule(_p(amax), amax.numel(), margin, fmt, _p(scale), _p(scale_inv),
                                  _stream(stream)), "fp8dp_scale_rule")


def fp8dp_set_grid_limit(blocks: int) -> int:
    return lib().fp8dp_set_grid_limit(blocks)


def fp8dp_set_codec(codec: int) -> int:
    return lib().fp8dp_set_codec(codec)
