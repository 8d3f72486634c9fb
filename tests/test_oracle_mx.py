"""Pins for the oracle's MXFP8 functions (CPU only).

"FP8 training: what it is and how it works" -- Trade-offs and edge cases: the
microscaling recipe (MXFP8) gives each block of 32 adjacent values its own
scale, and the scales are powers of two.  Step 2 gives the scale rule
(format maximum / amax).  The block exponent k (decode scale 2^k, stored as
the E8M0 byte k + 127) is read as the smallest k in [-127, 127] with
amax <= max * 2^k.

Independent formulations used here: the exponent from the BF16 exponent and
fraction bits (a closed form) and from exact rational search; codes from a
nearest-value search over torch's float8 decode table; the GEMM from a numpy
float64 matmul of the dequantized operands and from exact rationals.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import refcheck as R

FMT_EMAX = {O.E4M3: 8, O.E5M2: 15}          # max = 1.75 * 2^emax
MBITS = {O.E4M3: 3, O.E5M2: 2}
EMIN = {O.E4M3: -6, O.E5M2: -14}


def k_bits(mag16: int, fmt: int) -> int:
    """Closed form of the block exponent from a BF16 magnitude pattern: for a
    normal value 1.f * 2^e, amax <= 1.75 * 2^(e + k - emax) holds for
    k = e - emax exactly when the 7 fraction bits are <= 0b1100000 (1.75)."""
    ef, frac = mag16 >> 7, mag16 & 0x7F
    if ef == 0xFF:
        return 127
    if ef == 0:                      # zero and subnormals: far below max * 2^-127
        return -127
    k = (ef - 127) - FMT_EMAX[fmt] + (1 if frac > 0x60 else 0)
    return max(-127, min(127, k))


def k_rational(amax: Fraction, fmt: int) -> int:
    """Smallest k with amax / max <= 2^k, by exact rational search, clamped."""
    if amax == 0:
        return -127
    r = amax / Fraction(O.FMT_MAX[fmt])
    k = 0
    while Fraction(2) ** k < r:
        k += 1
    while Fraction(2) ** (k - 1) >= r:
        k -= 1
    return max(-127, min(127, k))


# ------------------------------------------------------------------ exponent
@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_exponent_closed_form_every_bf16_magnitude(fmt):
    for mag in range(0, 0x7F81):
        v = float(R.f32_from_bf16(np.array([mag], np.uint16))[0])
        k = O.mx_exponent(v, not np.isfinite(v), fmt)
        assert k == k_bits(mag, fmt), (hex(mag), k)


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_exponent_exact_rational_and_invariants(fmt):
    rng = np.random.default_rng(7 + fmt)
    mags = np.concatenate([rng.integers(1, 0x7F80, 600), [0x3F80, 0x3FE0, 0x3FE1, 0x4360, 0x4361,
                                                         0x0001, 0x0080, 0x7F7F]])
    for mag in mags:
        v = float(R.f32_from_bf16(np.array([mag], np.uint16))[0])
        k = O.mx_exponent(v, False, fmt)
        assert k == k_rational(Fraction(v), fmt)
        # no overflow at 2^k, and 2^(k-1) would overflow (unless clamped)
        assert Fraction(v) <= Fraction(O.FMT_MAX[fmt]) * Fraction(2) ** k
        if k > -127:
            assert Fraction(v) > Fraction(O.FMT_MAX[fmt]) * Fraction(2) ** (k - 1)


def test_exponent_worked_boundaries():
    # amax exactly 448 * 2^j -> k = j (the block maximum becomes the code 448)
    for j in (-20, -1, 0, 3):
        assert O.mx_exponent(448.0 * 2.0 ** j, False, O.E4M3) == j
        assert O.mx_exponent(57344.0 * 2.0 ** j, False, O.E5M2) == j
    # just above: one more power of two
    assert O.mx_exponent(448.0 * (1 + 2.0 ** -7), False, O.E4M3) == 1
    # amax 1.0: 1 <= 448 * 2^-8 = 1.75 and 1 > 0.875 -> k = -8
    assert O.mx_exponent(1.0, False, O.E4M3) == -8
    assert O.mx_exponent(0.0, False, O.E4M3) == -127
    assert O.mx_exponent(float("inf"), True, O.E4M3) == 127


# ------------------------------------------------------------------ quantize
def _blocks(rng, rows, cols):
    """BF16 patterns with block magnitudes spread over many binades."""
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(rng.integers(-30, 30, (rows, cols // 32, 1)).astype(np.float32)).repeat(
        32, axis=2).reshape(rows, cols)
    return R.torch_bf16(x)


def _act_ref(h: np.ndarray, act: int) -> np.ndarray:
    if act == O.ACT_IDENTITY:
        return h
    x = R.f32_from_bf16(h)
    t = torch.from_numpy(np.ascontiguousarray(x))
    y = torch.where(t > 0, t * t, torch.zeros_like(t))
    return y.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _mx_ref(b: np.ndarray, fmt: int):
    """Exponents per block (closed form) and codes by nearest-value search."""
    rows, cols = b.shape
    mags = (b & 0x7FFF).reshape(rows, cols // 32, 32)
    kk = np.vectorize(lambda m: k_bits(int(m), fmt))(mags.max(axis=2))
    v = R.f32_from_bf16(b).astype(np.float64).reshape(rows, cols // 32, 32)
    x = np.ldexp(v, -kk[..., None]).astype(np.float32)
    codes = R.nearest_code(x, fmt).reshape(rows, cols)
    return (kk + 127).astype(np.uint8), codes


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
@pytest.mark.parametrize("act", [O.ACT_IDENTITY, O.ACT_RELU2])
def test_quantize_mx_brute_force(fmt, act):
    rng = np.random.default_rng(11 + 2 * fmt + act)
    h = _blocks(rng, 24, 256)
    r = O.quantize_mx(h, act, fmt)
    b = _act_ref(h, act)
    assert np.array_equal(r.bf16, b)
    e, q = _mx_ref(b, fmt)
    assert np.array_equal(r.scale, e)
    assert np.array_equal(r.fp8, q)


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_quantize_mx_no_overflow_and_error_bound(fmt):
    rng = np.random.default_rng(23 + fmt)
    h = _blocks(rng, 64, 512)
    r = O.quantize_mx(h, O.ACT_IDENTITY, fmt)
    t = R.torch_decode_table(fmt)
    k = r.scale.astype(np.int64) - 127
    deq = t[r.fp8].reshape(64, 16, 32) * np.exp2(k)[..., None]
    b = R.f32_from_bf16(h).astype(np.float64).reshape(64, 16, 32)
    # the block maximum lands in (max/2, max]: nothing saturates, little range is wasted
    top = np.abs(t[r.fp8]).reshape(64, 16, 32).max(axis=2)
    assert (top <= O.FMT_MAX[fmt]).all()
    assert (top >= O.FMT_MAX[fmt] / 2 * (1 - 2.0 ** -MBITS[fmt])).all()
    # round to nearest: |error| <= half a grid step at the value's binade (or
    # half the smallest subnormal step), in units of the block scale
    ax = np.abs(b) * np.exp2(-k)[..., None]
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, EMIN[fmt])
    half_step = np.exp2(e - MBITS[fmt] - 1) * np.exp2(k)[..., None]
    assert (np.abs(deq - b) <= half_step).all()


def test_quantize_mx_block_locality():
    rng = np.random.default_rng(5)
    h = _blocks(rng, 4, 128)
    r0 = O.quantize_mx(h, O.ACT_IDENTITY, O.E4M3)
    h2 = h.copy()
    h2[2, 70] = R.torch_bf16(np.array([1e6], np.float32))[0]     # block 2 of row 2
    r1 = O.quantize_mx(h2, O.ACT_IDENTITY, O.E4M3)
    diff_s = np.argwhere(r0.scale != r1.scale)
    assert diff_s.tolist() == [[2, 2]]
    changed = np.argwhere(r0.fp8 != r1.fp8)
    assert ((changed[:, 0] == 2) & (changed[:, 1] // 32 == 2)).all()


def test_quantize_mx_special_blocks():
    h = np.zeros((1, 128), np.uint16)
    h[0, 32:64] = 0x8000                                   # block 1: negative zeros
    h[0, 64] = 0x7F80                                      # block 2: +inf, next a finite value
    h[0, 65] = R.torch_bf16(np.array([1e38], np.float32))[0]
    h[0, 66] = 0xFF80                                      # -inf
    h[0, 96] = 0xFFC0                                      # block 3: NaN (negative)
    h[0, 97] = R.torch_bf16(np.array([3.0], np.float32))[0]
    for fmt in (O.E4M3, O.E5M2):
        r = O.quantize_mx(h, O.ACT_IDENTITY, fmt)
        assert r.scale.tolist() == [[0, 0, 254, 254]]
        assert (r.fp8[0, :32] == 0x00).all() and (r.fp8[0, 32:64] == 0x80).all()
        mx = 0x7E if fmt == O.E4M3 else 0x7B
        assert r.fp8[0, 64] == mx and r.fp8[0, 66] == (0x80 | mx)
        # 1e38 (as BF16) times 2^-127 is about 0.588: a normal code, not zero
        v = float(R.f32_from_bf16(h[0, 65:66])[0]) * 2.0 ** -127
        assert r.fp8[0, 65] == R.nearest_code(np.array([v], np.float32), fmt)[0] != 0
        assert r.fp8[0, 96] == 0xFF
        assert r.fp8[0, 97] == 0      # 3 * 2^-127 is far below the smallest subnormal


# ------------------------------------------------------------------ GEMM
def _mx_operands(rng, rows, K, fmt):
    h = _blocks(rng, rows, K)
    r = O.quantize_mx(h, O.ACT_IDENTITY, fmt, want_bf16=False)
    return h, r.fp8, r.scale


def _dequant(q, e, fmt):
    t = R.torch_decode_table(fmt)
    return t[q] * np.repeat(np.exp2(e.astype(np.float64) - 127), 32, axis=1)


@pytest.mark.parametrize("fa,fb", [(O.E4M3, O.E4M3), (O.E5M2, O.E4M3)])
def test_gemm_mx_equals_dequantized_matmul(fa, fb):
    rng = np.random.default_rng(31 + fa)
    _, a, ea = _mx_operands(rng, 12, 256, fa)
    _, b, eb = _mx_operands(rng, 10, 256, fb)
    ref, absref = O.gemm_mx_f64(a, fa, ea, b, fb, eb)
    da, db = _dequant(a, ea, fa), _dequant(b, eb, fb)
    assert np.allclose(ref, da @ db.T, rtol=0, atol=1e-12 * absref.max())
    assert np.allclose(absref, np.abs(da) @ np.abs(db).T, rtol=1e-12, atol=0)


def test_gemm_mx_exact_rationals():
    rng = np.random.default_rng(37)
    _, a, ea = _mx_operands(rng, 2, 64, O.E4M3)
    _, b, eb = _mx_operands(rng, 3, 64, O.E5M2)
    ref, _ = O.gemm_mx_f64(a, O.E4M3, ea, b, O.E5M2, eb)
    ta, tb = R.torch_decode_table(O.E4M3), R.torch_decode_table(O.E5M2)
    for m in range(2):
        for n in range(3):
            tot = Fraction(0)
            for k in range(64):
                j = k // 32
                tot += (Fraction(float(ta[a[m, k]])) * Fraction(float(tb[b[n, k]]))
                        * Fraction(2) ** (int(ea[m, j]) - 127) * Fraction(2) ** (int(eb[n, j]) - 127))
            assert abs(Fraction(ref[m, n]) - tot) <= abs(tot) * Fraction(1, 2 ** 50)


def test_gemm_mx_close_to_unquantized_product():
    """Quantize both operands, multiply, compare with the exact product of the
    BF16 inputs: each element carries at most a relative error u = 2^-(m+1)
    (normal range; these inputs have no subnormal codes), so
    |y - x w| <= (2u + u^2) sum |x w|."""
    rng = np.random.default_rng(41)
    K = 512
    x = R.torch_bf16(rng.standard_normal((8, K)).astype(np.float32))
    w = R.torch_bf16((rng.standard_normal((6, K)) * 0.02).astype(np.float32))
    rx = O.quantize_mx(x, O.ACT_IDENTITY, O.E4M3)
    rw = O.quantize_mx(w, O.ACT_IDENTITY, O.E4M3)
    ref, _ = O.gemm_mx_f64(rx.fp8, O.E4M3, rx.scale, rw.fp8, O.E4M3, rw.scale)
    xf = R.f32_from_bf16(x).astype(np.float64)
    wf = R.f32_from_bf16(w).astype(np.float64)
    exact = xf @ wf.T
    u = 2.0 ** -4
    bound = (2 * u + u * u) * (np.abs(xf) @ np.abs(wf).T)
    # tiny elements of a block may fall to subnormal codes: allow their absolute step
    sub = 2.0 ** -10 * (np.repeat(np.exp2(rx.scale.astype(np.float64) - 127), 32, 1) @
                        np.abs(wf).T + np.abs(xf) @ np.repeat(
                            np.exp2(rw.scale.astype(np.float64) - 127), 32, 1).T)
    assert (np.abs(ref - exact) <= bound + sub).all()
    # and the error is genuinely small: a dropped scale or a transposed operand is not
    assert np.abs(ref - exact).max() < 0.05 * np.abs(exact).max()
