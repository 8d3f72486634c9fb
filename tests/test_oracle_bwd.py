"""Pins for the oracle's squared-ReLU backward from a cached activation (CPU).

"FP8 training: what it is and how it works", Step 3: the activations kept for
the backward pass may be stored in FP8, except a few sensitive ones.  For
A = relu(H)^2 the backward needs dH = dA * 2 relu(H) = dA * 2 sqrt(A), so the
cached activation (BF16 copy or FP8 codes with their inverse scale) is all it
reads.

Independent checks: torch autograd of relu(h)^2 in float64 (the chain rule)
within the error the cached format allows; exact squares; signed zeros; the
E5M2 codes of the result by nearest-code search over torch's float8 table;
amax and the saturation count from numpy / torch.
"""
import numpy as np
import pytest
import torch

import oracle as O
import refcheck as R


def _bf16(x):
    return R.torch_bf16(np.asarray(x, np.float32))


def _autograd_dh(h_bits, dA_bits):
    h = torch.from_numpy(R.f32_from_bf16(h_bits).astype(np.float64)).requires_grad_(True)
    a = torch.relu(h) ** 2
    a.backward(torch.from_numpy(R.f32_from_bf16(dA_bits).astype(np.float64)))
    return h.grad.numpy()


def _case(seed, n=4096):
    rng = np.random.default_rng(seed)
    h = _bf16(rng.standard_normal(n))
    dA = _bf16(rng.standard_normal(n) * np.exp2(rng.integers(-8, 8, n)))
    a16 = R.torch_bf16((torch.relu(torch.from_numpy(R.f32_from_bf16(h))) ** 2).numpy())
    return h, dA, a16


def test_bf16_cache_chain_rule():
    h, dA, a16 = _case(1)
    r = O.relu2_backward(dA, a16, O.CACHE_BF16, 1.0, O.E5M2, 1.0)
    g = R.f32_from_bf16(r.bf16).astype(np.float64)
    ref = _autograd_dh(h, dA)
    # a carries the BF16 rounding of h^2 (unit roundoff 2^-8 relative, 2^-9
    # after the square root); the result one more BF16 rounding (2^-8);
    # binary32 steps are far smaller
    assert np.all(np.abs(g - ref) <= (2.0 ** -9 + 2.0 ** -8 + 2.0 ** -20) * np.abs(ref))
    assert np.all((ref == 0) == (g == 0))


@pytest.mark.parametrize("cache_fmt", [O.E4M3, O.E5M2])
def test_fp8_cache_chain_rule(cache_fmt):
    h, dA, a16 = _case(2 + cache_fmt)
    # the forward cast: codes of bf16(relu(h)^2) * s, s from the tensor's amax
    amax = float(R.f32_from_bf16(a16).max())
    s = np.float32(O.FMT_MAX[cache_fmt] / (1.25 * amax))          # not a power of two
    codes = R.nearest_code(R.f32_from_bf16(a16) * s, cache_fmt)
    si = np.float32(1.0) / s
    r = O.relu2_backward(dA, codes, cache_fmt, float(si), O.E5M2, 1.0)
    g = R.f32_from_bf16(r.bf16).astype(np.float64)
    ref = _autograd_dh(h, dA)
    # FP8 rounding of a: 2^-(m+1) relative in the normal range (half that after
    # the square root) plus the BF16 roundings; small a fall into subnormal
    # codes, whose absolute step is bounded separately
    m = 3 if cache_fmt == O.E4M3 else 2
    a_true = R.f32_from_bf16(a16).astype(np.float64)
    sub_step = (2.0 ** (-9 if cache_fmt == O.E4M3 else -16)) / float(s)
    rel = 2.0 ** -(m + 2) + 2.0 ** -9 + 2.0 ** -8 + 2.0 ** -20
    abs_dA = np.abs(R.f32_from_bf16(dA).astype(np.float64))
    bound = rel * np.abs(ref) + 2.0 * np.sqrt(sub_step) * abs_dA * (a_true < 64 * sub_step)
    assert np.all(np.abs(g - ref) <= bound)
    # a dropped inverse scale would be off by sqrt(s), far outside the bound
    assert np.abs(ref).max() > 0


def test_exact_squares_and_signed_zeros():
    a = _bf16([4.0, 2.25, 0.0, 0.0, 1.0, 0.0625, 16.0])
    dA = _bf16([3.0, -1.0, 5.0, -5.0, -0.5, 8.0, 0.25])
    r = O.relu2_backward(dA, a, O.CACHE_BF16, 1.0, O.E5M2, 1.0)
    g = R.f32_from_bf16(r.bf16)
    assert g.tolist() == [12.0, -3.0, 0.0, 0.0, -1.0, 4.0, 2.0]
    assert np.signbit(g).tolist() == [False, True, False, True, True, False, False]
    assert r.fp8[2] == 0x00 and r.fp8[3] == 0x80
    # an FP8 cache of E4M3 code 0x41 (2.25) with inverse scale 4 -> a = 9
    r2 = O.relu2_backward(_bf16([0.5]), np.array([0x41], np.uint8), O.E4M3, 4.0, O.E5M2, 1.0)
    assert R.f32_from_bf16(r2.bf16).tolist() == [3.0]


def test_gradient_cast_codes_amax_and_saturation():
    h, dA, a16 = _case(5)
    for scale in (1.0, 3.0e4, 1.0e7):
        r = O.relu2_backward(dA, a16, O.CACHE_BF16, 1.0, O.E5M2, scale)
        v = R.f32_from_bf16(r.bf16) * np.float32(scale)
        assert np.array_equal(r.fp8, R.nearest_code(v, O.E5M2))
        assert r.sat == int(R.torch_overflows(v, O.E5M2).sum())
        mags = (r.bf16 & 0x7FFF).astype(np.uint32) << 16
        assert r.amax_bits == int(mags.max())
    assert r.sat > 0      # the largest scale saturates some elements


def _f32_order(dA_bits, dec, si, order):
    """dH in binary32, one nearest-even operation at a time, in a given order,
    evaluated with numpy float32 (an implementation separate from the oracle's
    C): 'oracle' is the stated reading a = dec * si; r = sqrt(a); g = (2 r) dA.
    (The doubling is exact, so where it sits does not matter.)"""
    with np.errstate(invalid="ignore", over="ignore"):
        dA = R.f32_from_bf16(dA_bits)
        dec = np.asarray(dec, np.float32)
        si = np.float32(si)
        if order == "oracle":
            return (np.float32(2.0) * np.sqrt(dec * si)) * dA
        if order == "divide":                 # a = dec / s instead of dec * (1/s)
            return (np.float32(2.0) * np.sqrt(dec / (np.float32(1.0) / si))) * dA
        if order == "split_sqrt":             # r = sqrt(dec) sqrt(si)
            return (np.float32(2.0) * (np.sqrt(dec) * np.sqrt(si))) * dA
        if order == "scale_last":             # g = 2 sqrt(dec) dA, then times sqrt(si)
            return ((np.float32(2.0) * np.sqrt(dec)) * dA) * np.sqrt(si)
    raise ValueError(order)


@pytest.mark.parametrize("cache_fmt", [O.E4M3, O.E5M2])
def test_operation_order_at_the_ulp(cache_fmt):
    """The BF16 dH of an FP8 cache bit for bit against the numpy float32
    formulation of the same order, for 1024 inverse scales that are not
    powers of two, each with every positive finite code x every BF16 dA in
    [1, 2): on a random subset, and on every input whose binary32 result lies
    within two ulps of a BF16 rounding midpoint (where a one-ulp change of the
    binary32 value flips the stored BF16 value; elsewhere the final BF16
    rounding hides it).  Each of three plausible reorderings differs from the
    oracle on some of those, so the comparison fixes the order, not just the
    value within the formats' error."""
    rng = np.random.default_rng(7 + cache_fmt)
    table = R.torch_decode_table(cache_fmt).astype(np.float32)
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[np.isfinite(table[codes]) & (table[codes] > 0)]
    mant = np.arange(127 << 7, 128 << 7, dtype=np.uint16)          # BF16 values in [1, 2)
    c = np.repeat(codes, mant.size)
    dA = np.tile(mant, codes.size)
    dec = table[c]
    hits = {"divide": 0, "split_sqrt": 0, "scale_last": 0}
    near_total = 0
    for si in rng.uniform(1e-3, 0.9, 1024).astype(np.float32):
        g = _f32_order(dA, dec, si, "oracle")
        low = (g.view(np.uint32) & 0xFFFF).astype(np.int64)
        pick = np.concatenate([np.flatnonzero(np.abs(low - 0x8000) <= 2),
                               rng.integers(0, c.size, 8)])
        near_total += pick.size - 8
        r = O.relu2_backward(dA[pick], c[pick], cache_fmt, float(si), O.E5M2, 1.0)
        want = R.torch_bf16(g[pick])
        assert np.array_equal(r.bf16, want), si
        for order in hits:
            other = R.torch_bf16(_f32_order(dA[pick], dec[pick], si, order))
            hits[order] += int((other != want).sum())
    assert near_total > 500, near_total
    assert all(v > 0 for v in hits.values()), hits
