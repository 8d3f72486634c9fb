"""Pins for the oracle's float64 reference GEMM (CPU only).

"FP8 training: what it is and how it works" -- Step 3: FP8 inputs, sums kept in
a wider format; Trade-offs (1 x 128 activation tiles, 128 x 128 weight
blocks).  "FP8 Training & Inference" -- Per-Tensor Scaling: the scales are
factored out of the product and the output is rescaled.

The reference is checked against exact rational arithmetic (Python
fractions over torch's float8 decode of each code), a scaled identity weight,
and constant inputs whose sum has a closed form.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import refcheck as R


def _finite_codes(rng, shape, fmt):
    t = R.torch_decode_table(fmt)
    ok = np.flatnonzero(np.isfinite(t))
    return rng.choice(ok, size=shape).astype(np.uint8)


def _exact(a, fa, b, fb, mode, sa, sb, bcols=None):
    """Exact sum over k of dec(a) dec(b) / (s_a s_b); bcols gives each row of b
    its column index in the full weight (for the 128-column block lookup)."""
    ta = R.torch_decode_table(fa)
    tb = R.torch_decode_table(fb)
    M, K = a.shape
    N = b.shape[0]
    ref = np.empty((M, N))
    absref = np.empty((M, N))
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            tot_abs = Fraction(0)
            for k in range(K):
                p = Fraction(float(ta[a[m, k]])) * Fraction(float(tb[b[n, k]]))
                g = k // 128
                if mode == O.PER_TENSOR:
                    d = Fraction(float(np.float32(sa))) * Fraction(float(np.float32(sb)))
                else:
                    col = n if bcols is None else bcols[n]
                    d = Fraction(float(sa[m, g])) * Fraction(float(sb[col // 128, g]))
                tot += p / d
                tot_abs += abs(p) / d
            ref[m, n] = float(tot)
            absref[m, n] = float(tot_abs)
    return ref, absref


@pytest.mark.parametrize("fa,fb", [(O.E4M3, O.E4M3), (O.E5M2, O.E4M3), (O.E4M3, O.E5M2)])
def test_gemm_per_tensor_vs_exact_rationals(fa, fb):
    rng = np.random.default_rng(3 + fa + 2 * fb)
    a = _finite_codes(rng, (3, 256), fa)
    b = _finite_codes(rng, (5, 256), fb)
    sa, sb = np.float32(37.125), np.float32(0.0123)
    ref, absref = O.gemm_f64(a, fa, b, fb, O.PER_TENSOR, sa, sb)
    eref, eabs = _exact(a, fa, b, fb, O.PER_TENSOR, sa, sb)
    assert np.allclose(ref, eref, rtol=1e-14, atol=1e-14 * eabs.max())
    assert np.allclose(absref, eabs, rtol=1e-14)


def test_gemm_per_group_vs_exact_rationals():
    rng = np.random.default_rng(17)
    M, N, K = 2, 256, 384
    a = _finite_codes(rng, (M, K), O.E4M3)
    b = _finite_codes(rng, (N, K), O.E4M3)
    sa = (2.0 ** rng.uniform(-8, 8, (M, K // 128))).astype(np.float32)
    sb = (2.0 ** rng.uniform(-8, 8, (N // 128, K // 128))).astype(np.float32)
    cols = [0, 1, 127, 128, 200, 255]
    ref, absref = O.gemm_f64(a, O.E4M3, b, O.E4M3, O.PER_GROUP128, sa, sb)
    eref, eabs = _exact(a, O.E4M3, b[cols], O.E4M3, O.PER_GROUP128, sa, sb, bcols=cols)
    assert np.allclose(ref[:, cols], eref, rtol=1e-14, atol=1e-13 * eabs.max())
    assert np.allclose(absref[:, cols], eabs, rtol=1e-14)


def test_gemm_scaled_identity_weight_returns_dequantized_input():
    rng = np.random.default_rng(1)
    K = 128
    a = _finite_codes(rng, (4, K), O.E4M3)
    b = np.zeros((K, K), dtype=np.uint8)
    np.fill_diagonal(b, 0x38)                               # E4M3 code of 1.0
    assert R.torch_decode_table(O.E4M3)[0x38] == 1.0
    sa, sb = np.float32(3.5), np.float32(1.0)
    ref, _ = O.gemm_f64(a, O.E4M3, b, O.E4M3, O.PER_TENSOR, sa, sb)
    deq = R.torch_decode_table(O.E4M3)[a] / 3.5
    assert np.array_equal(ref, deq)


def test_gemm_constant_max_inputs_closed_form():
    K = 16384
    a = np.full((2, K), 0x7E, dtype=np.uint8)               # +448
    b = np.full((3, K), 0xFE, dtype=np.uint8)               # -448
    ref, absref = O.gemm_f64(a, O.E4M3, b, O.E4M3, O.PER_TENSOR, np.float32(2.0),
                             np.float32(0.5))
    assert np.all(ref == -K * 448.0 * 448.0)
    assert np.all(absref == K * 448.0 * 448.0)


def test_gemm_row_sampling_matches_full():
    rng = np.random.default_rng(5)
    a = _finite_codes(rng, (64, 256), O.E4M3)
    b = _finite_codes(rng, (128, 256), O.E4M3)
    full, fabs = O.gemm_f64(a, O.E4M3, b, O.E4M3, O.PER_TENSOR, np.float32(2.0), np.float32(3.0))
    rows = [0, 7, 63, 31]
    part, pabs = O.gemm_f64(a, O.E4M3, b, O.E4M3, O.PER_TENSOR, np.float32(2.0), np.float32(3.0),
                            rows=rows)
    assert np.array_equal(part, full[rows]) and np.array_equal(pabs, fabs[rows])


def test_gemm_matches_float64_matmul_of_dequantized_inputs():
    # a library matmul over the dequantized operands agrees to float64 rounding
    rng = np.random.default_rng(8)
    a = _finite_codes(rng, (32, 512), O.E4M3)
    b = _finite_codes(rng, (64, 512), O.E4M3)
    sa, sb = np.float32(11.0), np.float32(0.25)
    ref, absref = O.gemm_f64(a, O.E4M3, b, O.E4M3, O.PER_TENSOR, sa, sb)
    t = R.torch_decode_table(O.E4M3)
    mm = (torch.from_numpy(t[a]) @ torch.from_numpy(t[b]).T).numpy() / (11.0 * 0.25)
    assert np.allclose(ref, mm, rtol=0, atol=1e-12 * absref.max())


# ---------------------------------------------------------------------------
# BF16 x BF16 reference of the up-projection whose epilogue carries the
# quantizer ("Paradigma Details FP8 and Optimizer Tricks Behind NanoGPT
# Records", FP8 paragraph).

def _bf16_bits(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_values(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()


def test_gemm_bf16_vs_exact_rationals():
    rng = np.random.default_rng(21)
    x = _bf16_bits(rng, (5, 96), 3.0)
    w = _bf16_bits(rng, (7, 96), 0.1)
    ref, absref = O.gemm_bf16_f64(x, w)
    xv, wv = _bf16_values(x), _bf16_values(w)
    for m in range(5):
        for n in range(7):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xv[m], wv[n]))
            exact_abs = sum(abs(Fraction(float(a)) * Fraction(float(b))) for a, b in zip(xv[m], wv[n]))
            assert abs(Fraction(ref[m, n]) - exact) <= Fraction(2.0 ** -50) * exact_abs
            assert abs(Fraction(absref[m, n]) - exact_abs) <= Fraction(2.0 ** -50) * exact_abs


def test_gemm_bf16_identity_weight_and_transpose_symmetry():
    rng = np.random.default_rng(22)
    x = _bf16_bits(rng, (16, 64), 5.0)
    one = np.uint16(0x3F80)
    eye = np.zeros((64, 64), np.uint16)
    np.fill_diagonal(eye, one)
    ref, _ = O.gemm_bf16_f64(x, eye)
    assert np.array_equal(ref, _bf16_values(x))
    # (X W^T)^T = W X^T: swapping the operands transposes the result
    w = _bf16_bits(rng, (24, 64))
    a, _ = O.gemm_bf16_f64(x, w)
    b, _ = O.gemm_bf16_f64(w, x)
    assert np.allclose(a, b.T, rtol=0, atol=1e-12 * np.abs(a).max())


def test_gemm_bf16_matches_float64_matmul_and_row_sampling():
    rng = np.random.default_rng(23)
    x = _bf16_bits(rng, (64, 768))
    w = _bf16_bits(rng, (96, 768), 768 ** -0.5)
    ref, absref = O.gemm_bf16_f64(x, w)
    mm = torch.from_numpy(_bf16_values(x)) @ torch.from_numpy(_bf16_values(w)).T
    assert np.all(np.abs(ref - mm.numpy()) <= 1e-13 * absref)
    rows = [0, 17, 63]
    r2, a2 = O.gemm_bf16_f64(x, w, rows=rows)
    assert np.array_equal(r2, ref[rows]) and np.array_equal(a2, absref[rows])
