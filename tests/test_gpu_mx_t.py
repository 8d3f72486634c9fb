"""MXFP8 with the blocks down the columns, and the MXFP8 backward GEMMs (GPU).

"FP8 training: what it is and how it works", Trade-offs and edge cases (one
power-of-two scale per 32 adjacent values) with the FP8 recipe's backward
GEMMs ("FP8 Training & Inference", FP8 Training Recipe): the input gradient
dX = dY W contracts along W's rows and the weight gradient dW = dY^T X along
the tokens, so those operands need their blocks along that dimension.
quantize_mx_transposed is compared bit for bit with the oracle's quantize_mx
of the transposed tensor (codes, E8M0 exponents) and its BF16 copy with the
oracle's; the MX dgrad (fp8_gemm_mx on quantize_mx(dY) and
quantize_mx_transposed(W)) with the oracle's float64 MX GEMM to the plain
bound on sampled rows.  Workloads: small tiles over every act / format pair
and both codecs, special values, the GPT-2 activation, gradient and weight
at full size.
"""
import numpy as np
import pytest
import torch

import oracle as O
import scaled_quantization_amd as sq
import workloads
from gpu_util import (DEV, bf16_np, check_gemm, fp8_mfma_allowance_mx, to_dev_bf16, to_dev_u8,
                      u8_np)

pytestmark = pytest.mark.gpu

EXACT, FP8 = sq.ACCUM_EXACT, sq.ACCUM_MFMA_FP8
BOTH = pytest.mark.parametrize("accum", [EXACT, FP8], ids=["exact", "fp8"])


@pytest.fixture(params=[0, 1], ids=["hw", "int"])
def codec(request):
    prev = sq.fp8dp_set_codec(request.param)
    yield request.param
    sq.fp8dp_set_codec(prev)


def _spread(rng, rows, cols, lo=-20, hi=20):
    """Values whose 32-row column blocks sit at random binades."""
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(rng.integers(lo, hi, (rows // 32, 1, cols)).astype(np.float32)).repeat(
        32, axis=1).reshape(rows, cols)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _run_t(h_np, act, fmt, want_bf16=True):
    rows, cols = h_np.shape
    h = to_dev_bf16(h_np)
    b = torch.empty_like(h) if want_bf16 else None
    qt = torch.empty((cols, rows), dtype=torch.uint8, device=DEV)
    et = torch.empty((cols, rows // 32), dtype=torch.uint8, device=DEV)
    sq.quantize_mx_transposed(h, act, fmt, qt, et, b)
    return b, qt, et


def _oracle_t(h_np, act, fmt):
    return O.quantize_mx(np.ascontiguousarray(h_np.T), act, fmt, want_bf16=False)


@pytest.mark.parametrize("fmt", [0, 1], ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("act", [0, 1], ids=["identity", "relu2"])
@pytest.mark.parametrize("rows,cols", [(64, 128), (128, 384), (320, 256)])
def test_transposed_mx_vs_oracle(rows, cols, act, fmt, codec):
    rng = np.random.default_rng(rows + cols + 10 * act + fmt)
    h = _spread(rng, rows, cols)
    b, qt, et = _run_t(h, act, fmt)
    r = _oracle_t(h, act, fmt)
    assert np.array_equal(u8_np(et), r.scale)
    assert np.array_equal(u8_np(qt), r.fp8)
    assert np.array_equal(bf16_np(b), O.quantize_mx(h, act, fmt).bf16)


@pytest.mark.parametrize("fmt", [0, 1], ids=["e4m3", "e5m2"])
def test_transposed_mx_special_blocks(fmt, codec):
    rng = np.random.default_rng(19)
    h = _spread(rng, 128, 256)
    h[0:32, 0] = 0                         # zero block
    h[32:64, 1] = 0x8000                   # negative zeros
    h[0:32, 2] = rng.integers(1, 0x80, 32)   # BF16 subnormals only
    h[5, 3] = 0x7F80                       # +inf with finite neighbours
    h[40, 4] = 0xFF80                      # -inf
    h[70, 5] = 0x7FC1                      # NaN
    h[100, 6] = 0xFFC0                     # -NaN
    h[64:96, 7] = 0x7F7F                   # largest finite BF16 everywhere
    h[9, 8] = 0x0001                       # smallest subnormal among normal values
    for act in (0, 1):
        b, qt, et = _run_t(h, act, fmt)
        r = _oracle_t(h, act, fmt)
        assert np.array_equal(u8_np(et), r.scale), act
        assert np.array_equal(u8_np(qt), r.fp8), act
        assert np.array_equal(bf16_np(b), O.quantize_mx(h, act, fmt).bf16), act


def test_transposed_mx_equals_quantize_mx_of_the_transpose():
    rng = np.random.default_rng(23)
    h_np = _spread(rng, 256, 512)
    _, qt, et = _run_t(h_np, sq.ACT_RELU2, sq.E4M3, want_bf16=False)
    ht = to_dev_bf16(np.ascontiguousarray(h_np.T))
    q2 = torch.empty((512, 256), dtype=torch.uint8, device=DEV)
    e2 = torch.empty((512, 8), dtype=torch.uint8, device=DEV)
    sq.quantize_mx(ht, sq.ACT_RELU2, sq.E4M3, q2, e2)
    assert torch.equal(qt, q2) and torch.equal(et, e2)


@pytest.mark.parametrize("which", ["activation", "gradient", "weight"])
def test_transposed_mx_gpt2_full_size(which):
    w = workloads.get("gpt2")
    if which == "activation":
        h, act, fmt = w.h0(), O.ACT_RELU2, O.E4M3
    elif which == "gradient":
        h, act, fmt = w.dy(), O.ACT_IDENTITY, O.E5M2
    else:
        h, act, fmt = w.weight(), O.ACT_IDENTITY, O.E4M3
    b, qt, et = _run_t(h, act, fmt, want_bf16=(act == O.ACT_RELU2))
    r = _oracle_t(h, act, fmt)
    assert np.array_equal(u8_np(et), r.scale)
    assert np.array_equal(u8_np(qt), r.fp8)
    if act == O.ACT_RELU2:
        assert np.array_equal(bf16_np(b), O.quantize(h, act, fmt, O.PER_TENSOR, 1.0,
                                                     want_fp8=False).bf16)


@BOTH
def test_mx_dgrad_gpt2(accum):
    """dA = dY W in MXFP8: dY [16384 x 768] cast by quantize_mx (blocks along
    the 768 output features), W [768 x 3072] by quantize_mx_transposed (its
    blocks along the same 768), then fp8_gemm_mx E5M2 x E4M3 -> [16384 x 3072]
    on sampled rows against the oracle."""
    w = workloads.get("gpt2")
    dy, wt = w.dy(), w.weight()
    M, N = dy.shape
    K = wt.shape[1]
    d = to_dev_bf16(dy)
    q_dy = torch.empty((M, N), dtype=torch.uint8, device=DEV)
    e_dy = torch.empty((M, N // 32), dtype=torch.uint8, device=DEV)
    sq.quantize_mx(d, sq.ACT_IDENTITY, sq.E5M2, q_dy, e_dy)
    _, q_wt, e_wt = _run_t(wt, sq.ACT_IDENTITY, sq.E4M3, want_bf16=False)
    y = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    sq.fp8_gemm_mx(q_dy, sq.E5M2, e_dy, q_wt, sq.E4M3, e_wt, y, accum)
    rows = np.sort(np.random.default_rng(29).choice(M, size=64, replace=False))
    ra = O.quantize_mx(dy[rows], O.ACT_IDENTITY, O.E5M2, want_bf16=False)
    rb = _oracle_t(wt, O.ACT_IDENTITY, O.E4M3)
    assert np.array_equal(u8_np(q_dy)[rows], ra.fp8) and np.array_equal(u8_np(e_dy)[rows], ra.scale)
    ref, absref = O.gemm_mx_f64(ra.fp8, O.E5M2, ra.scale, rb.fp8, O.E4M3, rb.scale)
    check_gemm(y.float().cpu().numpy()[rows], ref, absref, "mx dgrad", accum == EXACT,
               lambda sel: fp8_mfma_allowance_mx(ra.fp8, 1, ra.scale, rb.fp8, 0, rb.scale, sel))


def test_transposed_mx_argument_errors():
    h = torch.zeros((96, 128), dtype=torch.bfloat16, device=DEV)
    qt = torch.empty((128, 96), dtype=torch.uint8, device=DEV)
    et = torch.empty((128, 3), dtype=torch.uint8, device=DEV)
    with pytest.raises(sq.Fp8dpError, match="multiple of 64"):
        sq.quantize_mx_transposed(h, sq.ACT_RELU2, sq.E4M3, qt, et)
    h = torch.zeros((64, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(sq.Fp8dpError, match="cols x rows"):
        sq.quantize_mx_transposed(h, sq.ACT_RELU2, sq.E4M3, qt, et)


# ------------------------------------------------------------------ MX split-K
def _mx_operands(rng, M, N, K, fa, fb, spread):
    """Codes and exponents of two spread operands via the oracle's MX cast."""
    def one(rows, fmt):
        x = rng.standard_normal((rows, K)).astype(np.float32)
        x *= np.exp2(rng.integers(-spread, spread + 1, (rows, K // 32, 1)).astype(np.float32)).repeat(
            32, axis=2).reshape(rows, K)
        h = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        r = O.quantize_mx(h, O.ACT_IDENTITY, fmt, want_bf16=False)
        return r.fp8, r.scale
    a8, ea = one(M, fa)
    b8, eb = one(N, fb)
    return a8, ea, b8, eb


def _mx_split(a8, fa, ea, b8, fb, eb, splits, accum):
    M, N = a8.shape[0], b8.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(splits * M * N, dtype=torch.float32, device=DEV)
    sq.fp8_gemm_mx_splitk(to_dev_u8(a8), fa, to_dev_u8(ea), to_dev_u8(b8), fb, to_dev_u8(eb),
                          splits, ws, y, accum)
    return y


@BOTH
@pytest.mark.parametrize("N", [256, 384])
def test_mx_splitk_one_split_equals_mx_gemm(N, accum):
    rng = np.random.default_rng(31 + N)
    a8, ea, b8, eb = _mx_operands(rng, 512, N, 1024, 1, 0, 6)
    y1 = _mx_split(a8, 1, ea, b8, 0, eb, 1, accum)
    y0 = torch.empty_like(y1)
    sq.fp8_gemm_mx(to_dev_u8(a8), 1, to_dev_u8(ea), to_dev_u8(b8), 0, to_dev_u8(eb), y0, accum)
    assert torch.equal(y1.view(torch.int16), y0.view(torch.int16))


# uneven split ranges, fold-only (spreads 3, 6) and fallback tiles (spread 55)
# in exact mode, every format pair
@BOTH
@pytest.mark.parametrize("M,N,K,fa,fb,splits,spread", [(256, 384, 2048, 1, 0, 3, 3),
                                                       (512, 256, 4096, 1, 0, 5, 55),
                                                       (256, 128, 1280, 0, 0, 7, 6),
                                                       (256, 384, 1536, 0, 1, 4, 3),
                                                       (256, 256, 1024, 1, 1, 8, 3)])
def test_mx_splitk_vs_oracle(M, N, K, fa, fb, splits, spread, accum):
    rng = np.random.default_rng(M + N + K + splits + spread)
    a8, ea, b8, eb = _mx_operands(rng, M, N, K, fa, fb, spread)
    y = _mx_split(a8, fa, ea, b8, fb, eb, splits, accum).float().cpu().numpy()
    ref, absref = O.gemm_mx_f64(a8, fa, ea, b8, fb, eb)
    check_gemm(y, ref, absref, f"mx split {splits}", accum == EXACT,
               lambda sel: fp8_mfma_allowance_mx(a8, fa, ea, b8, fb, eb, sel))


@BOTH
def test_mx_wgrad_gpt2(accum):
    """dW [768 x 3072] = dY^T A in MXFP8 at the GPT-2 shape: dY^T and A^T =
    relu2(H)^T from quantize_mx_transposed (blocks along the 16384 tokens),
    K = 16384 split 5 ways, sampled rows against the oracle."""
    w = workloads.get("gpt2")
    dy, h = w.dy(), w.h0()
    _, q_dyt, e_dyt = _run_t(dy, sq.ACT_IDENTITY, sq.E5M2, want_bf16=False)
    _, q_at, e_at = _run_t(h, sq.ACT_RELU2, sq.E4M3, want_bf16=False)
    N, M = q_dyt.shape
    K = q_at.shape[0]
    y = torch.empty((N, K), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(5 * N * K, dtype=torch.float32, device=DEV)
    sq.fp8_gemm_mx_splitk(q_dyt, sq.E5M2, e_dyt, q_at, sq.E4M3, e_at, 5, ws, y, accum)
    rows = np.sort(np.random.default_rng(37).choice(N, size=24, replace=False))
    ra = O.quantize_mx(np.ascontiguousarray(dy.T[rows]), O.ACT_IDENTITY, O.E5M2, want_bf16=False)
    rb = _oracle_t(h, O.ACT_RELU2, O.E4M3)
    assert np.array_equal(u8_np(q_dyt)[rows], ra.fp8) and np.array_equal(u8_np(e_dyt)[rows], ra.scale)
    assert np.array_equal(u8_np(q_at), rb.fp8) and np.array_equal(u8_np(e_at), rb.scale)
    ref, absref = O.gemm_mx_f64(ra.fp8, O.E5M2, ra.scale, rb.fp8, O.E4M3, rb.scale)
    check_gemm(y.float().cpu().numpy()[rows], ref, absref, "mx wgrad", accum == EXACT,
               lambda sel: fp8_mfma_allowance_mx(ra.fp8, 1, ra.scale, rb.fp8, 0, rb.scale, sel))


def test_mx_splitk_argument_errors():
    a = torch.zeros((256, 512), dtype=torch.uint8, device=DEV)
    e = torch.zeros((256, 16), dtype=torch.uint8, device=DEV)
    y = torch.empty((256, 256), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(4 * 256 * 256, dtype=torch.float32, device=DEV)
    with pytest.raises(sq.Fp8dpError, match="splits"):
        sq.fp8_gemm_mx_splitk(a, 0, e, a, 0, e, 5, ws, y)      # K < 128 * splits
    with pytest.raises(sq.Fp8dpError, match="workspace"):
        sq.fp8_gemm_mx_splitk(a, 0, e, a, 0, e, 4, ws[:10], y)
