"""Scaled FP8 GEMM against the oracle's float64 reference (GPU).

Acceptance bound per output element, from the benchmark spec of the path:
    |y - ref| <= 2^-8 |ref| + 1e-5 * sum_k |a_k b_k|
with ref and the absolute sum in float64 over the dequantized codes ("FP8
training: what it is and how it works", Step 3: FP8 inputs are acceptable
only when the sum is kept in a wide format; "FP8 Training & Inference",
Per-Tensor Scaling).  BF16 output rounding alone is at most 2^-9 relative.

Two accumulation modes:
* ACCUM_EXACT (codes widened to FP16, FP16 matrix instructions summing at
  FP32; the default and the benchmarked path) must meet that bound on every
  element of every case, adversarial inputs included.
* ACCUM_MFMA_FP8 (the FP8 matrix instructions, which truncate small products
  in groups of 8 -- see gpu_util.fp8_mfma_allowance) is checked against the
  same plain bound.  Where elements leave it, the truncation rule must
  account for each of them (a diagnostic: any other error, e.g. a wrong
  index, still fails), and the case is reported as an expected failure with
  the count: the mode does not meet the contract on such data.

The GEMM's inputs are the oracle's own quantization of the seeded workloads,
uploaded, so no oracle input comes from the device path.  Full outputs at the
tiny size; every column of seeded rows at the larger sizes.
"""
import numpy as np
import pytest
import torch

import oracle as O
import scaled_quantization_amd as sq
import workloads
from gpu_util import (DEV, check_gemm, fp8_mfma_allowance, oracle_gemm_rows, oracle_quantize,
                      to_dev_u8)

pytestmark = pytest.mark.gpu
EXACT, FP8 = sq.ACCUM_EXACT, sq.ACCUM_MFMA_FP8
BOTH = pytest.mark.parametrize("accum", [EXACT, FP8], ids=["exact", "fp8"])


def _dev_f32(x):
    return torch.from_numpy(np.ascontiguousarray(np.atleast_1d(np.asarray(x, np.float32)))).to(DEV)


def _gemm(a8, fa, w8, fb, mode, sa_inv, sb_inv, accum):
    M, K = a8.shape
    N = w8.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    sq.fp8_gemm_scaled(to_dev_u8(a8), fa, to_dev_u8(w8), fb, mode, _dev_f32(sa_inv),
                       _dev_f32(sb_inv), y, accum)
    return y.float().cpu().numpy()


def _check(y, ref, absref, what, accum=EXACT, allowance=None):
    check_gemm(y, ref, absref, what, accum == EXACT, allowance)


def _tensor_case(name, t=0):
    w = workloads.get(name)
    h = w.h_step(t) if name == "tiny" else w.h0()
    st = O.State(O.E4M3, 1, w.margin, w.initial_amax)
    # one step of delayed scaling so the cast uses a realistic scale
    r0 = oracle_quantize(h, O.ACT_RELU2, O.E4M3, O.PER_TENSOR, st.scale, want_bf16=False,
                         want_fp8=False)
    st.accumulate(r0.amax_bits, r0.sat)
    st.update()
    r = oracle_quantize(h, O.ACT_RELU2, O.E4M3, O.PER_TENSOR, st.scale, want_bf16=False)
    q_w, s_w, si_w = O.quantize_weight_tensor(w.weight(), O.E4M3)
    return w, r.fp8, st.scale, st.scale_inv, q_w, s_w, si_w


@BOTH
@pytest.mark.parametrize("t", [0, 1, 2, 3])
def test_tiny_gemm_all_outputs(t, accum):
    # every output of every delayed-scaling step of the tiny workload
    w, a8, s_a, si_a, w8, s_w, si_w = _tensor_case("tiny", t=t)
    y = _gemm(a8, 0, w8, 0, sq.PER_TENSOR, si_a, si_w, accum)
    ref, absref = O.gemm_f64(a8, O.E4M3, w8, O.E4M3, O.PER_TENSOR, s_a, s_w)
    _check(y, ref, absref, f"tiny step {t}", accum,
           lambda sel: fp8_mfma_allowance(a8, 0, w8, 0, O.PER_TENSOR, s_a, s_w, sel))


@BOTH
@pytest.mark.parametrize("name,nrows", [("gpt2", 512), ("large", 48)])
def test_per_tensor_gemm_full_size_sampled_rows(name, nrows, accum):
    w, a8, s_a, si_a, w8, s_w, si_w = _tensor_case(name)
    y = _gemm(a8, 0, w8, 0, sq.PER_TENSOR, si_a, si_w, accum)
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(w.M, size=nrows, replace=False))
    rows[0], rows[-1] = 0, w.M - 1
    ref, absref = oracle_gemm_rows(a8, O.E4M3, w8, O.E4M3, O.PER_TENSOR, s_a, s_w, rows)
    assert np.isfinite(y).all()
    _check(y[rows], ref, absref, name, accum,
           lambda sel: fp8_mfma_allowance(a8, 0, w8, 0, O.PER_TENSOR, s_a, s_w, rows[sel]))


@BOTH
def test_fine_grained_block_scaled_gemm_sampled_rows(accum):
    w = workloads.get("fine")
    h = w.h0()
    r = oracle_quantize(h, O.ACT_IDENTITY, O.E4M3, O.PER_GROUP128, want_bf16=False)
    q_w, si_w, s_w = O.quantize_weight_blocks(w.weight(), O.E4M3, with_scale=True)
    s_a = r.group_scale
    y = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=DEV)
    sq.fp8_gemm_scaled(to_dev_u8(r.fp8), 0, to_dev_u8(q_w), 0, sq.PER_GROUP128,
                       torch.from_numpy(r.group_scale_inv).to(DEV),
                       torch.from_numpy(si_w).to(DEV), y, accum)
    yv = y.float().cpu().numpy()
    rng = np.random.default_rng(8)
    rows = np.sort(rng.choice(w.M, size=128, replace=False))
    rows[0], rows[-1] = 0, w.M - 1
    ref, absref = oracle_gemm_rows(r.fp8, O.E4M3, q_w, O.E4M3, O.PER_GROUP128, s_a, s_w, rows)
    assert np.isfinite(yv).all()
    _check(yv[rows], ref, absref, "fine", accum,
           lambda sel: fp8_mfma_allowance(r.fp8, 0, q_w, 0, O.PER_GROUP128, s_a, s_w, rows[sel]))


@BOTH
def test_gpt2_per_group_gemm_full_size_sampled_rows(accum):
    # the benchmark's per-group launch: the GPT-2 activation (relu2) cast with
    # per-128 group scales, the weight with 128 x 128 block scales; in FP8
    # mode on a 256-CU GPU this shape runs the 256 x 192 per-group tiles, in
    # exact mode the 256 x 128 ones
    w = workloads.get("gpt2")
    r = oracle_quantize(w.h0(), O.ACT_RELU2, O.E4M3, O.PER_GROUP128, want_bf16=False)
    q_w, si_w, s_w = O.quantize_weight_blocks(w.weight(), O.E4M3, with_scale=True)
    y = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=DEV)
    sq.fp8_gemm_scaled(to_dev_u8(r.fp8), 0, to_dev_u8(q_w), 0, sq.PER_GROUP128,
                       torch.from_numpy(r.group_scale_inv).to(DEV),
                       torch.from_numpy(si_w).to(DEV), y, accum)
    yv = y.float().cpu().numpy()
    rng = np.random.default_rng(9)
    rows = np.sort(rng.choice(w.M, size=256, replace=False))
    rows[0], rows[-1] = 0, w.M - 1
    ref, absref = oracle_gemm_rows(r.fp8, O.E4M3, q_w, O.E4M3, O.PER_GROUP128, r.group_scale,
                                   s_w, rows)
    assert np.isfinite(yv).all()
    _check(yv[rows], ref, absref, "gpt2 per-group", accum,
           lambda sel: fp8_mfma_allowance(r.fp8, 0, q_w, 0, O.PER_GROUP128, r.group_scale, s_w, rows[sel]))


@BOTH
@pytest.mark.parametrize("K", [128, 256, 1024, 4096, 16384])
def test_random_full_range_codes_over_long_k(K, accum):
    # every finite code equally likely: products span ~2^36, the hardest case
    # for the FP8 instructions' truncation ("FP8 training ...", Step 3: about
    # 14 bits of accumulation gave nearly 2% error at K = 4096 on one GPU)
    rng = np.random.default_rng(K)
    M, N = 256, 256
    t = np.flatnonzero(np.isfinite(O.fp8_decode_table(O.E4M3)))
    a8 = rng.choice(t, size=(M, K)).astype(np.uint8)
    w8 = rng.choice(t, size=(N, K)).astype(np.uint8)
    y = _gemm(a8, 0, w8, 0, sq.PER_TENSOR, 1.0 / 64, 1.0 / 32, accum)
    ref, absref = O.gemm_f64(a8, O.E4M3, w8, O.E4M3, O.PER_TENSOR, 64.0, 32.0)
    if accum == EXACT:
        # FP32-accurate accumulation: beyond the BF16 output rounding (at most
        # 2^-8 relative) the error stays far inside the 1e-5 term
        assert np.all(np.abs(y - ref) <= (2.0 ** -8) * np.abs(ref) + 1e-6 * absref)
    _check(y, ref, absref, f"K={K}", accum,
           lambda sel: fp8_mfma_allowance(a8, 0, w8, 0, O.PER_TENSOR, 64.0, 32.0, sel))


@BOTH
@pytest.mark.parametrize("M,N,K", [(256, 384, 640), (512, 768, 512)])
@pytest.mark.parametrize("fa,fb", [(0, 1), (1, 0), (1, 1)])
def test_operand_format_combinations(fa, fb, M, N, K, accum):
    # 256 x 384: small-tile per-group kernel (K % 512 != 0), 256 x 128 /
    # 256 x 192 large tiles per tensor; 512 x 768 x 512: the large-tile
    # per-group kernel
    rng = np.random.default_rng(10 + fa * 2 + fb + M)
    ta = np.flatnonzero(np.isfinite(O.fp8_decode_table(fa)))
    tb = np.flatnonzero(np.isfinite(O.fp8_decode_table(fb)))
    a8 = rng.choice(ta, size=(M, K)).astype(np.uint8)
    w8 = rng.choice(tb, size=(N, K)).astype(np.uint8)
    for mode in (sq.PER_TENSOR, sq.PER_GROUP128):
        if mode == sq.PER_TENSOR:
            sa, sb = np.float32(2.0 ** -10), np.float32(3.0)
        else:
            sa = (2.0 ** rng.integers(-6, 6, (M, K // 128))).astype(np.float32)
            sb = (2.0 ** rng.integers(-6, 6, (N // 128, K // 128))).astype(np.float32)
        y = _gemm(a8, fa, w8, fb, mode, 1 / sa, 1 / sb, accum)
        ref, absref = O.gemm_f64(a8, fa, w8, fb, mode, sa, sb)
        _check(y, ref, absref, f"fa={fa} fb={fb} mode={mode}", accum,
               lambda sel: fp8_mfma_allowance(a8, fa, w8, fb, mode, sa, sb, sel))


@BOTH
@pytest.mark.parametrize("fmt", [0, 1], ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("M", [384, 512])
def test_identity_weight_returns_every_code_exactly(fmt, M, accum):
    # a scaled identity weight: every product group holds one nonzero product,
    # so both modes must reproduce each decoded input code exactly
    K = 256
    t = O.fp8_decode_table(fmt)
    fin = np.flatnonzero(np.isfinite(t)).astype(np.uint8)
    # M = 384: 256 rows on the large tiles and 128 on the small-tile kernel
    a8 = np.resize(fin, (M, K)).astype(np.uint8)
    one = int(O.fp8_encode(np.array([1.0], np.float32), fmt)[0])
    w8 = np.zeros((K, K), dtype=np.uint8)
    np.fill_diagonal(w8, one)
    y = _gemm(a8, fmt, w8, fmt, sq.PER_TENSOR, 0.5, 1.0, accum)
    exp = torch.from_numpy((t[a8] * 0.5).astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(y, exp)


@BOTH
@pytest.mark.parametrize("M", [128, 256])
def test_all_max_inputs_closed_form(M, accum):
    K = 4096
    a8 = np.full((M, K), 0x7E, dtype=np.uint8)
    w8 = np.full((256, K), 0xFE, dtype=np.uint8)
    y = _gemm(a8, 0, w8, 0, sq.PER_TENSOR, 1.0 / 448, 1.0 / 448, accum)
    assert np.all(y == -float(K))


def test_fp8_instruction_truncation_and_exact_mode():
    # One product group holds 448 and seven 2^-6 values; the next group
    # cancels the 448.  The FP8 instructions drop the small products (below
    # 2^-13 of the group's largest exponent sum); the exact mode keeps them.
    K = 128
    a8 = np.zeros((128, K), dtype=np.uint8)
    a8[:, 0] = 0x7E                                    # 448
    a8[:, 1:8] = int(O.fp8_encode(np.array([2.0 ** -6], np.float32), 0)[0])
    a8[:, 8] = 0x7E
    w8 = np.zeros((128, K), dtype=np.uint8)
    w8[:, 0:8] = 0x38                                  # +1
    w8[:, 8] = 0xB8                                    # -1
    y8 = _gemm(a8, 0, w8, 0, sq.PER_TENSOR, 1.0, 1.0, FP8)
    ye = _gemm(a8, 0, w8, 0, sq.PER_TENSOR, 1.0, 1.0, EXACT)
    assert np.all(ye == 7 * 2.0 ** -6)
    assert np.all(y8 == 0.0)


@BOTH
def test_non_multiple_of_eight_tile_grid(accum):
    # 3 x 5 = 15 tiles: the XCD renumbering falls back to the identity order
    rng = np.random.default_rng(4)
    M, N, K = 384, 640, 384
    t = O.fp8_decode_table(O.E4M3)
    near = np.flatnonzero(np.isfinite(t) & (np.abs(t) >= 1) & (np.abs(t) <= 16))
    a8 = rng.choice(near, size=(M, K)).astype(np.uint8)
    w8 = rng.choice(near, size=(N, K)).astype(np.uint8)
    y = _gemm(a8, 0, w8, 0, sq.PER_TENSOR, 0.25, 0.125, accum)
    ref, absref = O.gemm_f64(a8, O.E4M3, w8, O.E4M3, O.PER_TENSOR, 4.0, 8.0)
    _check(y, ref, absref, "15 tiles", accum,
           lambda sel: fp8_mfma_allowance(a8, 0, w8, 0, O.PER_TENSOR, 4.0, 8.0, sel))


@pytest.mark.parametrize("M,N,K", [(512, 384, 256), (2304, 768, 640), (4096, 4096, 256),
                                   (256, 768, 128), (512, 640, 384), (768, 384, 256),
                                   (512, 384, 1280), (1024, 512, 1152), (512, 1024, 384),
                                   (2048, 2048, 640), (256, 256, 128)])
@BOTH
def test_large_tile_paths(M, N, K, accum):
    # per-tensor shapes that take the 256 x 192, 256 x 256 (FP8 mode only)
    # and 256 x 128 workgroup tiles: tile counts below, at and above the grid
    # renumbering's multiple of 8, and 1, 2, 3 and 9-10 stages of 128 k (the
    # pipeline's prologue, steady state and tail)
    rng = np.random.default_rng(M + N + K)
    t = O.fp8_decode_table(O.E4M3)
    near = np.flatnonzero(np.isfinite(t) & (np.abs(t) >= 0.5) & (np.abs(t) <= 8))
    a8 = rng.choice(near, size=(M, K)).astype(np.uint8)
    w8 = rng.choice(near, size=(N, K)).astype(np.uint8)
    y = _gemm(a8, 0, w8, 0, sq.PER_TENSOR, 0.5, 0.25, accum)
    rows = np.unique(np.concatenate([np.arange(0, M, max(1, M // 64)), [M - 1]]))
    ref, absref = O.gemm_f64(a8, O.E4M3, w8, O.E4M3, O.PER_TENSOR, 2.0, 4.0, rows=rows)
    _check(y[rows], ref, absref, f"{M}x{N}x{K}", accum,
           lambda sel: fp8_mfma_allowance(a8, 0, w8, 0, O.PER_TENSOR, 2.0, 4.0, rows[sel]))


@pytest.mark.parametrize("M,N,K", [(5376, 3072, 512), (33024, 384, 256), (20480, 1024, 1024),
                                   (16384, 3072, 2048)])
@BOTH
def test_persistent_grid_paths(M, N, K, accum):
    # more tiles than compute units with at most 16 stages of K: the
    # persistent grid, whose workgroups run tile after tile through one
    # pipeline -- 336 tiles (some workgroups run two, some one), 258 tiles
    # (not a multiple of 8: plain tile order), 320 tiles of 256 x 256, and
    # 1024 tiles of 16 stages; rows sampled from every tile row-block
    rng = np.random.default_rng(M + 3 * N + K)
    t = O.fp8_decode_table(O.E4M3)
    near = np.flatnonzero(np.isfinite(t) & (np.abs(t) >= 0.5) & (np.abs(t) <= 8))
    a8 = rng.choice(near, size=(M, K)).astype(np.uint8)
    w8 = rng.choice(near, size=(N, K)).astype(np.uint8)
    y = _gemm(a8, 0, w8, 0, sq.PER_TENSOR, 0.5, 0.25, accum)
    rows = np.unique(np.concatenate([np.arange(0, M, 256), np.arange(255, M, 256),
                                     rng.integers(0, M, 16)]))
    ref, absref = O.gemm_f64(a8, O.E4M3, w8, O.E4M3, O.PER_TENSOR, 2.0, 4.0, rows=rows)
    _check(y[rows], ref, absref, f"{M}x{N}x{K}", accum,
           lambda sel: fp8_mfma_allowance(a8, 0, w8, 0, O.PER_TENSOR, 2.0, 4.0, rows[sel]))


def _group_case(M, N, K, fa, fb):
    rng = np.random.default_rng(M * 7 + N + K)
    ta = O.fp8_decode_table(fa)
    tb = O.fp8_decode_table(fb)
    near_a = np.flatnonzero(np.isfinite(ta) & (np.abs(ta) >= 0.25) & (np.abs(ta) <= 16))
    near_b = np.flatnonzero(np.isfinite(tb) & (np.abs(tb) >= 0.25) & (np.abs(tb) <= 16))
    a8 = rng.choice(near_a, size=(M, K)).astype(np.uint8)
    w8 = rng.choice(near_b, size=(N, K)).astype(np.uint8)
    sa = rng.uniform(0.05, 40.0, (M, K // 128)).astype(np.float32)
    sb = rng.uniform(0.05, 40.0, (N // 128, K // 128)).astype(np.float32)
    return a8, w8, sa, sb


# K = 128 .. 1280 not multiples of 512 (and M = 1024 with 768 not): the 128 x 128
# tile kernel; K = 512, 1536, 2048, 4096 with M a multiple of 256: the 256 x 128
# tile kernel with transposed partial sums and the scales' four-stage ring
@pytest.mark.parametrize("M,N,K,fa,fb", [(256, 128, 128, 0, 0), (512, 384, 256, 0, 0),
                                         (768, 640, 1280, 0, 1), (2304, 1024, 384, 1, 0),
                                         (1024, 256, 640, 1, 1), (256, 128, 512, 0, 0),
                                         (768, 384, 1536, 0, 1), (512, 640, 2048, 1, 0),
                                         (2304, 256, 4096, 1, 1)])
@BOTH
def test_group_scaled_shapes(M, N, K, fa, fb, accum):
    # per-group FP8: per-stage partial sums promoted by sa[m, g] sb[n / 128, g]
    # over 1 to 32 stages, tile counts on and off the renumbering's multiple
    # of 8, every format pair, scales that are not powers of two
    a8, w8, sa, sb = _group_case(M, N, K, fa, fb)
    y = _gemm(a8, fa, w8, fb, sq.PER_GROUP128, 1 / sa, 1 / sb, accum)
    rows = np.unique(np.concatenate([np.arange(0, M, max(1, M // 48)), [M - 1]]))
    ref, absref = O.gemm_f64(a8, fa, w8, fb, O.PER_GROUP128, sa, sb, rows=rows)
    _check(y[rows], ref, absref, f"group {M}x{N}x{K} fa={fa} fb={fb}", accum,
           lambda sel: fp8_mfma_allowance(a8, fa, w8, fb, O.PER_GROUP128, sa, sb, rows[sel]))


# Ragged M (a token count that does not fill a tile): the rows that fill
# whole 256-row tiles run on the large-tile kernels, the rest on the small-tile
# kernel, which reads row M - 1 in place of rows past the end and does not
# store them.  Rows past M in the output buffer must keep their contents; rows
# below the last whole tile must equal the product of those rows alone, bit
# for bit (the same kernel computes them); every row meets the bound.
@pytest.mark.parametrize("M", [1, 37, 128, 255, 333, 4096 + 77])
@pytest.mark.parametrize("mode,accum", [(sq.PER_TENSOR, FP8), (sq.PER_GROUP128, FP8),
                                        (sq.PER_TENSOR, EXACT), (sq.PER_GROUP128, EXACT)],
                         ids=["tensor-fp8", "group-fp8", "tensor-exact", "group-exact"])
def test_ragged_rows(M, mode, accum):
    N, K = 384, 1024
    a8, w8, sa, sb = _group_case(M, N, K, 0, 0)
    if mode == sq.PER_TENSOR:
        sa, sb = np.float32(0.75), np.float32(3.0)
    guard = 3
    y_all = torch.empty((M + guard, N), dtype=torch.bfloat16, device=DEV)
    y_all.view(torch.int16).fill_(0x7FC1)   # a NaN pattern no output can take
    sq.fp8_gemm_scaled(to_dev_u8(a8), 0, to_dev_u8(w8), 0, mode, _dev_f32(1 / sa),
                       _dev_f32(1 / sb), y_all[:M], accum)
    bits = y_all.view(torch.int16).cpu().numpy()
    assert np.all(bits[M:] == 0x7FC1), "rows past M were written"
    y = y_all[:M].float().cpu().numpy()
    rows = np.arange(M) if M <= 512 else np.unique(np.concatenate(
        [np.arange(0, M, 61), np.arange(M - 90, M)]))
    ref, absref = O.gemm_f64(a8, 0, w8, 0, mode, sa, sb, rows=rows)
    Mb = M // 256 * 256
    if Mb > 0:
        sa_b = sa if mode == sq.PER_TENSOR else sa[:Mb]
        y_b = _gemm(a8[:Mb], 0, w8, 0, mode, 1 / sa_b, 1 / sb, accum)
        assert np.array_equal(y[:Mb].view(np.uint32), y_b.view(np.uint32))
    _check(y[rows], ref, absref, f"ragged M={M} mode={mode}", accum,
           lambda sel: fp8_mfma_allowance(a8, 0, w8, 0, mode, sa, sb, rows[sel]))


# On a 256-CU GPU these shapes take the 256 x 192 per-group tiles (one round
# of 256 tiles where 256 x 128 tiles need two); their column halves take the
# 256 x 128 tiles.  Each output's arithmetic does not depend on which tile
# computes it, so the halves must agree with the whole bit for bit.
@pytest.mark.parametrize("M,N,K,fa,fb", [(16384, 768, 512, 0, 0), (8192, 1536, 1024, 1, 0)])
def test_group_wide_tiles_match_narrow_tiles(M, N, K, fa, fb):
    a8, w8, sa, sb = _group_case(M, N, K, fa, fb)
    y = _gemm(a8, fa, w8, fb, sq.PER_GROUP128, 1 / sa, 1 / sb, FP8)
    h = N // 2
    left = _gemm(a8, fa, w8[:h], fb, sq.PER_GROUP128, 1 / sa, 1 / sb[: h // 128], FP8)
    right = _gemm(a8, fa, w8[h:], fb, sq.PER_GROUP128, 1 / sa, 1 / sb[h // 128:], FP8)
    whole = np.concatenate([left, right], axis=1)
    diff = np.flatnonzero(y.view(np.uint32) != whole.view(np.uint32))
    assert diff.size == 0, f"{diff.size} outputs differ, first at {np.unravel_index(diff[0], y.shape)}"
    rows = np.unique(np.concatenate([np.arange(0, M, M // 24), [M - 1]]))
    ref, absref = O.gemm_f64(a8, fa, w8, fb, O.PER_GROUP128, sa, sb, rows=rows)
    _check(y[rows], ref, absref, f"wide group tiles {M}x{N}x{K}", FP8,
           lambda sel: fp8_mfma_allowance(a8, fa, w8, fb, O.PER_GROUP128, sa, sb, rows[sel]))


@pytest.mark.parametrize("M,N,K", [(512, 384, 2048), (256, 256, 512)])
@BOTH
def test_group_scaled_kernels_agree(M, N, K, accum):
    """Scale arrays 4 bytes off 16-byte alignment send a K % 512 == 0 problem
    to the 128 x 128 tile kernel instead of the ring kernel: both meet the
    bound (in FP8 mode they differ by the FP8 instructions' truncation: the
    two order a stage's k values differently inside the instruction)."""
    a8, w8, sa, sb = _group_case(M, N, K, 0, 0)
    y = _gemm(a8, 0, w8, 0, sq.PER_GROUP128, 1 / sa, 1 / sb, accum)

    def off4(x):
        x = np.ascontiguousarray(x, np.float32)
        buf = torch.zeros(x.size + 4, dtype=torch.float32, device=DEV)
        v = buf[1:1 + x.size].view(x.shape)
        v.copy_(torch.from_numpy(x).to(DEV))
        assert v.data_ptr() % 16 == 4
        return v

    y2 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    sq.fp8_gemm_scaled(to_dev_u8(a8), 0, to_dev_u8(w8), 0, sq.PER_GROUP128, off4(1 / sa),
                       off4(1 / sb), y2, accum)
    y2 = y2.float().cpu().numpy()
    rows = np.arange(M)
    ref, absref = O.gemm_f64(a8, 0, w8, 0, O.PER_GROUP128, sa, sb, rows=rows)
    for got, what in ((y2, "small-tile kernel"), (y, "ring kernel")):
        _check(got, ref, absref, what, accum,
               lambda sel: fp8_mfma_allowance(a8, 0, w8, 0, O.PER_GROUP128, sa, sb, rows[sel]))


@pytest.mark.parametrize("mode", [sq.PER_TENSOR, sq.PER_GROUP128], ids=["tensor", "group"])
@pytest.mark.parametrize("accum", [FP8, EXACT], ids=["fp8", "exact"])
def test_zero_operand_gives_positive_zero(mode, accum):
    # every product is zero, so every output is the oracle's +0 (positive
    # zero bits), whatever the scales and the other operand
    M, N, K = 512, 384, 1024
    a8, w8, sa, sb = _group_case(M, N, K, 0, 0)
    a8 = np.zeros_like(a8)
    if mode == sq.PER_TENSOR:
        sa, sb = np.float32(0.75), np.float32(3.0)
    y = _gemm(a8, 0, w8, 0, mode, 1 / sa, 1 / sb, accum)
    assert not np.any(y.view(np.uint32))
