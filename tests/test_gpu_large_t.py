"""The transposed casts and the code transpose past 2^31 bytes (GPU).

"FP8 Training & Inference", FP8 Training Recipe: the weight gradient reads
the activation's codes transposed.  Here an activation H[65536 x 40960] BF16
(5 GiB; its codes 2.5 GiB), so both the kernels' input offsets and their
code offsets pass 2^31 bytes.  H is seeded N(0, 2) drawn on the GPU by
torch's generator (no arithmetic of the method); sampled 128-column blocks
(the first, one in the middle, the last) and 64-row blocks are copied back
and checked against the oracle, and the kernels against each other over the
whole tensors: quantize_mx_transposed's codes and E8M0 exponents against
the oracle's quantize_mx of the transposed block; quantize_fused_transposed's
row-major codes against the oracle's quantize, its transposed codes against
torch's transpose of the sampled blocks and against fp8_transpose of its
row-major codes; quantize_fused over the same elements against the
transposed cast's row-major codes.  And the exact GEMM with A8[163840 x
16384] (2.5 GiB of codes) on sampled rows against the oracle's float64 GEMM
("FP8 training: what it is and how it works", Step 3: FP32 sums of exact
products) to the plain bound.
"""
import numpy as np
import pytest
import torch

import oracle as O
import scaled_quantization_amd as sq
from gpu_util import DEV, bf16_np, check_gemm, oracle_quantize, u8_np

pytestmark = pytest.mark.gpu

ROWS, COLS_N = 65536, 40960
COLS = (0, 20480 + 128, COLS_N - 128)     # 128-column blocks: first, middle, last


@pytest.fixture(scope="module")
def big_h():
    g = torch.Generator(device=DEV)
    g.manual_seed(21)
    h = torch.empty((ROWS, COLS_N), dtype=torch.bfloat16, device=DEV)
    for r in range(0, ROWS, 4096):
        h[r:r + 4096] = (torch.randn((4096, COLS_N), generator=g, device=DEV) * 2).to(
            torch.bfloat16)
    yield h
    del h
    torch.cuda.empty_cache()


def test_offsets_pass_2_31():
    assert ROWS * COLS_N > 2 ** 31 and ROWS * COLS_N * 2 > 2 ** 31


def test_mx_transposed_cast_past_2_31(big_h):
    h = big_h
    qt = torch.empty((COLS_N, ROWS), dtype=torch.uint8, device=DEV)
    et = torch.empty((COLS_N, ROWS // 32), dtype=torch.uint8, device=DEV)
    sq.quantize_mx_transposed(h, sq.ACT_RELU2, sq.E4M3, qt, et)
    for c0 in COLS:
        blk = bf16_np(h[:, c0:c0 + 128].contiguous())
        r = O.quantize_mx(np.ascontiguousarray(blk.T), O.ACT_RELU2, O.E4M3, want_bf16=False)
        assert np.array_equal(u8_np(qt[c0:c0 + 128]), r.fp8), c0
        assert np.array_equal(u8_np(et[c0:c0 + 128]), r.scale), c0


def test_transposed_cast_and_transpose_past_2_31(big_h):
    h = big_h
    st = sq.TensorState(sq.E4M3, 1, 1.25, 20.0)
    scale = O.State(O.E4M3, 1, 1.25, 20.0).scale
    a8 = torch.empty((ROWS, COLS_N), dtype=torch.uint8, device=DEV)
    qt = torch.empty((COLS_N, ROWS), dtype=torch.uint8, device=DEV)
    sq.quantize_fused_transposed(h, sq.ACT_RELU2, sq.E4M3, st, qt, None, a8)
    for r0 in (0, ROWS // 2, ROWS - 64):
        r = oracle_quantize(bf16_np(h[r0:r0 + 64]), O.ACT_RELU2, O.E4M3, O.PER_TENSOR, scale,
                            want_bf16=False)
        assert np.array_equal(u8_np(a8[r0:r0 + 64]), r.fp8), r0
    for c0 in COLS:
        assert torch.equal(qt[c0:c0 + 128], a8[:, c0:c0 + 128].t().contiguous()), c0
    at = torch.empty((COLS_N, ROWS), dtype=torch.uint8, device=DEV)
    sq.fp8_transpose(a8, at)
    assert torch.equal(at, qt)


def test_quantize_fused_past_2_31_equals_transposed_cast(big_h):
    # the row-major cast over 2.68 G elements equals the transposed cast's
    # row-major codes (checked against the oracle above), state included
    h = big_h
    st1 = sq.TensorState(sq.E4M3, 1, 1.25, 20.0)
    st2 = sq.TensorState(sq.E4M3, 1, 1.25, 20.0)
    a8 = torch.empty((ROWS, COLS_N), dtype=torch.uint8, device=DEV)
    qt = torch.empty((COLS_N, ROWS), dtype=torch.uint8, device=DEV)
    sq.quantize_fused_transposed(h, sq.ACT_RELU2, sq.E4M3, st1, qt, None, a8)
    del qt
    b8 = torch.empty_like(a8)
    sq.quantize_fused(h, sq.ACT_RELU2, sq.E4M3, sq.PER_TENSOR, st2, None, b8)
    assert torch.equal(a8, b8)
    d1, d2 = st1.read(), st2.read()
    assert d1["amax_acc"] == d2["amax_acc"] and d1["sat_acc"] == d2["sat_acc"] > 0


def test_exact_gemm_past_2_31():
    # A8[163840 x 16384]: 2.5 GiB of codes, row offsets past 2^31 bytes;
    # 32 sampled rows (first, middle, last among them) against the oracle's
    # float64 GEMM to the plain bound
    M, N, K = 163840, 256, 16384
    assert M * K > 2 ** 31
    t = O.fp8_decode_table(O.E4M3)
    near = torch.from_numpy(np.flatnonzero(np.isfinite(t) & (np.abs(t) >= 0.5) &
                                           (np.abs(t) <= 8)).astype(np.int64)).to(DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(22)
    a8 = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    for r in range(0, M, 8192):
        a8[r:r + 8192] = near[torch.randint(0, near.numel(), (8192, K), generator=g,
                                            device=DEV)].to(torch.uint8)
    w8 = near[torch.randint(0, near.numel(), (N, K), generator=g, device=DEV)].to(torch.uint8)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    sa = torch.full((1,), 0.5, dtype=torch.float32, device=DEV)
    sb = torch.full((1,), 0.25, dtype=torch.float32, device=DEV)
    sq.fp8_gemm_scaled(a8, sq.E4M3, w8, sq.E4M3, sq.PER_TENSOR, sa, sb, y, sq.ACCUM_EXACT)
    rng = np.random.default_rng(22)
    rows = np.unique(np.concatenate([[0, 1, M // 2, M // 2 + 1, M - 2, M - 1],
                                     rng.integers(0, M, 26)]))
    a_rows = u8_np(a8[torch.from_numpy(rows).to(DEV)])
    ref, absref = O.gemm_f64(a_rows, O.E4M3, u8_np(w8), O.E4M3, O.PER_TENSOR, 2.0, 4.0)
    yr = y[torch.from_numpy(rows).to(DEV)].float().cpu().numpy()
    check_gemm(yr, ref, absref, f"{M}x{N}x{K}")
