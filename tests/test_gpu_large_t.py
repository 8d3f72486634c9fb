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
row-major codes.
"""
import numpy as np
import pytest
import torch

import oracle as O
import scaled_quantization_amd as sq
from gpu_util import DEV, bf16_np, oracle_quantize, u8_np

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
