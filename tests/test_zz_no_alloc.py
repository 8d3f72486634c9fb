"""The no-allocation split-K GEMM against the split-K GEMM with a workspace (GPU).

fp8_gemm_scaled_splitk_noalloc runs the same kernels as
fp8_gemm_scaled_splitk with the library's per-GPU scratch array in place of
the caller's workspace, so its output must equal the workspace form's bit for
bit.  Two calls in a row, the second on a smaller input (the array keeps the
first call's partials, which the second must not read), through the C ABI;
then the size limit (16 Mi floats of partials) is rejected without a launch.
The workspace form itself is held to the oracle by the backward GEMM tests.
"""
import numpy as np
import pytest
import torch

import oracle as O
import scaled_quantization_amd as sq
from gpu_util import DEV, check_gemm, oracle_gemm_rows, to_dev_u8

pytestmark = pytest.mark.gpu


def _codes(rng, shape, fmt):
    t = O.fp8_decode_table(fmt)
    ok = np.flatnonzero(np.isfinite(t) & (np.abs(t) >= 0.25) & (np.abs(t) <= 16.0))
    return rng.choice(ok, size=shape).astype(np.uint8)


def _f32(x):
    return torch.tensor([x], dtype=torch.float32, device=DEV)


def _raw_noalloc(a, fa, b, fb, splits, sa, sb, y, accum):
    M, K = a.shape
    N = b.shape[0]
    return sq.lib().fp8_gemm_scaled_splitk_noalloc(
        a.data_ptr(), fa, b.data_ptr(), fb, M, N, K, splits, accum, sa.data_ptr(), sb.data_ptr(),
        y.data_ptr(), torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("accum", [sq.ACCUM_EXACT, sq.ACCUM_MFMA_FP8], ids=["exact", "fp8"])
def test_noalloc_equals_workspace_form_on_two_calls(accum):
    rng = np.random.default_rng(1234 + accum)
    # first call: 768 x 3072 output, K 16384 in 5 splits (11.8 Mi floats of partials);
    # second: a smaller input, 256 x 384, K 1024 in 3 uneven splits
    for (M, N, K, splits, fa, fb) in ((768, 3072, 16384, 5, 1, 0), (256, 384, 1024, 3, 0, 1)):
        a8, b8 = _codes(rng, (M, K), fa), _codes(rng, (N, K), fb)
        a, b = to_dev_u8(a8), to_dev_u8(b8)
        sa, sb = _f32(0.5), _f32(0.25)
        y_ws = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        ws = torch.empty(splits * M * N, dtype=torch.float32, device=DEV)
        sq.fp8_gemm_scaled_splitk(a, fa, b, fb, splits, sa, sb, ws, y_ws, accum)
        y_na = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        assert _raw_noalloc(a, fa, b, fb, splits, sa, sb, y_na, accum) == 0, \
            sq.lib().fp8dp_last_error()
        torch.cuda.synchronize()
        assert torch.equal(y_ws.view(torch.int16), y_na.view(torch.int16)), (M, N, K, splits)
        if accum == sq.ACCUM_EXACT:
            rows = np.unique(np.concatenate([np.arange(0, M, max(1, M // 16)), [M - 1]]))
            ref, absref = oracle_gemm_rows(a8, fa, b8, fb, O.PER_TENSOR, 2.0, 4.0, rows)
            check_gemm(y_na.float().cpu().numpy()[rows], ref, absref, f"noalloc {M}x{N}x{K}")


def test_noalloc_binding_and_limit():
    rng = np.random.default_rng(7)
    M, N, K, splits = 512, 256, 2048, 4
    a8, b8 = _codes(rng, (M, K), 0), _codes(rng, (N, K), 0)
    a, b = to_dev_u8(a8), to_dev_u8(b8)
    sa, sb = _f32(1.0), _f32(1.0)
    y1 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    y2 = torch.empty_like(y1)
    ws = torch.empty(splits * M * N, dtype=torch.float32, device=DEV)
    sq.fp8_gemm_scaled_splitk(a, 0, b, 0, splits, sa, sb, ws, y1)
    sq.fp8_gemm_scaled_splitk_noalloc(a, 0, b, 0, splits, sa, sb, y2)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    # 8 splits of a 4096 x 4096 output need 128 Mi floats: rejected before any launch
    big_a = torch.empty((4096, 1024), dtype=torch.uint8, device=DEV)
    big_b = torch.empty((4096, 1024), dtype=torch.uint8, device=DEV)
    big_y = torch.empty((4096, 4096), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(sq.Fp8dpError, match="scratch"):
        sq.fp8_gemm_scaled_splitk_noalloc(big_a, 0, big_b, 0, 8, sa, sb, big_y)
