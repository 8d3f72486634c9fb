"""The dgrad GEMM with the squared ReLU's backward in its epilogue (GPU).

fp8_gemm_relu2_backward must equal, bit for bit, fp8_gemm_scaled (E5M2 dY8 x
E4M3 W8^T -> dA BF16, same accumulation mode) followed by
relu2_backward_quantize on dA with the activation's FP8 cache -- gradient
codes, and the amax and saturation count folded into the gradient state.
Against the oracle: the GEMM half within the bound |dA - ref| <= 2^-8 |ref| +
1e-5 sum|ab| (every element in exact mode), and the fused gradient codes
equal, bit for bit, to the oracle's squared-ReLU backward of that dA -- so
they are the oracle's backward of a BF16 dA the GEMM bound admits (the GEMM's
result is one of several correct ones; the backward and the cast are then
exact).  Workloads: the GPT-2
down-projection's tensors at full size (the activation A = relu2(H0) cached
as E4M3 at the delayed scale, the log-normal gradient as E5M2, the weight as
E4M3) and seeded random codes on every tile width.
"""
import numpy as np
import pytest
import torch

import oracle as O
import scaled_quantization_amd as sq
import workloads
from gpu_util import (DEV, bf16_np, check_gemm, fp8_mfma_allowance,
                      oracle_gemm_rows, oracle_quantize, to_dev_u8, u8_np)

pytestmark = pytest.mark.gpu
EXACT, FP8 = sq.ACCUM_EXACT, sq.ACCUM_MFMA_FP8
BOTH = pytest.mark.parametrize("accum", [EXACT, FP8], ids=["exact", "fp8"])


def _f32(x):
    return torch.tensor([x], dtype=torch.float32, device=DEV)


def _fused_and_unfused(dy8, w8t, cache, cache_kind, s_dy, s_w, s_a, fmt, state_amax, accum):
    M, N = dy8.shape[0], w8t.shape[0]
    a, b, c = to_dev_u8(dy8), to_dev_u8(w8t), to_dev_u8(cache)
    sia = _f32(float(np.float32(1.0) / np.float32(s_dy)))
    sib = _f32(float(np.float32(1.0) / np.float32(s_w)))
    sic = _f32(float(np.float32(1.0) / np.float32(s_a)))
    st1 = sq.TensorState(fmt, 1, 1.25, state_amax)
    st2 = sq.TensorState(fmt, 1, 1.25, state_amax)
    dh_f = torch.empty((M, N), dtype=torch.uint8, device=DEV)
    sq.fp8_gemm_relu2_backward(a, sq.E5M2, b, sq.E4M3, sia, sib, c, cache_kind, sic, fmt, st1, dh_f,
                               accum)
    dA = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    sq.fp8_gemm_scaled(a, sq.E5M2, b, sq.E4M3, sq.PER_TENSOR, sia, sib, dA, accum)
    dh_u = torch.empty((M, N), dtype=torch.uint8, device=DEV)
    sq.relu2_backward_quantize(dA, c, cache_kind, sic, fmt, st2, dh_u)
    return dh_f, st1, dA, dh_u, st2


def _codes(rng, shape, fmt, lo=0.25, hi=16.0):
    t = O.fp8_decode_table(fmt)
    ok = np.flatnonzero(np.isfinite(t) & (np.abs(t) >= lo) & (np.abs(t) <= hi))
    return rng.choice(ok, size=shape).astype(np.uint8)


def _codes_vs_oracle(dA, dh, cache, cache_kind, s_a, fmt, state_amax, rows, what):
    """The fused gradient codes of the sampled rows equal, bit for bit, the
    oracle's squared-ReLU backward of dA -- the plain GEMM's output, which the
    caller has checked against the oracle's GEMM bound -- so they are the
    oracle's backward of a dA the bound admits."""
    scale = O.State(fmt, 1, 1.25, state_amax).scale
    r = O.relu2_backward(bf16_np(dA)[rows], np.asarray(cache)[rows], cache_kind,
                         float(np.float32(1.0) / np.float32(s_a)), fmt, scale)
    got = u8_np(dh)[rows]
    bad = got != r.fp8
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} codes differ from the "
                             f"oracle's backward, e.g. row {rows[i[0]]} col {i[1]}: "
                             f"{got[i]:#04x} vs {r.fp8[i]:#04x}")


@BOTH
@pytest.mark.parametrize("M,N,K", [(256, 384, 256), (512, 512, 384), (256, 640, 128),
                                   (768, 1024, 768)])
@pytest.mark.parametrize("cache_kind,fmt", [(0, 1), (1, 1), (0, 0)])
def test_fused_equals_composition_and_oracle(M, N, K, cache_kind, fmt, accum):
    rng = np.random.default_rng(M + N + K + 10 * cache_kind + fmt)
    dy8 = _codes(rng, (M, K), O.E5M2)
    w8t = _codes(rng, (N, K), O.E4M3)
    t = O.fp8_decode_table(cache_kind)
    ok = np.flatnonzero(np.isfinite(t) & (t >= 0))
    cache = rng.choice(ok, size=(M, N)).astype(np.uint8)
    s_dy, s_w, s_a = 0.5, 2.0, 3.0
    rows = np.unique(np.concatenate([np.arange(0, M, max(1, M // 16)), [M - 1]]))
    ref, absref = oracle_gemm_rows(dy8, O.E5M2, w8t, O.E4M3, O.PER_TENSOR, s_dy, s_w, rows)
    for state_amax in (1.0, 1e6):          # a scale that saturates, and one that does not
        dh_f, st1, dA, dh_u, st2 = _fused_and_unfused(dy8, w8t, cache, cache_kind, s_dy, s_w,
                                                        s_a, fmt, state_amax, accum)
        assert torch.equal(dh_f, dh_u)
        d1, d2 = st1.read(), st2.read()
        assert d1["amax_acc"] == d2["amax_acc"] and d1["sat_acc"] == d2["sat_acc"]
        # the backward half bit for bit on the GPU's dA
        st_o = O.State(fmt, 1, 1.25, state_amax)
        r = O.relu2_backward(bf16_np(dA), cache, cache_kind,
                             float(np.float32(1.0) / np.float32(s_a)), fmt, st_o.scale)
        assert np.array_equal(u8_np(dh_u), r.fp8)
    # the GEMM half against the oracle, then the fused codes against the
    # oracle's backward of the admissible dA values
    check_gemm(dA.float().cpu().numpy()[rows], ref, absref, "dgrad", accum == EXACT,
               lambda sel: fp8_mfma_allowance(dy8, O.E5M2, w8t, O.E4M3, O.PER_TENSOR, s_dy, s_w,
                                              rows[sel]))
    _codes_vs_oracle(dA, dh_f, cache, cache_kind, s_a, fmt, 1e6, rows, "fused")


@BOTH
def test_fused_gpt2_down_projection(accum):
    w = workloads.get("gpt2")
    h = w.h0()
    s_a = 11.0
    ra = oracle_quantize(h, O.ACT_RELU2, O.E4M3, O.PER_TENSOR, s_a, want_bf16=False)
    del h
    w8, s_w, _ = O.quantize_weight_tensor(w.weight(), O.E4M3)
    dy = w.dy()
    s_dy = O.scale_from_amax(float(np.abs((dy.astype(np.uint32) << 16).view(np.float32)).max()),
                             1.0, O.E5M2)[0][0]
    rd = oracle_quantize(dy, O.ACT_IDENTITY, O.E5M2, O.PER_TENSOR, s_dy, want_bf16=False)
    w8t = np.ascontiguousarray(w8.T)                       # [3072 x 768]
    M = rd.fp8.shape[0]
    rng = np.random.default_rng(43)
    rows = np.sort(rng.choice(M, size=256, replace=False))
    rows[0], rows[-1] = 0, M - 1
    ref, absref = oracle_gemm_rows(rd.fp8, O.E5M2, w8t, O.E4M3, O.PER_TENSOR, s_dy, s_w, rows)
    for state_amax in (1.0, 2.0e4):
        dh_f, st1, dA, dh_u, st2 = _fused_and_unfused(rd.fp8, w8t, ra.fp8, O.E4M3, s_dy, s_w,
                                                        s_a, O.E5M2, state_amax, accum)
        assert torch.equal(dh_f, dh_u)
        d1, d2 = st1.read(), st2.read()
        assert d1["amax_acc"] == d2["amax_acc"] and d1["sat_acc"] == d2["sat_acc"]
        if state_amax == 1.0:
            check_gemm(dA.float().cpu().numpy()[rows], ref, absref, "gpt2 dgrad", accum == EXACT,
                       lambda sel: fp8_mfma_allowance(rd.fp8, O.E5M2, w8t, O.E4M3, O.PER_TENSOR,
                                                      s_dy, s_w, rows[sel]))
        _codes_vs_oracle(dA, dh_f, ra.fp8, O.E4M3, s_a, O.E5M2, state_amax, rows,
                         f"gpt2 fused, state amax {state_amax}")


def test_fused_rejects_other_formats():
    z = torch.zeros((256, 128), dtype=torch.uint8, device=DEV)
    one = _f32(1.0)
    st = sq.TensorState(sq.E5M2, 1, 1.25, 1.0)
    out = torch.empty((256, 128), dtype=torch.uint8, device=DEV)
    b = torch.zeros((128, 128), dtype=torch.uint8, device=DEV)
    rc = sq.lib().fp8_gemm_relu2_backward(z.data_ptr(), 0, b.data_ptr(), 0, 256, 128, 128,
                                          sq.ACCUM_EXACT, one.data_ptr(), one.data_ptr(),
                                          out.data_ptr(), 0,
                                          one.data_ptr(), 1, st.ptr, out.data_ptr(), None)
    assert rc == -2
