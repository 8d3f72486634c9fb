"""Overflow-triggered recompute under delayed scaling (GPU).

"FP8 Training & Inference", Delayed Scaling: the scale comes from the
previous iterations' amax; when it turns out too large for the current
tensor the overflow is detected and the step recomputed with a corrected
scale.  Here a step is: quantize_fused with the delayed scale, the GEMM,
amax_history_update (which flags a saturating step), then quantize_recompute
and fp8_gemm_scaled_if, which act only when the flag is set -- decided on the
GPU.  Oracle: the same composition of oracle.quantize, oracle.State and
oracle.gemm_f64: when the step saturated, the codes are the oracle's cast
with the updated scale (bit for bit) and the GEMM uses that scale; when it
did not, the codes and the GEMM output are left exactly as they were.
"""
import numpy as np
import pytest
import torch

import oracle as O
import scaled_quantization_amd as sq
import workloads
from gpu_util import DEV, bf16_np, check_gemm, to_dev_bf16, to_dev_u8, u8_np

pytestmark = pytest.mark.gpu


# step multipliers of the tiny workload's H0: 1.0 overflows the initial scale
# (initial amax 1 vs relu2 amax ~20), 1.1 stays inside the 1.25 margin, 4.0
# jumps past it, then the tensor shrinks
FACTORS = [1.0, 1.1, 4.0, 1.0, 0.5]


@pytest.mark.parametrize("fmt", [0, 1], ids=["e4m3", "e5m2"])
def test_recompute_sequence_tiny(fmt):
    w = workloads.get("tiny")
    h0 = w.h0()
    wq, s_w, si_w = O.quantize_weight_tensor(w.weight(), O.E4M3)
    w8 = to_dev_u8(wq)
    wsi = torch.tensor([si_w], dtype=torch.float32, device=DEV)
    st = sq.TensorState(fmt, 1, w.margin, w.initial_amax)
    ost = O.State(fmt, 1, w.margin, w.initial_amax)
    M, K, N = w.M, w.K, w.N
    a16 = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    a8 = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    flagged = []
    for t, f in enumerate(FACTORS):
        h = h0.copy() if f == 1.0 else workloads.scale_bf16(h0, f)
        hd = to_dev_bf16(h)
        sq.quantize_fused(hd, sq.ACT_RELU2, fmt, sq.PER_TENSOR, st, a16, a8)
        sq.fp8_gemm_scaled(a8, fmt, w8, sq.E4M3, sq.PER_TENSOR, st.field_ptr("scale_inv"), wsi, y)
        sq.amax_history_update(st)
        a8_first, y_first = u8_np(a8).copy(), bf16_np(y).copy()
        sq.quantize_recompute(hd, sq.ACT_RELU2, fmt, st, a8)
        sq.fp8_gemm_scaled_if(a8, fmt, w8, sq.E4M3, st.field_ptr("scale_inv"), wsi, y,
                              st.field_ptr("overflow"))
        d = st.read()

        r = O.quantize(h, O.ACT_RELU2, fmt, O.PER_TENSOR, ost.scale)
        s_used = ost.scale
        ost.accumulate(r.amax_bits, r.sat)
        ost.update()
        assert d["overflow"] == (1 if r.sat > 0 else 0) == ost.overflow, t
        assert d["scale"] == ost.scale, t
        assert np.array_equal(bf16_np(a16), r.bf16), t
        assert np.array_equal(a8_first, r.fp8), t
        if r.sat > 0:
            flagged.append(t)
            r2 = O.quantize(h, O.ACT_RELU2, fmt, O.PER_TENSOR, ost.scale, want_bf16=False)
            assert r2.sat == 0, t            # the corrected scale fits the step's amax
            q, s_used = r2.fp8, ost.scale
        else:
            q = r.fp8
            assert np.array_equal(bf16_np(y), y_first), t     # untouched
        assert np.array_equal(u8_np(a8), q), t
        ref, absref = O.gemm_f64(q, fmt, wq, O.E4M3, O.PER_TENSOR, s_used, s_w)
        # the GEMMs run in exact mode (the binding's default): every element
        check_gemm(y.float().cpu().numpy(), ref, absref, f"step {t}")
    assert flagged == [0, 2]


@pytest.mark.parametrize("n", [1003, 8, 4096 + 5])
def test_recompute_ragged_gradient_cast(n):
    """Identity / E5M2 (the gradient cast) over ragged lengths: the tail
    elements are recast too."""
    rng = np.random.default_rng(n)
    x = (rng.standard_normal(n) * 1000.0).astype(np.float32)
    h = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    hd = to_dev_bf16(h.reshape(1, -1))
    q = torch.empty((1, n), dtype=torch.uint8, device=DEV)
    st = sq.TensorState(sq.E5M2, 1, 1.0, 1.0)          # scale 57344: everything saturates
    ost = O.State(O.E5M2, 1, 1.0, 1.0)
    sq.quantize_fused(hd, sq.ACT_IDENTITY, sq.E5M2, sq.PER_TENSOR, st, None, q)
    sq.amax_history_update(st)
    sq.quantize_recompute(hd, sq.ACT_IDENTITY, sq.E5M2, st, q)
    r = O.quantize(h, O.ACT_IDENTITY, O.E5M2, O.PER_TENSOR, ost.scale, want_bf16=False)
    ost.accumulate(r.amax_bits, r.sat)
    ost.update()
    assert r.sat > 0 and st.read()["overflow"] == 1
    r2 = O.quantize(h, O.ACT_IDENTITY, O.E5M2, O.PER_TENSOR, ost.scale, want_bf16=False)
    assert np.array_equal(u8_np(q).reshape(-1), r2.fp8.reshape(-1))


def test_recompute_is_a_no_op_without_overflow():
    rng = np.random.default_rng(2)
    h = torch.from_numpy(rng.standard_normal((256, 512)).astype(np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    hd = to_dev_bf16(h)
    st = sq.TensorState(sq.E4M3, 1, 1.25, 100.0)       # generous: nothing saturates
    q = torch.empty((256, 512), dtype=torch.uint8, device=DEV)
    sq.quantize_fused(hd, sq.ACT_RELU2, sq.E4M3, sq.PER_TENSOR, st, None, q)
    sq.amax_history_update(st)
    assert st.read()["overflow"] == 0
    sentinel = torch.full_like(q, 0x5A)
    sq.quantize_recompute(hd, sq.ACT_RELU2, sq.E4M3, st, sentinel)
    y = torch.full((256, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    w8 = torch.zeros((128, 512), dtype=torch.uint8, device=DEV)
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    sq.fp8_gemm_scaled_if(q, 0, w8, 0, one, one, y, st.field_ptr("overflow"))
    torch.cuda.synchronize()
    assert (sentinel == 0x5A).all() and (y == 7.0).all()


@pytest.mark.parametrize("M", [100, 256 + 77])
def test_conditional_gemm_ragged_rows(M):
    # any row count, as fp8_gemm_scaled: with the flag clear the output stays
    # untouched; with it set the output is fp8_gemm_scaled's, bit for bit
    # (the same split of rows over the same kernels)
    rng = np.random.default_rng(M)
    K, N = 512, 384
    codes = np.flatnonzero(np.isfinite(O.fp8_decode_table(O.E4M3))).astype(np.uint8)
    a = torch.from_numpy(rng.choice(codes, (M, K))).to(DEV)
    w = torch.from_numpy(rng.choice(codes, (N, K))).to(DEV)
    sa = torch.tensor([0.5], dtype=torch.float32, device=DEV)
    sb = torch.tensor([0.25], dtype=torch.float32, device=DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=DEV)
    sq.fp8_gemm_scaled_if(a, 0, w, 0, sa, sb, y, flag)
    torch.cuda.synchronize()
    assert (y == 7.0).all()
    flag.fill_(1)
    sq.fp8_gemm_scaled_if(a, 0, w, 0, sa, sb, y, flag)
    ref = torch.empty_like(y)
    sq.fp8_gemm_scaled(a, 0, w, 0, sq.PER_TENSOR, sa, sb, ref)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16))
