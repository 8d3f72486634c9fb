"""The fused quantizer with a transposed copy of its codes (GPU).

"FP8 Training & Inference", FP8 Training Recipe: the weight gradient
dW = dY^T X reads both cast tensors transposed.  quantize_fused_transposed
writes the codes a second time as [cols x rows]; everything else is
quantize_fused's.  Parity: the BF16 copy and codes bit for bit against the
oracle's quantization (and against quantize_fused on the same input), the
transposed codes against numpy's transpose of the oracle's codes, the state
after amax_history_update field by field against quantize_fused's; the
weight-gradient GEMM on the transposed outputs bit for bit equal to the same
GEMM on fp8_transpose's outputs.  Workloads: small tiles over every
format / activation pair and both codecs, the GPT-2 activation and gradient
at full size.
"""
import numpy as np
import pytest
import torch

import oracle as O
import scaled_quantization_amd as sq
import workloads
from gpu_util import DEV, bf16_np, oracle_quantize, to_dev_bf16, u8_np

pytestmark = pytest.mark.gpu


@pytest.fixture(params=[0, 1], ids=["hw", "int"])
def codec(request):
    prev = sq.fp8dp_set_codec(request.param)
    yield request.param
    sq.fp8dp_set_codec(prev)


def _h(rng, rows, cols, spread=4.0):
    x = (rng.standard_normal((rows, cols)) * spread).astype(np.float32)
    x[rng.random((rows, cols)) < 0.01] *= 300.0       # a few values that saturate
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _run(h_np, act, fmt, amax0, outputs=(True, True)):
    rows, cols = h_np.shape
    h = to_dev_bf16(h_np)
    st = sq.TensorState(fmt, 1, 1.25, amax0, device=DEV)
    b16 = torch.empty_like(h) if outputs[0] else None
    q8 = torch.empty((rows, cols), dtype=torch.uint8, device=DEV) if outputs[1] else None
    qt = torch.empty((cols, rows), dtype=torch.uint8, device=DEV)
    sq.quantize_fused_transposed(h, act, fmt, st, qt, b16, q8)
    sq.amax_history_update(st)
    return b16, q8, qt, st


def _state_matches(st, s, r):
    """st (after amax_history_update) against oracle state s stepped with result r."""
    s.accumulate(r.amax_bits, r.sat)
    s.update()
    d = st.read()
    assert d["scale"] == s.scale and d["scale_inv"] == s.scale_inv
    assert d["sat_last"] == s.sat_last and d["overflow"] == s.overflow
    assert d["amax_last"] == s.history[0]


@pytest.mark.parametrize("rows,cols", [(64, 128), (128, 384), (320, 256)])
@pytest.mark.parametrize("act,fmt", [(1, 0), (0, 0), (0, 1), (1, 1)])
def test_transposed_codes_vs_oracle(codec, rows, cols, act, fmt):
    rng = np.random.default_rng(rows + cols + 10 * act + fmt)
    h_np = _h(rng, rows, cols)
    amax0 = 40.0 if act == 0 else 1000.0
    b16, q8, qt, st = _run(h_np, act, fmt, amax0)
    s = O.State(fmt, 1, 1.25, amax0)
    r = O.quantize(h_np, act, fmt, O.PER_TENSOR, s.scale)
    assert np.array_equal(bf16_np(b16), r.bf16)
    assert np.array_equal(u8_np(q8), r.fp8)
    assert np.array_equal(u8_np(qt), r.fp8.T)
    _state_matches(st, s, r)
    assert r.sat > 0 or fmt == 1


def test_optional_outputs_and_equality_with_quantize_fused():
    rng = np.random.default_rng(3)
    h_np = _h(rng, 256, 512)
    _, _, qt_only, st1 = _run(h_np, 1, 0, 500.0, outputs=(False, False))
    h = to_dev_bf16(h_np)
    st2 = sq.TensorState(sq.E4M3, 1, 1.25, 500.0, device=DEV)
    q8 = torch.empty((256, 512), dtype=torch.uint8, device=DEV)
    sq.quantize_fused(h, sq.ACT_RELU2, sq.E4M3, sq.PER_TENSOR, st2, None, q8)
    sq.amax_history_update(st2)
    assert torch.equal(qt_only, q8.t().contiguous())
    assert st1.read() == st2.read()


@pytest.mark.parametrize("which", ["activation", "gradient"])
def test_gpt2_full_size(which):
    w = workloads.get("gpt2")
    if which == "activation":
        h_np, act, fmt, amax0 = w.h0(), O.ACT_RELU2, O.E4M3, 11.0
    else:
        h_np, act, fmt, amax0 = w.dy(), O.ACT_IDENTITY, O.E5M2, 1.0
    b16, q8, qt, st = _run(h_np, act, fmt, amax0)
    scale = O.State(fmt, 1, 1.25, amax0).scale
    r = oracle_quantize(h_np, act, fmt, O.PER_TENSOR, scale, want_bf16=(act == O.ACT_RELU2))
    del h_np
    got = u8_np(q8)
    assert np.array_equal(got, r.fp8)
    if act == O.ACT_RELU2:
        assert np.array_equal(bf16_np(b16), r.bf16)
    assert np.array_equal(u8_np(qt), np.ascontiguousarray(r.fp8.T))
    _state_matches(st, O.State(fmt, 1, 1.25, amax0), r)


def test_wgrad_on_transposed_outputs_equals_wgrad_on_transposes():
    rng = np.random.default_rng(11)
    M, K, N = 2048, 768, 256                 # tokens, activation width, gradient width
    a_np = _h(rng, M, K, 1.0)
    g_np = _h(rng, M, N, 0.01)
    _, a8, a8t, st_a = _run(a_np, 1, 0, 20.0)
    _, g8, g8t, st_g = _run(g_np, 0, 1, 0.1)
    at = torch.empty((K, M), dtype=torch.uint8, device=DEV)
    gt = torch.empty((N, M), dtype=torch.uint8, device=DEV)
    sq.fp8_transpose(a8, at)
    sq.fp8_transpose(g8, gt)
    assert torch.equal(at, a8t) and torch.equal(gt, g8t)
    ws = torch.empty(4 * N * K, dtype=torch.float32, device=DEV)
    y1 = torch.empty((N, K), dtype=torch.bfloat16, device=DEV)
    y2 = torch.empty_like(y1)
    sa, sb = st_g.field_ptr("scale_inv_used"), st_a.field_ptr("scale_inv_used")
    sq.fp8_gemm_scaled_splitk(g8t, sq.E5M2, a8t, sq.E4M3, 4, sa, sb, ws, y1)
    sq.fp8_gemm_scaled_splitk(gt, sq.E5M2, at, sq.E4M3, 4, sa, sb, ws, y2)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_transposed_argument_errors():
    h = torch.zeros((96, 128), dtype=torch.bfloat16, device=DEV)
    st = sq.TensorState(sq.E4M3, device=DEV)
    qt = torch.empty((128, 96), dtype=torch.uint8, device=DEV)
    with pytest.raises(sq.Fp8dpError, match="multiple of 64"):
        sq.quantize_fused_transposed(h, sq.ACT_RELU2, sq.E4M3, st, qt)
    h = torch.zeros((64, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(sq.Fp8dpError, match="cols x rows"):
        sq.quantize_fused_transposed(h, sq.ACT_RELU2, sq.E4M3, st, qt)
