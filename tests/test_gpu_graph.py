"""The benchmark step captured in a HIP graph (GPU).

Every entry point enqueues kernels on the caller's stream, never allocates
and never synchronizes, so a whole step -- quantize_fused on H, the FP8 GEMM,
amax_history_update, the E5M2 cast of dY, its update, and the overflow
recompute of both casts; or the benchmark's form with each cast closing its
own step (quantize_fused_update) -- can be captured once and replayed.  Each replay
is one more step of delayed scaling: the test replays the graph several
times, with eager work and host synchronizations in between, and checks
every replay bit for bit against the same steps run eagerly on a second set
of buffers and states (codes, BF16 copies, GEMM output, both states).
"""
import numpy as np
import pytest
import torch

import scaled_quantization_amd as sq
import workloads
from gpu_util import DEV, to_dev_bf16

pytestmark = pytest.mark.gpu


def _step(bufs, fused=False, recompute=True):
    """fused: the benchmark's step -- each cast closes its step itself
    (quantize_fused_update) and the GEMM reads the used scale's inverse."""
    h, a16, a8, w8, wsc, y, dy, dy8, st_a, st_g = bufs
    if fused:
        sq.quantize_fused_update(h, sq.ACT_RELU2, sq.E4M3, st_a, a16, a8)
        sq.fp8_gemm_scaled(a8, sq.E4M3, w8, sq.E4M3, sq.PER_TENSOR,
                           st_a.field_ptr("scale_inv_used"), wsc, y)
    else:
        sq.quantize_fused(h, sq.ACT_RELU2, sq.E4M3, sq.PER_TENSOR, st_a, a16, a8)
        sq.fp8_gemm_scaled(a8, sq.E4M3, w8, sq.E4M3, sq.PER_TENSOR, st_a.field_ptr("scale_inv"),
                           wsc, y)
        sq.amax_history_update(st_a)
    if recompute:
        sq.quantize_recompute(h, sq.ACT_RELU2, sq.E4M3, st_a, a8)
        sq.fp8_gemm_scaled_if(a8, sq.E4M3, w8, sq.E4M3, st_a.field_ptr("scale_inv"), wsc, y,
                              st_a.field_ptr("overflow"))
    if fused:
        sq.quantize_fused_update(dy, sq.ACT_IDENTITY, sq.E5M2, st_g, None, dy8)
    else:
        sq.quantize_fused(dy, sq.ACT_IDENTITY, sq.E5M2, sq.PER_TENSOR, st_g, None, dy8)
        sq.amax_history_update(st_g)
    if recompute:
        sq.quantize_recompute(dy, sq.ACT_IDENTITY, sq.E5M2, st_g, dy8)


def _buffers(w, h, dy, wt):
    M, K, N = w.M, w.K, w.N
    w8 = torch.empty((N, K), dtype=torch.uint8, device=DEV)
    wsc = torch.empty(2, dtype=torch.float32, device=DEV)
    sq.quantize_weight(wt, sq.E4M3, sq.PER_TENSOR, w8, wsc)
    return [h, torch.empty((M, K), dtype=torch.bfloat16, device=DEV),
            torch.empty((M, K), dtype=torch.uint8, device=DEV), w8, wsc,
            torch.empty((M, N), dtype=torch.bfloat16, device=DEV), dy,
            torch.empty((M, N), dtype=torch.uint8, device=DEV),
            sq.TensorState(sq.E4M3, 1, w.margin, w.initial_amax),
            sq.TensorState(sq.E5M2, 1, w.margin, w.initial_amax)]


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused_update"])
@pytest.mark.parametrize("name", ["tiny", "gpt2"])
def test_step_graph_replays_equal_eager_steps(name, fused):
    w = workloads.get(name)
    h = to_dev_bf16(w.h0())
    dy = to_dev_bf16(w.dy())
    wt = to_dev_bf16(w.weight())
    g_bufs = _buffers(w, h, dy, wt)
    e_bufs = _buffers(w, h, dy, wt)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up outside the capture (library load)
        _step(g_bufs, fused)
    torch.cuda.current_stream().wait_stream(side)
    _step(e_bufs, fused)                   # the eager twin runs the same warm-up step
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _step(g_bufs, fused)
    # capture enqueues nothing: the captured step has not run yet
    torch.cuda.synchronize()
    for rep in range(4):
        graph.replay()
        _step(e_bufs, fused)
        torch.cuda.synchronize()
        for k in (1, 2, 5, 7):             # a16, a8, y, dy8
            assert torch.equal(g_bufs[k].view(torch.uint8), e_bufs[k].view(torch.uint8)), (rep, k)
        for k in (8, 9):                   # every field of both states (not the padding)
            assert g_bufs[k].read() == e_bufs[k].read(), (rep, k)
        # eager work between replays
        torch.cuda.synchronize()
    assert g_bufs[8].read()["steps"] == 5


def test_calls_enqueue_on_the_current_stream():
    """The binding passes the current stream's raw handle: the default stream,
    a stream made current by torch.cuda.stream, and the capture stream."""
    assert sq._stream(None) == torch.cuda.current_stream().cuda_stream
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        assert sq._stream(None) == s.cuda_stream != torch.cuda.default_stream().cuda_stream
    assert sq._stream(None) == torch.cuda.default_stream().cuda_stream
    src = torch.arange(64 * 128, device=DEV).to(torch.uint8).view(64, 128)
    dst = torch.zeros((128, 64), dtype=torch.uint8, device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sq.fp8_transpose(src, dst)
    torch.cuda.synchronize()
    assert not dst.any()                     # captured, not run
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(dst, src.t().contiguous())


def test_step_on_a_side_stream_equals_default_stream():
    """The step's calls issued inside torch.cuda.stream(s) give the same codes,
    BF16 copy, GEMM output and state as on the default stream."""
    rng = np.random.default_rng(5)
    M, K, N = 512, 1024, 256
    h = to_dev_bf16((rng.standard_normal((M, K)) * 3).astype(np.float32)
                    .view(np.uint32).__rshift__(16).astype(np.uint16))
    wt = to_dev_bf16((rng.standard_normal((N, K)) * 0.02).astype(np.float32)
                     .view(np.uint32).__rshift__(16).astype(np.uint16))

    def run():
        w8 = torch.empty((N, K), dtype=torch.uint8, device=DEV)
        wsc = torch.empty(2, dtype=torch.float32, device=DEV)
        sq.quantize_weight(wt, sq.E4M3, sq.PER_TENSOR, w8, wsc)
        st = sq.TensorState(sq.E4M3, 4, 1.25, 10.0)
        a16 = torch.empty_like(h)
        a8 = torch.empty((M, K), dtype=torch.uint8, device=DEV)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        for _ in range(3):
            sq.quantize_fused(h, sq.ACT_RELU2, sq.E4M3, sq.PER_TENSOR, st, a16, a8)
            sq.fp8_gemm_scaled(a8, sq.E4M3, w8, sq.E4M3, sq.PER_TENSOR,
                               st.field_ptr("scale_inv"), wsc, y)
            sq.amax_history_update(st)
        return a16, a8, y, st

    r0 = run()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        r1 = run()
    s.synchronize()
    for a, b in zip(r0[:3], r1[:3]):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    assert r0[3].read() == r1[3].read()
