"""The up-projection BF16 GEMM with the quantizer in its epilogue (GPU).

"Paradigma Details FP8 and Optimizer Tricks Behind NanoGPT Records", FP8
paragraph: the fused kernel works on the preceding computation's results
while they are still in registers.  The entry point computes
H = bf16_rne(X W^T) with FP32 accumulation and applies quantize_fused to H
in the same kernel.

Parity against the oracle:
* H: the oracle's float64 GEMM gives ref and sum |x w|; the GPU's H must be a
  BF16 rounding of an FP32 value within e = 2^-20 sum|x w| of ref (FP32
  accumulation of exact products), which also meets the GEMM bound
  |H - ref| <= 2^-8 |ref| + 1e-5 sum|x w|.
* BF16 copy, FP8 code: for each element the oracle enumerates every BF16
  value H may take (bf16(fp32(ref - e)) .. bf16(fp32(ref + e)), usually one
  or two) and quantizes each with its own arithmetic; the GPU's triple
  (H, copy, code) must be one of those.  Elements with more than 64
  candidates (|ref| within ~2^-17 sum|x w| of zero) are checked on H only,
  and their share is asserted to be tiny.
* amax and saturation count: within the range the candidates allow, and the
  amax equal to the largest |copy| the GPU wrote.
At full GPT-2 size the fused call is also compared bit for bit with the
plain GEMM followed by quantize_fused on its H, both through the C ABI.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle as O
import scaled_quantization_amd as sq
import workloads
from gpu_util import DEV, THREADS, bf16_np, to_dev_bf16, u8_np

pytestmark = pytest.mark.gpu
E_REL = 2.0 ** -20
CAP = 64


def oracle_gemm_bf16_rows(x, w, rows):
    rows = np.asarray(rows, dtype=np.int64)
    chunks = np.array_split(rows, min(THREADS, len(rows)))
    with ThreadPoolExecutor(THREADS) as ex:
        parts = list(ex.map(lambda rr: O.gemm_bf16_f64(x, w, rows=rr), chunks))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def _key(bits):
    b = bits.astype(np.int64)
    return np.where(b < 0x8000, b, -(b & 0x7FFF))


def _bits(key):
    return np.where(key >= 0, key, 0x8000 | (-key)).astype(np.uint16)


def _bf16_value(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def candidate_ranges(ref, absref):
    """Key range [lo, hi] of the BF16 values H may take, per element."""
    e = E_REL * absref + 1e-30
    lo = O.bf16_rne((ref - e).astype(np.float32))
    hi = O.bf16_rne((ref + e).astype(np.float32))
    return _key(lo), _key(hi)


def check_fused(h_gpu, b_gpu, q_gpu, ref, absref, act, fmt, scale, what):
    """Element-wise candidate check; returns (amax_lo, amax_hi, sat_lo, sat_hi)
    over the checked elements from the oracle's candidates."""
    ref = ref.ravel()
    absref = absref.ravel()
    h_gpu = h_gpu.ravel()
    klo, khi = candidate_ranges(ref, absref)
    kg = _key(h_gpu)
    inside = (kg >= klo) & (kg <= khi)
    assert inside.all(), f"{what}: {int((~inside).sum())} H values outside the FP32 bound"
    hv = _bf16_value(h_gpu)
    bound = (2.0 ** -8) * np.abs(ref) + 1e-5 * absref
    assert np.all(np.abs(hv - ref) <= bound), f"{what}: H outside the GEMM bound"
    n = khi - klo + 1
    wide = n > CAP
    assert wide.mean() <= 1e-3, f"{what}: {wide.mean():.2e} of elements near zero"
    idx = np.flatnonzero(~wide)
    counts = n[idx]
    offs = np.concatenate([[0], np.cumsum(counts)])
    cand_keys = np.repeat(klo[idx], counts) + (np.arange(offs[-1]) - np.repeat(offs[:-1], counts))
    cand = _bits(cand_keys)
    r = O.quantize(cand.reshape(1, -1), act, fmt, O.PER_TENSOR, scale)
    cb, cq = r.bf16.ravel(), r.fp8.ravel()
    csat = O.fp8_saturates(_bf16_value(cb).astype(np.float32) * np.float32(scale), fmt)
    pos = offs[:-1] + (kg[idx] - klo[idx])
    bad_b = cb[pos] != b_gpu.ravel()[idx]
    bad_q = cq[pos] != q_gpu.ravel()[idx]
    if bad_b.any() or bad_q.any():
        j = np.flatnonzero(bad_b | bad_q)[:5]
        raise AssertionError(f"{what}: {int(bad_b.sum())} copies, {int(bad_q.sum())} codes differ; "
                             f"e.g. H={h_gpu[idx][j]} copy={b_gpu.ravel()[idx][j]} vs {cb[pos][j]} "
                             f"code={q_gpu.ravel()[idx][j]} vs {cq[pos][j]}")
    mag = (cb & 0x7FFF).astype(np.int64)
    seg_min = np.minimum.reduceat(mag, offs[:-1])
    seg_max = np.maximum.reduceat(mag, offs[:-1])
    sat_min = np.minimum.reduceat(csat.astype(np.int64), offs[:-1])
    sat_max = np.maximum.reduceat(csat.astype(np.int64), offs[:-1])
    return int(seg_min.max()), int(seg_max.max()), int(sat_min.sum()), int(sat_max.sum()), wide.sum()


def _state(fmt, initial_amax=1.0):
    return sq.TensorState(fmt, 1, 1.25, initial_amax, device=DEV)


def _run_fused(x, w, act, fmt, st, with_h=True, with_b=True):
    M, N = x.shape[0], w.shape[0]
    h = torch.empty((M, N), dtype=torch.bfloat16, device=DEV) if with_h else None
    b = torch.empty((M, N), dtype=torch.bfloat16, device=DEV) if with_b else None
    q = torch.empty((M, N), dtype=torch.uint8, device=DEV)
    sq.gemm_bf16_quantize_fused(x, w, act, fmt, st, h, b, q)
    return h, b, q


def _random_bf16(rng, shape, std):
    return workloads.bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


# ------------------------------------------------------------------ plain GEMM
@pytest.mark.parametrize("M,N,K", [(256, 128, 64), (512, 384, 192), (768, 640, 320),
                                   (256, 256, 128), (1024, 768, 768)])
def test_plain_bf16_gemm_vs_oracle(M, N, K):
    rng = np.random.default_rng(M + 3 * N + 7 * K)
    x = _random_bf16(rng, (M, K), 1.0)
    w = _random_bf16(rng, (N, K), K ** -0.5)
    h = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    sq.gemm_bf16_quantize_fused(to_dev_bf16(x), to_dev_bf16(w), h_out=h)
    hv = bf16_np(h)
    rows = np.unique(np.concatenate([np.arange(0, M, max(1, M // 96)), [M - 1]]))
    ref, absref = oracle_gemm_bf16_rows(x, w, rows)
    klo, khi = candidate_ranges(ref.ravel(), absref.ravel())
    kg = _key(hv[rows].ravel())
    assert np.all((kg >= klo) & (kg <= khi))


# ------------------------------------------------------------------ fused, tiny in full
@pytest.mark.parametrize("act,fmt", [(O.ACT_RELU2, O.E4M3), (O.ACT_IDENTITY, O.E5M2),
                                     (O.ACT_RELU2, O.E5M2), (O.ACT_IDENTITY, O.E4M3)])
def test_fused_tiny_every_element(act, fmt):
    w_ = workloads.get("tiny")
    x, w1 = w_.up_x(), w_.up_weight()
    st = _state(fmt)
    ost = O.State(fmt, 1, 1.25, 1.0)
    ref, absref = O.gemm_bf16_f64(x, w1)
    xd, wd = to_dev_bf16(x), to_dev_bf16(w1)
    for step in range(2):   # step 0 saturates (initial amax 1.0); step 1 uses the updated scale
        scale = ost.scale
        h, b, q = _run_fused(xd, wd, act, fmt, st)
        torch.cuda.synchronize()
        hv, bv, qv = bf16_np(h), bf16_np(b), u8_np(q)
        alo, ahi, slo, shi, nwide = check_fused(hv, bv, qv, ref, absref, act, fmt, scale,
                                                f"tiny step {step}")
        stv = st.read()
        amax_bits = stv["amax_acc"]
        assert amax_bits == int(np.max(bv & 0x7FFF)) << 16
        if nwide == 0:
            assert (alo << 16) <= amax_bits <= (ahi << 16)
            assert slo <= stv["sat_acc"] <= shi
        if step == 0:
            assert stv["sat_acc"] > 0
        sq.amax_history_update(st)
        # the oracle's state advances on the oracle's own amax and count (any
        # candidate choice that the checks above accepted gives the same scale
        # when the candidates' amax agree)
        r = O.quantize(O.bf16_rne(ref.astype(np.float32)), act, fmt, O.PER_TENSOR, scale)
        ost.accumulate(r.amax_bits, r.sat)
        ost.update()
        if alo == ahi:
            assert st.read()["scale"] == np.float32(ost.scale)


# ------------------------------------------------------------------ fused, GPT-2 size
def test_fused_gpt2_sampled_rows_and_equals_gemm_then_quantize():
    w_ = workloads.get("gpt2")
    x, w1 = w_.up_x(), w_.up_weight()
    xd, wd = to_dev_bf16(x), to_dev_bf16(w1)
    M, N = x.shape[0], w1.shape[0]
    st = _state(O.E4M3)
    # a realistic delayed scale: one step on the plain GEMM's output first
    h0 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    sq.gemm_bf16_quantize_fused(xd, wd, h_out=h0)
    sq.quantize_fused(h0, sq.ACT_RELU2, sq.E4M3, sq.PER_TENSOR, st, None, None)
    sq.amax_history_update(st)
    scale = st.read()["scale"]
    st2 = _state(O.E4M3)
    st2.buf.copy_(st.buf)
    h, b, q = _run_fused(xd, wd, O.ACT_RELU2, O.E4M3, st)
    # the same through the plain GEMM and the element-wise quantizer
    b2 = torch.empty_like(b)
    q2 = torch.empty_like(q)
    sq.quantize_fused(h0, sq.ACT_RELU2, sq.E4M3, sq.PER_TENSOR, st2, b2, q2)
    torch.cuda.synchronize()
    assert torch.equal(h.view(torch.int16), h0.view(torch.int16))
    assert torch.equal(b.view(torch.int16), b2.view(torch.int16))
    assert torch.equal(q, q2)
    s1, s2 = st.read(), st2.read()
    assert s1["amax_acc"] == s2["amax_acc"] and s1["sat_acc"] == s2["sat_acc"]
    # oracle parity on sampled rows
    rng = np.random.default_rng(31)
    rows = np.sort(rng.choice(M, size=48, replace=False))
    rows[0], rows[-1] = 0, M - 1
    ref, absref = oracle_gemm_bf16_rows(x, w1, rows)
    hv, bv, qv = bf16_np(h), bf16_np(b), u8_np(q)
    check_fused(hv[rows], bv[rows], qv[rows], ref, absref, O.ACT_RELU2, O.E4M3, scale, "gpt2")


# ------------------------------------------------------------------ shapes, optional outputs
@pytest.mark.parametrize("M,N,K,act,fmt", [(256, 128, 64, O.ACT_RELU2, O.E4M3),
                                           (512, 384, 192, O.ACT_IDENTITY, O.E5M2),
                                           (768, 640, 320, O.ACT_RELU2, O.E4M3),
                                           (256, 512, 128, O.ACT_RELU2, O.E5M2),
                                           (2304, 1152, 256, O.ACT_IDENTITY, O.E4M3)])
def test_fused_shapes_and_optional_outputs(M, N, K, act, fmt):
    rng = np.random.default_rng(5 * M + N + K)
    x = _random_bf16(rng, (M, K), 1.0)
    w = _random_bf16(rng, (N, K), K ** -0.5)
    xd, wd = to_dev_bf16(x), to_dev_bf16(w)
    st_a = _state(fmt, initial_amax=8.0)
    st_b = _state(fmt, initial_amax=8.0)
    h, b, q = _run_fused(xd, wd, act, fmt, st_a)
    # without H and without the BF16 copy: the same codes, amax and count
    _, _, q2 = _run_fused(xd, wd, act, fmt, st_b, with_h=False, with_b=False)
    torch.cuda.synchronize()
    assert torch.equal(q, q2)
    sa, sb_ = st_a.read(), st_b.read()
    assert sa["amax_acc"] == sb_["amax_acc"] and sa["sat_acc"] == sb_["sat_acc"]
    scale = sa["scale"]
    rows = np.unique(np.concatenate([np.arange(0, M, max(1, M // 64)), [M - 1]]))
    ref, absref = oracle_gemm_bf16_rows(x, w, rows)
    check_fused(bf16_np(h)[rows], bf16_np(b)[rows], u8_np(q)[rows], ref, absref, act, fmt,
                scale, f"{M}x{N}x{K}")


def test_fused_accumulates_across_calls():
    rng = np.random.default_rng(77)
    x1 = _random_bf16(rng, (256, 128), 1.0)
    x2 = _random_bf16(rng, (256, 128), 3.0)
    w = _random_bf16(rng, (256, 128), 128 ** -0.5)
    st = _state(O.E4M3)
    wd = to_dev_bf16(w)
    _, b1, _ = _run_fused(to_dev_bf16(x1), wd, O.ACT_RELU2, O.E4M3, st)
    a1 = st.read()
    _, b2, _ = _run_fused(to_dev_bf16(x2), wd, O.ACT_RELU2, O.E4M3, st)
    a2 = st.read()
    m1 = int(np.max(bf16_np(b1) & 0x7FFF)) << 16
    m2 = int(np.max(bf16_np(b2) & 0x7FFF)) << 16
    assert a1["amax_acc"] == m1 and a2["amax_acc"] == max(m1, m2)
    assert a2["sat_acc"] >= a1["sat_acc"]
