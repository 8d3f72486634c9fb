"""Backward of the squared ReLU from the cached activation (GPU).

"FP8 training: what it is and how it works", Step 3: the activations kept for
the backward pass may be stored in FP8.  relu2_backward_quantize computes
dH = dA * 2 sqrt(A) from the cached A (FP8 codes with their inverse scale, or
the BF16 copy) and casts it with the gradient state's delayed scale.  Parity:
bit for bit against oracle.relu2_backward (BF16 copy of dH, codes, amax and
saturation count in the state) over both codecs, all cache kinds, both output
formats and ragged lengths, and on the GPT-2 activation at full size.  The
square root it uses is checked on all 2^32 binary32 inputs against numpy's
(IEEE, correctly rounded).
"""
import numpy as np
import pytest
import torch

import oracle as O
import scaled_quantization_amd as sq
import workloads
from gpu_util import DEV, THREADS, bf16_np, device_arange_f32, oracle_quantize, to_dev_bf16, \
    to_dev_u8, u8_np

pytestmark = pytest.mark.gpu

CHUNK = 1 << 28


@pytest.fixture(params=[0, 1], ids=["hw", "int"])
def codec(request):
    prev = sq.fp8dp_set_codec(request.param)
    yield request.param
    sq.fp8dp_set_codec(prev)


def test_square_root_every_binary32_input():
    out = torch.empty(CHUNK, dtype=torch.float32, device=DEV)
    for lo in range(0, 1 << 32, CHUNK):
        x = device_arange_f32(lo, CHUNK)
        sq.fp8dp_convert_f32(x, 5, out)
        got = out.cpu().numpy()
        xs = (np.arange(lo, lo + CHUNK, dtype=np.uint64).astype(np.uint32)).view(np.float32)
        with np.errstate(invalid="ignore"):
            exp = np.sqrt(xs)
        same = (got.view(np.uint32) == exp.view(np.uint32)) | (np.isnan(got) & np.isnan(exp))
        if not same.all():
            bad = np.flatnonzero(~same)[:8]
            raise AssertionError([(hex(lo + int(i)), got[i], exp[i]) for i in bad])
        del x


def _inputs(rng, n, cache):
    h = torch.from_numpy(rng.standard_normal(n).astype(np.float32))
    a = (torch.relu(h) ** 2).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    dA = torch.from_numpy((rng.standard_normal(n) * np.exp2(rng.integers(-6, 6, n))).astype(
        np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if cache == O.CACHE_BF16:
        return dA, a, 1.0
    s = O.scale_from_amax(float(((a.astype(np.uint32) << 16).view(np.float32)).max()), 1.25,
                          cache)[0][0]
    r = O.quantize(a, O.ACT_IDENTITY, cache, O.PER_TENSOR, float(s), want_bf16=False)
    return dA, r.fp8.reshape(-1), float(np.float32(1.0) / np.float32(s))


def _run(dA, cache_arr, cache, si, fmt, st, want_bf16=True):
    n = dA.size
    d = to_dev_bf16(dA.reshape(1, -1))
    c = to_dev_bf16(cache_arr.reshape(1, -1)) if cache == O.CACHE_BF16 else \
        to_dev_u8(cache_arr.reshape(1, -1))
    si_t = torch.tensor([si], dtype=torch.float32, device=DEV)
    q = torch.empty((1, n), dtype=torch.uint8, device=DEV)
    b = torch.empty((1, n), dtype=torch.bfloat16, device=DEV) if want_bf16 else None
    sq.relu2_backward_quantize(d, c, cache, si_t, fmt, st, q, b)
    return b, q


@pytest.mark.parametrize("fmt", [O.E5M2, O.E4M3], ids=["e5m2", "e4m3"])
@pytest.mark.parametrize("cache", [O.E4M3, O.E5M2, O.CACHE_BF16], ids=["c-e4m3", "c-e5m2", "c-bf16"])
@pytest.mark.parametrize("n", [8, 1003, 65536 + 5, 1 << 20])
def test_relu2_backward_vs_oracle(n, cache, fmt, codec):
    rng = np.random.default_rng(n + 3 * cache + fmt)
    dA, c, si = _inputs(rng, n, cache)
    st = sq.TensorState(fmt, 1, 1.25, 1.0)
    ost = O.State(fmt, 1, 1.25, 1.0)
    b, q = _run(dA, c, cache, si, fmt, st)
    r = O.relu2_backward(dA, c, cache, si, fmt, ost.scale)
    assert np.array_equal(bf16_np(b).reshape(-1), r.bf16)
    assert np.array_equal(u8_np(q).reshape(-1), r.fp8)
    d = st.read()
    assert d["amax_acc"] == r.amax_bits and d["sat_acc"] == r.sat


@pytest.mark.parametrize("cache", [O.E4M3, O.CACHE_BF16], ids=["c-e4m3", "c-bf16"])
@pytest.mark.parametrize("want_bf16", [True, False], ids=["bf16", "codes"])
def test_relu2_backward_does_not_depend_on_grid_size(cache, want_bf16):
    """No grid limit: one or two vectors per thread without a loop, by the
    launch's read/write mix; small limits: the grid-stride loop.  Same bytes,
    same accumulators, and the oracle's."""
    n = 40000 + 3
    rng = np.random.default_rng(77 + cache)
    dA, c, si = _inputs(rng, n, cache)
    outs = []
    for limit in (0, 1, 7, 100):
        prev = sq.fp8dp_set_grid_limit(limit)
        try:
            st = sq.TensorState(O.E5M2, 1, 1.25, 1.0)
            b, q = _run(dA, c, cache, si, O.E5M2, st, want_bf16)
            d = st.read()
            outs.append((None if b is None else bf16_np(b).tobytes(), u8_np(q).tobytes(),
                         d["amax_acc"], d["sat_acc"]))
        finally:
            sq.fp8dp_set_grid_limit(prev)
    assert all(o == outs[0] for o in outs)
    r = O.relu2_backward(dA, c, cache, si, O.E5M2, O.State(O.E5M2, 1, 1.25, 1.0).scale)
    assert outs[0][1] == r.fp8.tobytes() and outs[0][2] == r.amax_bits
    if want_bf16:
        assert outs[0][0] == r.bf16.tobytes()


def test_relu2_backward_special_values(codec):
    # zero, exact squares, NaN / negative / infinite cache values, zero and
    # infinite gradients
    a = np.array([0x0000, 0x4080, 0x4010, 0x7FC0, 0xBF80, 0x7F80, 0x3F80, 0x3F80,
                  0x0001, 0x0000, 0x4080], np.uint16)
    dA = np.array([0x4040, 0x4040, 0xBF80, 0x3F80, 0x3F80, 0x3F80, 0x7F80, 0x0000,
                   0x3F80, 0x8000, 0xFF80], np.uint16)
    st = sq.TensorState(O.E5M2, 1, 1.0, 1.0)
    b, q = _run(dA, a, O.CACHE_BF16, 1.0, O.E5M2, st)
    ost = O.State(O.E5M2, 1, 1.0, 1.0)
    r = O.relu2_backward(dA, a, O.CACHE_BF16, 1.0, O.E5M2, ost.scale)
    got_b, got_q = bf16_np(b).reshape(-1), u8_np(q).reshape(-1)
    nan_b = (r.bf16 & 0x7FFF) > 0x7F80
    # NaN results match as NaN (their sign is not specified); everything else bit for bit
    assert np.array_equal(got_b[~nan_b], r.bf16[~nan_b])
    assert ((got_b[nan_b] & 0x7FFF) > 0x7F80).all()
    assert np.array_equal(got_q[~nan_b], r.fp8[~nan_b])
    assert ((got_q[nan_b] & 0x7F) == 0x7F).all()


def test_relu2_backward_gpt2_full_size():
    """The GPT-2 MLP activation A = relu2(H0) cached as E4M3 with its delayed
    scale, dA [16384 x 3072] signed log-normal: dH as E5M2 with the gradient
    state, checked element for element."""
    w = workloads.get("gpt2")
    h = w.h0()
    s_a = 11.0
    ra = oracle_quantize(h, O.ACT_RELU2, O.E4M3, O.PER_TENSOR, s_a, want_bf16=False)
    del h
    dA = w.da()
    si = float(np.float32(1.0) / np.float32(s_a))
    st = sq.TensorState(O.E5M2, 1, 1.25, 1.0)
    ost = O.State(O.E5M2, 1, 1.25, 1.0)
    d = to_dev_bf16(dA)
    c = to_dev_u8(ra.fp8)
    si_t = torch.tensor([si], dtype=torch.float32, device=DEV)
    q = torch.empty(dA.shape, dtype=torch.uint8, device=DEV)
    b = torch.empty(dA.shape, dtype=torch.bfloat16, device=DEV)
    sq.relu2_backward_quantize(d, c, sq.CACHE_E4M3, si_t, sq.E5M2, st, q, b)
    from concurrent.futures import ThreadPoolExecutor
    rows = dA.shape[0]
    step = rows // (4 * THREADS)
    with ThreadPoolExecutor(THREADS) as ex:
        parts = list(ex.map(lambda r0: O.relu2_backward(dA[r0:r0 + step], ra.fp8[r0:r0 + step],
                                                        O.E4M3, si, O.E5M2, ost.scale),
                            range(0, rows, step)))
    assert np.array_equal(bf16_np(b), np.concatenate([p.bf16 for p in parts]))
    assert np.array_equal(u8_np(q), np.concatenate([p.fp8 for p in parts]))
    dd = st.read()
    assert dd["amax_acc"] == max(p.amax_bits for p in parts)
    assert dd["sat_acc"] == sum(p.sat for p in parts)


def test_relu2_backward_errors():
    L = sq.lib()
    assert L.relu2_backward_quantize(16, 16, 0, None, 4, 8, 1, 16, None, 16, None) == -1
    assert L.relu2_backward_quantize(16, 16, 5, 16, 4, 8, 1, 16, None, 16, None) == -1
    assert L.relu2_backward_quantize(16, 16, 2, None, 4, 8, 1, 24, None, 16, None) == -1
