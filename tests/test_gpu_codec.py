"""Device conversion routines against the oracle (GPU).

* The FP8 cast the kernels use, for every one of the 2^32 binary32 inputs,
  with both the hardware-instruction path and the integer path (the kernels
  choose per 8-value vector exactly as fp8dp_convert_f32 does).
* BF16 rounding and the saturation predicate on boundary sets and a large
  random sample.
* The scale rule (binary32 max / (amax * margin), correctly rounded) on every
  positive finite BF16 amax ("FP8 training: what it is and how it works",
  Step 2).
"""
import numpy as np
import pytest
import torch

import oracle as O
import refcheck as R
import scaled_quantization_amd as sq
from gpu_util import DEV, device_arange_f32, encode_range_parallel

pytestmark = pytest.mark.gpu

CHUNK = 1 << 28


@pytest.fixture(params=[0, 1], ids=["hw", "int"])
def codec(request):
    prev = sq.fp8dp_set_codec(request.param)
    yield request.param
    sq.fp8dp_set_codec(prev)


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2], ids=["e4m3", "e5m2"])
def test_fp8_cast_every_binary32_input(fmt, codec):
    out = torch.empty(CHUNK, dtype=torch.uint8, device=DEV)
    for lo in range(0, 1 << 32, CHUNK):
        x = device_arange_f32(lo, CHUNK)
        sq.fp8dp_convert_f32(x, fmt, out)
        got = out.cpu().numpy()
        exp = encode_range_parallel(lo, lo + CHUNK, fmt)
        if not np.array_equal(got, exp):
            bad = np.flatnonzero(got != exp)[:8]
            raise AssertionError([(hex(lo + int(i)), hex(got[i]), hex(exp[i])) for i in bad])
        del x


def _sample_f32():
    rng = np.random.default_rng(2024)
    u = rng.integers(0, 2 ** 32, size=1 << 24, dtype=np.uint64).astype(np.uint32)
    hi = rng.integers(0, 2 ** 16, size=1 << 16, dtype=np.uint64).astype(np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000],
                    dtype=np.uint32)
    ties = (hi[:, None] | lows[None, :]).reshape(-1)
    b4 = R.boundary_values(O.E4M3).view(np.uint32)
    b5 = R.boundary_values(O.E5M2).view(np.uint32)
    allu = np.concatenate([u, ties, b4, b5])
    pad = (-allu.size) % 8
    allu = np.concatenate([allu, np.zeros(pad, dtype=np.uint32)])
    return allu.view(np.float32)


def test_bf16_rounding_sampled(codec):
    x = _sample_f32()
    xd = torch.from_numpy(x).to(DEV)
    out = torch.empty(x.size, dtype=torch.int16, device=DEV)
    sq.fp8dp_convert_f32(xd, 2, out)
    got = out.cpu().numpy().view(np.uint16)
    exp = O.bf16_rne(x)
    assert np.array_equal(got, exp)


def test_saturation_predicate_sampled():
    x = _sample_f32()
    xd = torch.from_numpy(x).to(DEV)
    out = torch.empty(x.size, dtype=torch.uint8, device=DEV)
    for fmt, target in ((O.E4M3, 3), (O.E5M2, 4)):
        sq.fp8dp_convert_f32(xd, target, out)
        got = out.cpu().numpy().astype(bool)
        assert np.array_equal(got, O.fp8_saturates(x, fmt))


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2], ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("margin", [1.0, 1.25, 3.0e38])
def test_scale_rule_every_bf16_amax(fmt, margin):
    bits = np.arange(0, 0x10000, dtype=np.uint32) << 16        # every BF16 pattern, NaN included
    amax = bits.view(np.float32)
    ad = torch.from_numpy(amax).to(DEV)
    s = torch.empty_like(ad)
    si = torch.empty_like(ad)
    sq.fp8dp_scale_rule(ad, margin, fmt, s, si)
    es, esi = O.scale_from_amax(amax, margin, fmt)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), es.view(np.uint32))
    assert np.array_equal(si.cpu().numpy().view(np.uint32), esi.view(np.uint32))
