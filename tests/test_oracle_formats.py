"""Pins for the oracle's number formats (CPU only).

Facts the pages print: "FP8 training: what it is and how it works" -- Step 1
(E4M3 largest 448, gap after 1 of 0.125; E5M2 largest 57344, gap 0.25), Step 2
(E4M3 smallest nonzero 0.001953, smallest normal 0.015625), the worked example
(normal range about 4.46 orders of magnitude) and the follow-up questions (E5M2
smallest nonzero near 0.000015); "FP8 Training & Inference" -- FP8 Formats
(8 values per power-of-2 interval for E4M3, 4 for E5M2) and Exercise 1 (a 128x
range ratio); "Pretraining at scale" 4a (BF16 bit layout of 1/3).
"""
import math

import numpy as np
import pytest

import oracle as O
import refcheck as R


def test_format_facts_printed_on_pages():
    t4 = O.fp8_decode_table(O.E4M3)
    t5 = O.fp8_decode_table(O.E5M2)
    fin4 = t4[np.isfinite(t4)]
    fin5 = t5[np.isfinite(t5)]
    assert fin4.max() == 448.0
    assert fin5.max() == 57344.0
    assert fin5.max() / fin4.max() == 128.0                    # Exercise 1
    pos4 = np.unique(fin4[fin4 > 0])
    pos5 = np.unique(fin5[fin5 > 0])
    # gap between 1 and the next number
    assert pos4[np.searchsorted(pos4, 1.0) + 1] - 1.0 == 0.125
    assert pos5[np.searchsorted(pos5, 1.0) + 1] - 1.0 == 0.25
    # smallest nonzero / smallest normal (printed as 0.001953 and 0.015625)
    assert round(pos4[0], 6) == 0.001953 and pos4[0] == 2.0 ** -9
    assert pos4[7] == 0.015625                                   # 7 subnormals, then 2^-6
    assert abs(pos5[0] - 0.000015) < 1e-6 and pos5[0] == 2.0 ** -16
    # values per power-of-2 interval
    assert np.sum((pos4 >= 1) & (pos4 < 2)) == 8
    assert np.sum((pos5 >= 1) & (pos5 < 2)) == 4
    # normal range of E4M3: log10(448 / 0.015625) ~ 4.46 orders of magnitude
    assert round(math.log10(448 / 0.015625), 2) == 4.46
    # NaN codes: E4M3 only S.1111.111; E5M2 exponent all ones with mantissa != 0
    assert sorted(np.flatnonzero(np.isnan(t4)).tolist()) == [0x7F, 0xFF]
    assert sorted(np.flatnonzero(np.isnan(t5)).tolist()) == [0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF]
    assert t5[0x7C] == np.inf and t5[0xFC] == -np.inf
    assert not np.isinf(t4).any()


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_decode_matches_library_all_codes(fmt):
    mine = O.fp8_decode_table(fmt)
    lib = R.torch_decode_table(fmt)
    same = (mine == lib) | (np.isnan(mine) & np.isnan(lib))
    assert same.all()
    # signed zero
    assert np.signbit(mine[0x80]) and not np.signbit(mine[0x00])


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_encode_every_rounding_boundary_vs_nearest_search(fmt):
    x = R.boundary_values(fmt)
    got = O.fp8_encode(x, fmt)
    exp = R.nearest_code(x, fmt)
    bad = np.flatnonzero(got != exp)
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(exp[i])) for i in bad[:10]]


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_encode_random_bits_vs_nearest_search(fmt):
    rng = np.random.default_rng(123 + fmt)
    u = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    # bias half the samples into the format's dynamic range
    near = rng.uniform(-40, 20, size=200_000)
    y = (np.sign(rng.standard_normal(200_000)) * 2.0 ** near).astype(np.float32)
    x = np.concatenate([u.view(np.float32), y])
    got = O.fp8_encode(x, fmt)
    exp = R.nearest_code(x, fmt)
    assert np.array_equal(got, exp)


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_encode_vs_library_cast_on_clamped_inputs(fmt):
    rng = np.random.default_rng(7 + fmt)
    u = rng.integers(0, 2 ** 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[~np.isnan(x)]
    m = R.FMAX[fmt]
    xc = np.clip(x, -m, m).astype(np.float32)
    assert np.array_equal(O.fp8_encode(xc, fmt), R.torch_cast_codes(xc, fmt))
    # the scaled-range band where most real values land
    y = (rng.standard_normal(2_000_000) * 2.0 ** rng.uniform(-20, 10, 2_000_000)).astype(np.float32)
    y = np.clip(y, -m, m)
    assert np.array_equal(O.fp8_encode(y, fmt), R.torch_cast_codes(y, fmt))


def test_encode_special_values():
    for fmt, top in [(O.E4M3, 0x7E), (O.E5M2, 0x7B)]:
        x = np.array([np.inf, -np.inf, np.nan, -np.nan, 0.0, -0.0, 1e38, -1e38], dtype=np.float32)
        c = O.fp8_encode(x, fmt)
        assert c.tolist() == [top, 0x80 | top, 0x7F, 0xFF, 0x00, 0x80, top, 0x80 | top]
    # flush boundary: exactly half the smallest subnormal is a tie -> even code 0
    assert O.fp8_encode(np.float32(2.0 ** -10), O.E4M3) == 0x00
    assert O.fp8_encode(np.nextafter(np.float32(2.0 ** -10), np.float32(1)), O.E4M3) == 0x01
    assert O.fp8_encode(np.float32(-(2.0 ** -17)), O.E5M2) == 0x80
    # 464 is the tie between 448 and the (NaN) next step: even -> 448, no saturation
    assert O.fp8_encode(np.float32(464.0), O.E4M3) == 0x7E


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_saturation_predicate_vs_library_nonsaturating_cast(fmt):
    x = R.boundary_values(fmt)
    rng = np.random.default_rng(11)
    y = (rng.standard_normal(1_000_000) * R.FMAX[fmt] * 1.2).astype(np.float32)
    for arr in (x, y):
        assert np.array_equal(O.fp8_saturates(arr, fmt), R.torch_overflows(arr, fmt))
    # thresholds: E4M3 counts |v| > 464, E5M2 counts |v| >= 61440
    assert not O.fp8_saturates(np.float32(464.0), O.E4M3)
    assert O.fp8_saturates(np.nextafter(np.float32(464.0), np.float32(1e9)), O.E4M3)
    assert O.fp8_saturates(np.float32(61440.0), O.E5M2)
    assert not O.fp8_saturates(np.nextafter(np.float32(61440.0), np.float32(0)), O.E5M2)
    assert not O.fp8_saturates(np.float32(np.nan), fmt)
    assert O.fp8_saturates(np.float32(-np.inf), fmt)


def test_bf16_rne_vs_library():
    rng = np.random.default_rng(5)
    u = rng.integers(0, 2 ** 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    # every tie and near-tie pattern in the low 16 bits over many high halves
    hi = rng.integers(0, 2 ** 16, size=20000, dtype=np.uint64).astype(np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    v = (hi[:, None] | lows[None, :]).reshape(-1)
    special = np.array([0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x00008000, 0x00018000, 0x80008000,
                        0x7F800000, 0xFF800000, 0x00000000, 0x80000000, 0x00000001],
                       dtype=np.uint32)
    x = np.concatenate([u, v, special]).view(np.float32)
    fin = ~np.isnan(x)
    got = O.bf16_rne(x[fin])
    assert np.array_equal(got, R.torch_bf16(x[fin]))
    # NaN stays NaN with its sign
    n = O.bf16_rne(x[~fin])
    assert np.all((n & 0x7F80) == 0x7F80) and np.all((n & 0x007F) != 0)
    assert np.array_equal(n >> 15, (x[~fin].view(np.uint32) >> 31).astype(np.uint16))


def test_bf16_one_third_worked_example():
    # "Pretraining at scale" 4a: 1/3 in bf16 has sign 0, exponent field 125,
    # fraction field 43 and value 0.333984375.
    b = int(O.bf16_rne(np.array([1.0 / 3.0], dtype=np.float32))[0])
    assert b >> 15 == 0 and (b >> 7) & 0xFF == 125 and b & 0x7F == 43
    assert float(O.bf16_to_f32(np.array([b], dtype=np.uint16))[0]) == 0.333984375
