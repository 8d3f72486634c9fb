"""Pins for the oracle's quantizer, scale rule and delayed-scaling state (CPU only).

The quantizer is checked against a brute-force composition built from torch's
casts and a nearest-neighbour search (tests/refcheck.py); the scale rule
against numpy float32 division over every positive finite BF16 amax; the
delayed-scaling recurrence against its closed form on the tiny workload
("Paradigma Details FP8 ..." -- previous step's amax times a safety margin;
"FP8 training ..." -- Trade-offs: delayed scaling keeps a history of amaxes).
"""
import collections

import numpy as np
import pytest

import oracle as O
import refcheck as R
import workloads


def _special_inputs(rng, rows, cols):
    x = (rng.standard_normal((rows, cols)) * 2.0 ** rng.uniform(-30, 12, (rows, cols)))
    h = R.torch_bf16(x.astype(np.float32))
    specials = np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x0000, 0x8000, 0x0001, 0x8001,
                         0x7F7F, 0xFF7F, 0x0080, 0x1F80, 0x3F80, 0xBF80, 0x4400, 0x43E0,
                         0x5F80, 0x2000, 0x2080, 0x1000], dtype=np.uint16)
    h.reshape(-1)[: specials.size] = specials
    return h


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
@pytest.mark.parametrize("act", [O.ACT_IDENTITY, O.ACT_RELU2])
@pytest.mark.parametrize("scale", [1.0, 358.4, 0.00448, 3.0e-7, 1.7e30])
def test_quantize_per_tensor_vs_brute_force(fmt, act, scale):
    rng = np.random.default_rng(hash((fmt, act, scale)) & 0xFFFF)
    h = _special_inputs(rng, 8, 256)
    got = O.quantize(h, act, fmt, O.PER_TENSOR, scale)
    b, codes, amax, sat, _ = R.brute_quantize(h, act == O.ACT_RELU2, fmt, np.float32(scale))
    assert np.array_equal(got.bf16, b)
    assert np.array_equal(got.fp8, codes)
    assert got.amax_bits == amax
    assert got.sat == sat


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
@pytest.mark.parametrize("act", [O.ACT_IDENTITY, O.ACT_RELU2])
def test_quantize_per_group_vs_brute_force(fmt, act):
    rng = np.random.default_rng(99 + fmt + 2 * act)
    h = _special_inputs(rng, 6, 512)
    h[2, 128:256] = 0            # an all-zero group -> amax 0 -> fallback scale 1
    h[3, 0:128] = 0x0001         # a group of tiny subnormals -> quotient overflows -> fallback
    got = O.quantize(h, act, fmt, O.PER_GROUP128)
    b, codes, amax, sat, gsi = R.brute_quantize(h, act == O.ACT_RELU2, fmt, group=True)
    assert np.array_equal(got.bf16, b)
    assert np.array_equal(got.fp8, codes)
    assert got.amax_bits == amax
    assert got.sat == sat
    assert np.array_equal(got.group_scale_inv.view(np.uint32), gsi.view(np.uint32))


def test_group_invariants_student_t():
    # current per-group scaling maps each group's amax onto the format maximum:
    # every group with a usable scale holds a +-max code and nothing saturates.
    h = workloads.student_t(77, 64, 1024)
    for fmt, top in ((O.E4M3, 0x7E), (O.E5M2, 0x7B)):
        r = O.quantize(h, O.ACT_IDENTITY, fmt, O.PER_GROUP128)
        assert r.sat == 0
        codes = r.fp8.reshape(64, 8, 128) & 0x7F
        assert np.all((codes == top).any(axis=2))


def test_fused_equals_naive_three_pass():
    # Reading: the FP8 copy is cast from the BF16 copy.  Then quantizing the
    # stored BF16 copy again (identity) with the same scale gives the same
    # bytes -- the naive write / scan / reread path and the fused path agree.
    h = workloads.normal(5, 64, 512)
    fused = O.quantize(h, O.ACT_RELU2, O.E4M3, O.PER_TENSOR, 123.25)
    naive = O.quantize(fused.bf16, O.ACT_IDENTITY, O.E4M3, O.PER_TENSOR, 123.25)
    assert np.array_equal(fused.fp8, naive.fp8)
    assert fused.amax_bits == naive.amax_bits and fused.sat == naive.sat
    # and a current-scaling naive pass: scan, scale, cast
    s, _ = O.scale_from_amax(fused.amax, 1.0, O.E4M3)
    naive2 = O.quantize(fused.bf16, O.ACT_IDENTITY, O.E4M3, O.PER_TENSOR, float(s[0]))
    assert naive2.sat == 0 and ((naive2.fp8 & 0x7F) == 0x7E).any()


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
@pytest.mark.parametrize("margin", [1.0, 1.25])
def test_scale_rule_all_bf16_amax_values(fmt, margin):
    bits = np.arange(0, 0x7F80, dtype=np.uint32) << 16        # +0 .. largest finite BF16
    amax = bits.view(np.float32)
    s, sinv = O.scale_from_amax(amax, margin, fmt)
    exp = R.np_scale(amax, margin, fmt)
    assert np.array_equal(s.view(np.uint32), exp.view(np.uint32))
    with np.errstate(all="ignore"):
        assert np.array_equal(sinv.view(np.uint32), (np.float32(1) / exp).view(np.uint32))
    # the fallback happens exactly where the quotient cannot be formed: amax 0,
    # amax * margin overflowing, and tiny amax values whose quotient overflows
    with np.errstate(all="ignore"):
        d = (amax * np.float32(margin)).astype(np.float32)
        q = np.float32(R.FMAX[fmt]) / d
    fallback = (d == 0) | ~np.isfinite(d) | ~np.isfinite(q)
    assert np.array_equal(s == 1.0, fallback | (q == 1.0))
    assert fallback.sum() > 1


def test_scale_rule_degenerate_cases():
    for a in [0.0, -0.0, np.nan, np.inf, 1e-45]:
        for fmt in (O.E4M3, O.E5M2):
            s, _ = O.scale_from_amax(np.float32(a), 1.25, fmt)
            assert s[0] == 1.0, (a, fmt)
    # 448 / 2^-126 overflows binary32 (falls back); 448 / 2^-118 = 1.75 * 2^126 does not
    s, _ = O.scale_from_amax(np.float32(2.0 ** -126), 1.0, O.E4M3)
    assert s[0] == 1.0
    s, _ = O.scale_from_amax(np.float32(2.0 ** -118), 1.0, O.E4M3)
    assert s[0] == np.float32(1.75 * 2.0 ** 126)


def _tiny_amax(h):
    x = R.f32_from_bf16(h)
    a = np.where(x > 0, (x * x).astype(np.float32), np.float32(0)).astype(np.float32)
    return float(np.abs(R.f32_from_bf16(R.torch_bf16(a))).max())


def test_delayed_recurrence_tiny_closed_form():
    w = workloads.get("tiny")
    h0 = w.h0()
    st = O.State(O.E4M3, hist_len=1, margin=1.25, initial_amax=1.0)
    assert st.scale == np.float32(448.0) / np.float32(1.25) == np.float32(358.4)
    expected_scale = np.float32(358.4)
    for t in range(w.steps):
        h = w.h_step(t, h0)
        assert st.scale == expected_scale
        r = O.quantize(h, O.ACT_RELU2, O.E4M3, O.PER_TENSOR, st.scale)
        amax = _tiny_amax(h)                       # brute force, independent of the oracle
        assert r.amax == amax
        st.accumulate(r.amax_bits, r.sat)
        used = st.scale
        st.update()
        assert st.scale_inv_used == np.float32(1.0) / np.float32(used)
        assert st.history[0] == np.float32(amax)
        expected_scale = np.float32(448.0) / np.float32(np.float32(amax) * np.float32(1.25))
        # step 0 is cast with the cold-start scale 358.4 and an amax near 20: it saturates
        if t == 0:
            assert st.overflow == 1 and st.sat_last > 0
        else:
            assert st.overflow == 0 and st.sat_last == 0
        assert st.amax_acc == 0 and st.sat_acc == 0 and st.steps == t + 1


def test_history_window_max_and_ring():
    # hist_len > 1: the next scale uses the largest amax in the window
    amaxes = [3.0, 1.0, 7.5, 2.0, 0.5, 0.25, 9.0, 1.0]
    L = 3
    st = O.State(O.E5M2, hist_len=L, margin=2.0, initial_amax=4.0)
    window = collections.deque([4.0] * L, maxlen=L)
    for a in amaxes:
        st.accumulate(int(np.float32(a).view(np.uint32)), 0)
        st.update()
        window.append(a)
        exp = np.float32(57344.0) / np.float32(np.float32(max(window)) * np.float32(2.0))
        assert st.scale == exp
    assert sorted(st.history.tolist()) == sorted(window)


def test_accumulate_combines_calls_by_max_and_sum():
    st = O.State(O.E4M3)
    st.accumulate(int(np.float32(2.0).view(np.uint32)), 3)
    st.accumulate(int(np.float32(5.0).view(np.uint32)), 4)
    st.accumulate(int(np.float32(1.0).view(np.uint32)), 0)
    assert st.amax_acc == int(np.float32(5.0).view(np.uint32)) and st.sat_acc == 7
    st.update()
    assert st.sat_last == 7 and st.overflow == 1 and st.history[0] == 5.0


def test_amax_jump_saturates_and_flags_overflow():
    # "FP8 Training & Inference", Exercise 5 / Delayed Scaling: a sudden jump of
    # the activation magnitude overflows the delayed scale and must be detected.
    h = workloads.normal(9, 256, 512)
    st = O.State(O.E4M3, hist_len=1, margin=1.25, initial_amax=1.0)
    r = O.quantize(h, O.ACT_IDENTITY, O.E4M3, O.PER_TENSOR, st.scale)
    st.accumulate(r.amax_bits, r.sat)
    st.update()
    r = O.quantize(h, O.ACT_IDENTITY, O.E4M3, O.PER_TENSOR, st.scale)
    assert r.sat == 0                                 # same statistics: in range
    h8 = workloads.scale_bf16(h, 8.0)
    r8 = O.quantize(h8, O.ACT_IDENTITY, O.E4M3, O.PER_TENSOR, st.scale)
    x8 = np.abs(R.f32_from_bf16(h8)) * st.scale
    assert r8.sat == int(np.sum(x8 > 464.0)) > 0
    st.accumulate(r8.amax_bits, r8.sat)
    st.update()
    assert st.overflow == 1


def test_state_rejects_bad_history_length():
    with pytest.raises(ValueError):
        O.State(O.E4M3, hist_len=0)
    with pytest.raises(ValueError):
        O.State(O.E4M3, hist_len=O.MAX_HIST + 1)


@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2])
def test_weight_blocks_vs_brute_force(fmt):
    w = workloads.normal(31, 256, 384, std=0.02)
    w[0, 0] = R.torch_bf16(np.array([3.0], dtype=np.float32))[0]       # outlier in block (0, 0)
    w[200, 300] = 0x7F80                                                # +inf in block (1, 2)
    q, si = O.quantize_weight_blocks(w, fmt)
    for bi in range(2):
        for bj in range(3):
            blk = w[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
            amax = np.float32(np.abs(R.f32_from_bf16(blk)).max())
            s = R.np_scale(amax, 1.0, fmt)
            with np.errstate(all="ignore"):
                assert si[bi, bj].view(np.uint32) == (np.float32(1) / s).view(np.uint32)
                v = (R.f32_from_bf16(blk) * s).astype(np.float32)
            exp = R.nearest_code(v, fmt).reshape(128, 128)
            assert np.array_equal(q[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128], exp)
    # only the block with the infinity falls back to scale 1
    assert si[1, 2] == 1.0 and np.all(si[0] != 1.0)


def test_weight_tensor_current_scaling():
    w = workloads.normal(32, 128, 256, std=0.02)
    q, s, si = O.quantize_weight_tensor(w, O.E4M3)
    amax = np.float32(np.abs(R.f32_from_bf16(w)).max())
    assert s == R.np_scale(amax, 1.0, O.E4M3) and si == np.float32(1) / np.float32(s)
    assert ((q & 0x7F) == 0x7E).sum() >= 1
    exp = R.nearest_code((R.f32_from_bf16(w) * np.float32(s)).astype(np.float32), O.E4M3)
    assert np.array_equal(q, exp.reshape(q.shape))
