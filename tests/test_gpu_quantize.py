"""Fused quantizer, delayed-scaling state, weight cast and the naive three-pass
comparison against the oracle (GPU).  Bit-exact: BF16 copies, FP8 codes,
group scales, amax and saturation counts.

Workloads are the seeded synthetic ones of workloads.py at their full sizes
(tiny, GPT-2-scale, outlier stress, fine-grained, large) plus edge cases:
every BF16 input pattern, ragged element counts, NaN / infinity / subnormal
inputs, and several grid sizes.
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


def _run(h_np, act, fmt, mode, st, want_bf16=True, want_fp8=True):
    rows, cols = h_np.shape
    h = to_dev_bf16(h_np)
    b = torch.empty_like(h) if want_bf16 else None
    q = torch.empty((rows, cols), dtype=torch.uint8, device=DEV) if want_fp8 else None
    g = (torch.empty((rows, cols // 128), dtype=torch.float32, device=DEV)
         if mode == sq.PER_GROUP128 else None)
    sq.quantize_fused(h, act, fmt, mode, st, b, q, g)
    return b, q, g


def _compare_state(st: sq.TensorState, ost: O.State):
    d = st.read()
    for k in ("scale", "scale_inv", "scale_inv_used", "overflow", "sat_last", "hist_pos", "steps"):
        assert d[k] == getattr(ost, k), (k, d[k], getattr(ost, k))
    assert d["history"][: ost.hist_len] == list(ost.history)
    assert d["amax_acc"] == 0 and d["sat_acc"] == 0


def test_state_init_matches_oracle():
    for fmt, L, margin, a0 in ((0, 1, 1.25, 1.0), (1, 4, 2.0, 3.5), (0, 16, 1.0, 0.0),
                               (1, 2, 1.25, float("nan"))):
        st = sq.TensorState(fmt, L, margin, a0)
        ost = O.State(fmt, L, margin, a0)
        d = st.read()
        assert d["scale"] == ost.scale and d["scale_inv"] == ost.scale_inv
        assert d["hist_len"] == L and d["steps"] == 0 and d["sat_acc"] == 0


def test_tiny_four_delayed_steps(codec):
    w = workloads.get("tiny")
    h0 = w.h0()
    st = sq.TensorState(sq.E4M3, 1, w.margin, w.initial_amax)
    ost = O.State(O.E4M3, 1, w.margin, w.initial_amax)
    for t in range(w.steps):
        h = w.h_step(t, h0)
        b, q, _ = _run(h, sq.ACT_RELU2, sq.E4M3, sq.PER_TENSOR, st)
        r = O.quantize(h, O.ACT_RELU2, O.E4M3, O.PER_TENSOR, ost.scale)
        assert np.array_equal(bf16_np(b), r.bf16), t
        assert np.array_equal(u8_np(q), r.fp8), t
        d = st.read()
        assert d["amax_acc"] == r.amax_bits and d["sat_acc"] == r.sat, t
        sq.amax_history_update(st)
        ost.accumulate(r.amax_bits, r.sat)
        ost.update()
        _compare_state(st, ost)
    assert ost.steps == 4


@pytest.mark.parametrize("fmt", [0, 1], ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("act", [0, 1], ids=["identity", "relu2"])
def test_every_bf16_input_pattern(fmt, act, codec):
    h = np.arange(0x10000, dtype=np.uint32).astype(np.uint16).reshape(512, 128)
    for scale in (1.0, 358.4, 0.00448, 3.0e-7, 1.7e30, 2.0 ** -140):
        st = sq.TensorState(fmt, 1, 1.0, 1.0)
        # set the multiplier directly: a one-step history with amax = max / scale
        # is not exact, so write the scale field
        st.buf[0:4] = torch.tensor([scale], dtype=torch.float32).view(torch.uint8).to(DEV)
        b, q, _ = _run(h, act, fmt, sq.PER_TENSOR, st)
        s32 = float(np.float32(scale))
        r = O.quantize(h, act, fmt, O.PER_TENSOR, s32)
        assert np.array_equal(bf16_np(b), r.bf16)
        assert np.array_equal(u8_np(q), r.fp8), scale
        d = st.read()
        assert d["amax_acc"] == r.amax_bits and d["sat_acc"] == r.sat, scale
    # group mode over the same patterns (each row is one group)
    b, q, g = _run(h, act, fmt, sq.PER_GROUP128, None)
    r = O.quantize(h, act, fmt, O.PER_GROUP128)
    assert np.array_equal(bf16_np(b), r.bf16)
    assert np.array_equal(u8_np(q), r.fp8)
    assert np.array_equal(g.cpu().numpy().view(np.uint32), r.group_scale_inv.view(np.uint32))


@pytest.mark.parametrize("shape", [(1, 1), (1, 7), (3, 1001), (129, 129), (2, 4096 + 5),
                                   (1000, 24)])
def test_ragged_element_counts(shape, codec):
    h = workloads.normal(41, *shape)
    h.reshape(-1)[-1] = 0x7FC0                   # NaN in the tail
    st = sq.TensorState(sq.E4M3, 1, 1.25, 0.5)
    b, q, _ = _run(h, sq.ACT_RELU2, sq.E4M3, sq.PER_TENSOR, st)
    ost = O.State(O.E4M3, 1, 1.25, 0.5)
    r = O.quantize(h, O.ACT_RELU2, O.E4M3, O.PER_TENSOR, ost.scale)
    assert np.array_equal(bf16_np(b), r.bf16)
    assert np.array_equal(u8_np(q), r.fp8)
    d = st.read()
    assert d["amax_acc"] == r.amax_bits and d["sat_acc"] == r.sat
    # identity keeps the NaN: amax becomes NaN and the next scale falls back to 1
    st2 = sq.TensorState(sq.E5M2, 1, 1.25, 0.5)
    b2, q2, _ = _run(h, sq.ACT_IDENTITY, sq.E5M2, sq.PER_TENSOR, st2)
    r2 = O.quantize(h, O.ACT_IDENTITY, O.E5M2, O.PER_TENSOR, O.State(O.E5M2, 1, 1.25, 0.5).scale)
    assert np.array_equal(u8_np(q2), r2.fp8)
    sq.amax_history_update(st2)
    assert st2.read()["scale"] == 1.0


@pytest.mark.parametrize("rows,cols", [(1, 128), (3, 384), (257, 1024)])
def test_group_mode_ragged_rows(rows, cols, codec):
    h = workloads.student_t(43, rows, cols)
    h[0, :128] = 0                                  # zero group -> scale 1
    st = sq.TensorState(sq.E4M3)
    b, q, g = _run(h, sq.ACT_IDENTITY, sq.E4M3, sq.PER_GROUP128, st, want_bf16=False)
    r = O.quantize(h, O.ACT_IDENTITY, O.E4M3, O.PER_GROUP128, want_bf16=False)
    assert np.array_equal(u8_np(q), r.fp8)
    assert np.array_equal(g.cpu().numpy().view(np.uint32), r.group_scale_inv.view(np.uint32))
    d = st.read()
    assert d["amax_acc"] == r.amax_bits and d["sat_acc"] == r.sat == 0


def test_gpt2_sixteen_delayed_steps_full_size():
    """All 16 steps of the GPT-2 workload (amax drifting by up to 5% a step)
    under delayed scaling: every step's codes in full, the state field by
    field after every update, and the BF16 copy on the first and last steps."""
    w = workloads.get("gpt2")
    h0 = w.h0()
    st = sq.TensorState(sq.E4M3, 1, w.margin, w.initial_amax)
    ost = O.State(O.E4M3, 1, w.margin, w.initial_amax)
    scales = []
    for t in range(w.steps):
        h = w.h_step(t, h0)
        copy = t in (0, w.steps - 1)
        b, q, _ = _run(h, sq.ACT_RELU2, sq.E4M3, sq.PER_TENSOR, st, want_bf16=copy)
        r = oracle_quantize(h, O.ACT_RELU2, O.E4M3, O.PER_TENSOR, ost.scale, want_bf16=copy)
        if copy:
            assert np.array_equal(bf16_np(b), r.bf16), t
        assert np.array_equal(u8_np(q), r.fp8), t
        d = st.read()
        assert d["amax_acc"] == r.amax_bits and d["sat_acc"] == r.sat, t
        sq.amax_history_update(st)
        ost.accumulate(r.amax_bits, r.sat)
        ost.update()
        _compare_state(st, ost)
        scales.append(ost.scale)
    # after the cold start the scale follows the drifting amax: no step saturates
    assert ost.overflow == 0 and len(set(scales[1:])) > 1


@pytest.mark.parametrize("shape,limit", [((1, 8), 0), ((3, 1001), 0), ((64, 256), 1),
                                         ((300, 2048), 3), ((300, 2048), 64), ((300, 2048), 100),
                                         ((1031, 777), 0), ((16384, 3072), 0)])
def test_fused_update_equals_quantize_then_update(shape, limit, codec):
    """quantize_fused_update against quantize_fused followed by
    amax_history_update: codes, BF16 copy and every field of the state equal
    after each of 5 steps (so the tickets are back at zero for the next call),
    for grids of 1, 3, 64, 100 workgroups and unlimited ones (a workgroup
    count below, at and off the 64 accumulator slots, and the looping form),
    with an earlier quantize_fused call of the same step folded in on step 2;
    and the state sequence against the oracle's."""
    h0 = workloads.normal(47 + shape[0], *shape)
    prev = sq.fp8dp_set_grid_limit(limit)
    try:
        st_a = sq.TensorState(sq.E4M3, 4, 1.25, 0.5)
        st_b = sq.TensorState(sq.E4M3, 4, 1.25, 0.5)
        ost = O.State(O.E4M3, 4, 1.25, 0.5)
        for t, f in enumerate((1.0, 3.0, 0.5, 40.0, 1.0)):
            h = h0 if f == 1.0 else workloads.scale_bf16(h0, f)
            hd = to_dev_bf16(h)
            b1, q1 = torch.empty_like(hd), torch.empty(shape, dtype=torch.uint8, device=DEV)
            b2, q2 = torch.empty_like(hd), torch.empty(shape, dtype=torch.uint8, device=DEV)
            if t == 2:                     # an earlier call of the same step
                extra = to_dev_bf16(workloads.scale_bf16(h0, 7.0))
                qx = torch.empty(shape, dtype=torch.uint8, device=DEV)
                for st in (st_a, st_b):
                    sq.quantize_fused(extra, sq.ACT_RELU2, sq.E4M3, sq.PER_TENSOR, st, None, qx)
            sq.quantize_fused(hd, sq.ACT_RELU2, sq.E4M3, sq.PER_TENSOR, st_a, b1, q1)
            sq.amax_history_update(st_a)
            sq.quantize_fused_update(hd, sq.ACT_RELU2, sq.E4M3, st_b, b2, q2)
            assert torch.equal(b1.view(torch.int16), b2.view(torch.int16)), t
            assert torch.equal(q1, q2), t
            da, d = st_a.read(), st_b.read()          # every field (not the padding)
            assert da == d, (t, {k: (da[k], d[k]) for k in d if da[k] != d[k]})
            assert d["ticket"] == 0 and d["slot_tickets"] == 0, t
            r = oracle_quantize(h, O.ACT_RELU2, O.E4M3, O.PER_TENSOR, ost.scale)
            assert np.array_equal(u8_np(q2), r.fp8), t
            amax, sat = r.amax_bits, r.sat
            if t == 2:
                re = oracle_quantize(workloads.scale_bf16(h0, 7.0), O.ACT_RELU2, O.E4M3,
                                     O.PER_TENSOR, ost.scale, want_bf16=False)
                amax, sat = max(amax, re.amax_bits), sat + re.sat
            ost.accumulate(amax, sat)
            ost.update()
            _compare_state(st_b, ost)
    finally:
        sq.fp8dp_set_grid_limit(prev)


def test_fused_update_gradient_cast_identity_e5m2():
    """The gradient form: identity, E5M2, no BF16 copy, ragged length."""
    x = workloads.signed_lognormal(48, 7, 4099)
    st_a = sq.TensorState(sq.E5M2, 1, 1.25, 1.0)
    st_b = sq.TensorState(sq.E5M2, 1, 1.25, 1.0)
    for t in range(3):
        hd = to_dev_bf16(x)
        q1 = torch.empty(x.shape, dtype=torch.uint8, device=DEV)
        q2 = torch.empty_like(q1)
        sq.quantize_fused(hd, sq.ACT_IDENTITY, sq.E5M2, sq.PER_TENSOR, st_a, None, q1)
        sq.amax_history_update(st_a)
        sq.quantize_fused_update(hd, sq.ACT_IDENTITY, sq.E5M2, st_b, None, q2)
        assert torch.equal(q1, q2) and st_a.read() == st_b.read(), t


@pytest.mark.parametrize("hist_len", [2, 4, 16])
def test_history_window_sequence(hist_len):
    """Delayed scaling with a window of hist_len steps ("FP8 training: what it
    is and how it works", Trade-offs: a stored amax history): 40 steps whose
    amax rises, falls and jumps, state compared field by field with the
    oracle after every update."""
    rng = np.random.default_rng(hist_len)
    levels = np.concatenate([np.geomspace(0.5, 300.0, 12), np.geomspace(300.0, 0.01, 12),
                             [5.0, 5000.0, 5.0, 0.0, 7.0], rng.uniform(0.1, 50.0, 11)])
    st = sq.TensorState(sq.E4M3, hist_len, 1.25, 1.0)
    ost = O.State(O.E4M3, hist_len, 1.25, 1.0)
    q = torch.empty((4, 64), dtype=torch.uint8, device=DEV)
    for t, lv in enumerate(levels):
        x = (rng.standard_normal((4, 64)) * lv).astype(np.float32)
        h = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        sq.quantize_fused(to_dev_bf16(h), sq.ACT_IDENTITY, sq.E4M3, sq.PER_TENSOR, st, None, q)
        r = O.quantize(h, O.ACT_IDENTITY, O.E4M3, O.PER_TENSOR, ost.scale, want_bf16=False)
        assert np.array_equal(u8_np(q), r.fp8), t
        sq.amax_history_update(st)
        ost.accumulate(r.amax_bits, r.sat)
        ost.update()
        _compare_state(st, ost)
        assert st.read()["amax_last"] == np.float32(r.amax), t


def test_outlier_stress_65_steps():
    w = workloads.get("outlier")
    st = sq.TensorState(sq.E4M3, 1, w.margin, w.initial_amax)
    ost = O.State(O.E4M3, 1, w.margin, w.initial_amax)
    q = torch.empty((w.M, w.K), dtype=torch.uint8, device=DEV)
    flags, zeroed = [], []
    for k in range(w.steps):
        x = workloads.outlier_tensor(k)
        sq.quantize_fused(to_dev_bf16(x), sq.ACT_IDENTITY, sq.E4M3, sq.PER_TENSOR, st, None, q)
        r = oracle_quantize(x, O.ACT_IDENTITY, O.E4M3, O.PER_TENSOR, ost.scale, want_bf16=False)
        got = u8_np(q)
        assert np.array_equal(got, r.fp8), k
        sq.amax_history_update(st)
        ost.accumulate(r.amax_bits, r.sat)
        ost.update()
        _compare_state(st, ost)
        flags.append(ost.overflow)
        zeroed.append(float(np.mean((got & 0x7F) == 0)))
    # cold start (scale from amax 1.0) saturates; the steady steps do not; the
    # 8x jump at the last step does, and is flagged
    assert flags[0] == 1 and flags[-1] == 1 and not any(flags[1:-1])
    # with one +-1e5 outlier per tensor the delayed scale flushes about a fifth
    # of the N(0,1) values to zero ("FP8 training ...", Step 2 worked example)
    assert all(0.15 < z < 0.30 for z in zeroed[1:-1]), zeroed[1:4]


def test_fine_grained_group_full_size():
    w = workloads.get("fine")
    h = w.h0()
    st = sq.TensorState(sq.E4M3)
    b, q, g = _run(h, sq.ACT_IDENTITY, sq.E4M3, sq.PER_GROUP128, st, want_bf16=False)
    r = oracle_quantize(h, O.ACT_IDENTITY, O.E4M3, O.PER_GROUP128, want_bf16=False)
    assert np.array_equal(u8_np(q), r.fp8)
    assert np.array_equal(g.cpu().numpy().view(np.uint32), r.group_scale_inv.view(np.uint32))
    d = st.read()
    assert d["amax_acc"] == r.amax_bits and d["sat_acc"] == 0 == r.sat


def test_large_forward_and_gradient_casts_full_size():
    """The large workload at full size: the cold-start step (scale 448 / 1.25:
    most vectors saturate and take the integer codec) and the steady step
    with the delayed scale from step 0's amax (nothing saturates: every vector
    takes the hardware-convert path the timed steps run); then two delayed
    steps of the E5M2 gradient cast."""
    w = workloads.get("large")
    h = w.h0()
    st = sq.TensorState(sq.E4M3, 1, w.margin, w.initial_amax)
    ost = O.State(O.E4M3, 1, w.margin, w.initial_amax)
    for t in range(2):
        b, q, _ = _run(h, sq.ACT_RELU2, sq.E4M3, sq.PER_TENSOR, st)
        r = oracle_quantize(h, O.ACT_RELU2, O.E4M3, O.PER_TENSOR, ost.scale)
        assert np.array_equal(bf16_np(b), r.bf16), t
        assert np.array_equal(u8_np(q), r.fp8), t
        d = st.read()
        assert d["amax_acc"] == r.amax_bits and d["sat_acc"] == r.sat, t
        del b, q
        sq.amax_history_update(st)
        ost.accumulate(r.amax_bits, r.sat)
        ost.update()
        _compare_state(st, ost)
        if t == 0:
            assert r.sat > 0             # the cold start saturates
        else:
            assert r.sat == 0            # the steady step does not
        del r
    del h
    dy = w.dy()
    sg = sq.TensorState(sq.E5M2, 1, w.margin, w.initial_amax)
    og = O.State(O.E5M2, 1, w.margin, w.initial_amax)
    for t in range(2):
        _, q8, _ = _run(dy, sq.ACT_IDENTITY, sq.E5M2, sq.PER_TENSOR, sg, want_bf16=False)
        rg = oracle_quantize(dy, O.ACT_IDENTITY, O.E5M2, O.PER_TENSOR, og.scale, want_bf16=False)
        assert np.array_equal(u8_np(q8), rg.fp8), t
        sq.amax_history_update(sg)
        og.accumulate(rg.amax_bits, rg.sat)
        og.update()
        _compare_state(sg, og)


def test_results_do_not_depend_on_grid_size():
    h = workloads.normal(44, 1031, 777)
    outs = []
    for limit in (0, 1, 3, 64, 1000):
        prev = sq.fp8dp_set_grid_limit(limit)
        try:
            st = sq.TensorState(sq.E4M3, 1, 1.25, 0.25)
            b, q, _ = _run(h, sq.ACT_RELU2, sq.E4M3, sq.PER_TENSOR, st)
            d = st.read()
            outs.append((bf16_np(b).tobytes(), u8_np(q).tobytes(), d["amax_acc"], d["sat_acc"]))
        finally:
            sq.fp8dp_set_grid_limit(prev)
    assert all(o == outs[0] for o in outs)
    assert outs[0][3] > 0


@pytest.mark.parametrize("mode", ["group", "mx"])
def test_group_and_mx_results_do_not_depend_on_grid_size(mode):
    """With no grid limit each thread takes one vector (no loop); with small
    limits the grid-stride loops run: the outputs are the same bytes, and the
    oracle's."""
    h = workloads.normal(46, 333, 768)
    outs = []
    for limit in (0, 1, 3, 64, 1000):
        prev = sq.fp8dp_set_grid_limit(limit)
        try:
            if mode == "group":
                st = sq.TensorState(sq.E4M3, 1, 1.25, 0.25)
                b, q, g = _run(h, sq.ACT_RELU2, sq.E4M3, sq.PER_GROUP128, st)
                d = st.read()
                outs.append((bf16_np(b).tobytes(), u8_np(q).tobytes(),
                             g.cpu().numpy().tobytes(), d["amax_acc"], d["sat_acc"]))
            else:
                hd = to_dev_bf16(h)
                b = torch.empty_like(hd)
                q = torch.empty(h.shape, dtype=torch.uint8, device=DEV)
                e = torch.empty((h.shape[0], h.shape[1] // 32), dtype=torch.uint8, device=DEV)
                sq.quantize_mx(hd, sq.ACT_RELU2, sq.E4M3, q, e, b)
                outs.append((bf16_np(b).tobytes(), u8_np(q).tobytes(), u8_np(e).tobytes()))
        finally:
            sq.fp8dp_set_grid_limit(prev)
    assert all(o == outs[0] for o in outs)
    if mode == "group":
        r = oracle_quantize(h, O.ACT_RELU2, O.E4M3, O.PER_GROUP128)
        assert outs[0][1] == r.fp8.tobytes() and outs[0][0] == r.bf16.tobytes()
    else:
        r = O.quantize_mx(h, O.ACT_RELU2, O.E4M3)
        assert outs[0][1] == r.fp8.tobytes() and outs[0][2] == r.scale.tobytes()


def test_two_calls_accumulate_into_one_step():
    h = workloads.normal(45, 512, 256)
    st = sq.TensorState(sq.E4M3, 1, 1.25, 1.0)
    _run(h[:200], sq.ACT_RELU2, sq.E4M3, sq.PER_TENSOR, st)
    _run(h[200:], sq.ACT_RELU2, sq.E4M3, sq.PER_TENSOR, st)
    r = O.quantize(h, O.ACT_RELU2, O.E4M3, O.PER_TENSOR, O.State(O.E4M3, 1, 1.25, 1.0).scale)
    d = st.read()
    assert d["amax_acc"] == r.amax_bits and d["sat_acc"] == r.sat


def test_naive_three_pass_matches_fused_and_oracle(codec):
    w = workloads.get("gpt2")
    h = w.h0(0, 2048)
    hd = to_dev_bf16(h)
    n = h.size
    a16 = torch.empty_like(hd)
    a8 = torch.empty(h.shape, dtype=torch.uint8, device=DEV)
    st = sq.TensorState(sq.E4M3, 1, 1.0, 1.0)       # current scaling: margin 1, one step
    sq.fp8dp_bench_act_bf16(hd, sq.ACT_RELU2, a16)
    sq.fp8dp_bench_amax(a16, st)
    sq.amax_history_update(st)
    sq.fp8dp_bench_cast(a16, sq.E4M3, st, a8)
    d = st.read()
    # oracle: activation copy, its amax, the current scale, the cast
    r0 = oracle_quantize(h, O.ACT_RELU2, O.E4M3, O.PER_TENSOR, 1.0)
    s, _ = O.scale_from_amax(r0.amax, 1.0, O.E4M3)
    r = oracle_quantize(h, O.ACT_RELU2, O.E4M3, O.PER_TENSOR, float(s[0]))
    assert np.array_equal(bf16_np(a16), r.bf16)
    assert d["scale"] == s[0]
    assert np.array_equal(u8_np(a8), r.fp8)
    assert d["sat_acc"] == r.sat == 0
    # the fused kernel with the same multiplier writes the same bytes
    st2 = sq.TensorState(sq.E4M3, 1, 1.0, 1.0)
    st2.buf[0:4] = torch.tensor([float(s[0])], dtype=torch.float32).view(torch.uint8).to(DEV)
    b2 = torch.empty_like(hd)
    q2 = torch.empty_like(a8)
    sq.quantize_fused(hd, sq.ACT_RELU2, sq.E4M3, sq.PER_TENSOR, st2, b2, q2)
    assert torch.equal(b2.view(torch.int16), a16.view(torch.int16)) and torch.equal(q2, a8)
    assert n == a16.numel()


def test_state_copy_out_and_back_resumes_exactly():
    w = workloads.get("tiny")
    h0 = w.h0()
    st = sq.TensorState(sq.E4M3, 3, 1.25, 1.0)
    for t in range(2):
        _run(w.h_step(t, h0), sq.ACT_RELU2, sq.E4M3, sq.PER_TENSOR, st)
        sq.amax_history_update(st)
    saved = st.buf.clone()
    _run(w.h_step(2, h0), sq.ACT_RELU2, sq.E4M3, sq.PER_TENSOR, st)
    sq.amax_history_update(st)
    after = st.raw()
    st.buf.copy_(saved)
    _run(w.h_step(2, h0), sq.ACT_RELU2, sq.E4M3, sq.PER_TENSOR, st)
    sq.amax_history_update(st)
    assert st.raw() == after


@pytest.mark.parametrize("fmt", [0, 1], ids=["e4m3", "e5m2"])
def test_weight_cast_per_tensor_and_blocks(fmt, codec):
    for name in ("tiny", "gpt2", "fine"):
        w = workloads.get(name)
        wn = w.weight()
        wd = to_dev_bf16(wn)
        w8 = torch.empty(wn.shape, dtype=torch.uint8, device=DEV)
        sc = torch.empty(2, dtype=torch.float32, device=DEV)
        sq.quantize_weight(wd, fmt, sq.PER_TENSOR, w8, sc)
        q, s, si = O.quantize_weight_tensor(wn, fmt)
        assert np.array_equal(u8_np(w8), q), name
        assert sc.cpu().tolist() == [si, s], name
        bs = torch.empty((w.N // 128, w.K // 128), dtype=torch.float32, device=DEV)
        sq.quantize_weight(wd, fmt, sq.PER_GROUP128, w8, bs)
        qb, sib = O.quantize_weight_blocks(wn, fmt)
        assert np.array_equal(u8_np(w8), qb), name
        assert np.array_equal(bs.cpu().numpy().view(np.uint32), sib.view(np.uint32)), name


@pytest.mark.parametrize("case", ["zeros", "negative_relu2", "max_bf16", "zero_groups"])
def test_degenerate_inputs(case, codec):
    """The method's degenerate cases against the oracle, bytes and state:
    an all-zero tensor and a squared ReLU of only negative values (amax 0:
    the next scale takes the rule's fallback), every element at the largest
    finite BF16 (every code saturates and is counted), and per-128 groups
    that are all zero or hold a single nonzero value."""
    rows, cols = 64, 512
    act, fmt, mode = sq.ACT_RELU2, sq.E4M3, sq.PER_TENSOR
    if case == "zeros":
        h = np.zeros((rows, cols), dtype=np.uint16)
        act, fmt = sq.ACT_IDENTITY, sq.E5M2
    elif case == "negative_relu2":
        h = workloads.normal(43, rows, cols) | np.uint16(0x8000)     # every value <= -0
    elif case == "max_bf16":
        h = np.full((rows, cols), 0x7F7F, dtype=np.uint16)
        h[::2] |= np.uint16(0x8000)
        act = sq.ACT_IDENTITY
    else:
        h = workloads.normal(44, rows, cols)
        h[:, 0:128] = 0
        h[:, 128:256] = 0
        h[:, 130] = 0x4040                                           # one value: 3.0
        mode = sq.PER_GROUP128
    st = sq.TensorState(fmt, 1, 1.25, 3.0)
    ost = O.State(fmt, 1, 1.25, 3.0)
    b, q, g = _run(h, act, fmt, mode, st if mode == sq.PER_TENSOR else None)
    r = O.quantize(h, act, fmt, mode, ost.scale if mode == sq.PER_TENSOR else 1.0)
    assert np.array_equal(bf16_np(b), r.bf16)
    assert np.array_equal(u8_np(q), r.fp8)
    if mode == sq.PER_GROUP128:
        assert np.array_equal(g.cpu().numpy().view(np.uint32), r.group_scale_inv.view(np.uint32))
        return
    if case == "max_bf16":
        assert r.sat == rows * cols
    else:
        assert r.amax_bits == 0 and not np.any(r.fp8 & 0x7F)
    sq.amax_history_update(st)
    ost.accumulate(r.amax_bits, r.sat)
    ost.update()
    _compare_state(st, ost)
