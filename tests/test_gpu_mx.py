"""MXFP8 cast and MXFP8 GEMM against the oracle (GPU).

"FP8 training: what it is and how it works", Trade-offs and edge cases: the
microscaling recipe gives each block of 32 adjacent values its own
power-of-two scale.  quantize_mx is compared bit for bit with oracle
quantize_mx (BF16 copy, codes, E8M0 block exponents); fp8_gemm_mx with the
oracle's float64 MX GEMM to |y - ref| <= 2^-8 |ref| + 1e-5 sum|a b| on every
element in exact mode (the default), both where a tile's block exponents fold
into the BF16 widening (rows spanning at most 90 binades, E4M3, or 78, E5M2)
and where a tile takes the per-block fallback (wider spans; tiles of both
kinds in one launch).  The microscaled FP8 instructions' mode is held to the
same bound and reported as an expected failure where their truncation takes
elements outside it.  Workloads: the seeded synthetic tensors of workloads.py
(the GPT-2 MLP activation and down-projection weight at full size), block
magnitudes spread over many binades, and special blocks (zero, signed zero,
subnormal, infinity, NaN).
"""
import numpy as np
import pytest
import torch

import oracle as O
import scaled_quantization_amd as sq
import workloads
from gpu_util import (DEV, THREADS, bf16_np, check_gemm, fp8_mfma_allowance_mx, to_dev_bf16, to_dev_u8,
                      u8_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(params=[0, 1], ids=["hw", "int"])
def codec(request):
    prev = sq.fp8dp_set_codec(request.param)
    yield request.param
    sq.fp8dp_set_codec(prev)


def _spread(rng, rows, cols, lo=-30, hi=30):
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(rng.integers(lo, hi, (rows, cols // 32, 1)).astype(np.float32)).repeat(
        32, axis=2).reshape(rows, cols)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _run_mx(h_np, act, fmt, want_bf16=True):
    rows, cols = h_np.shape
    h = to_dev_bf16(h_np)
    b = torch.empty_like(h) if want_bf16 else None
    q = torch.empty((rows, cols), dtype=torch.uint8, device=DEV)
    e = torch.empty((rows, cols // 32), dtype=torch.uint8, device=DEV)
    sq.quantize_mx(h, act, fmt, q, e, b)
    return b, q, e


def _oracle_mx(h, act, fmt, want_bf16=True):
    """oracle quantize_mx over row ranges in parallel (rows are independent)."""
    from concurrent.futures import ThreadPoolExecutor
    rows = h.shape[0]
    if rows < 64:
        return O.quantize_mx(h, act, fmt, want_bf16)
    step = (rows + 4 * THREADS - 1) // (4 * THREADS)
    with ThreadPoolExecutor(THREADS) as ex:
        parts = list(ex.map(lambda r0: O.quantize_mx(h[r0:r0 + step], act, fmt, want_bf16),
                            range(0, rows, step)))
    return O.MXResult(np.concatenate([p.bf16 for p in parts]) if want_bf16 else None,
                      np.concatenate([p.fp8 for p in parts]),
                      np.concatenate([p.scale for p in parts]))


# ------------------------------------------------------------------ cast
@pytest.mark.parametrize("fmt", [0, 1], ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("act", [0, 1], ids=["identity", "relu2"])
@pytest.mark.parametrize("rows,cols", [(1, 32), (3, 96), (17, 4128), (257, 768)])
def test_quantize_mx_vs_oracle(rows, cols, act, fmt, codec):
    rng = np.random.default_rng(rows * 7 + cols + act + 2 * fmt)
    h = _spread(rng, rows, cols)
    b, q, e = _run_mx(h, act, fmt)
    r = O.quantize_mx(h, act, fmt)
    assert np.array_equal(bf16_np(b), r.bf16)
    assert np.array_equal(u8_np(e), r.scale)
    assert np.array_equal(u8_np(q), r.fp8)


def test_quantize_mx_without_copy():
    rng = np.random.default_rng(3)
    h = _spread(rng, 64, 512)
    _, q, e = _run_mx(h, sq.ACT_RELU2, sq.E4M3, want_bf16=False)
    r = O.quantize_mx(h, O.ACT_RELU2, O.E4M3, want_bf16=False)
    assert np.array_equal(u8_np(q), r.fp8) and np.array_equal(u8_np(e), r.scale)


@pytest.mark.parametrize("fmt", [0, 1], ids=["e4m3", "e5m2"])
def test_quantize_mx_special_blocks(fmt, codec):
    rng = np.random.default_rng(9)
    h = _spread(rng, 4, 256)
    h[0, 0:32] = 0                        # zero block
    h[0, 32:64] = 0x8000                  # negative zeros
    h[0, 64:96] = rng.integers(1, 0x80, 32)   # BF16 subnormals only
    h[1, 0] = 0x7F80                      # +inf with finite neighbours
    h[1, 33] = 0xFF80                     # -inf
    h[1, 64] = 0x7FC1                     # NaN
    h[1, 97] = 0xFFC0                     # -NaN
    h[2, 128:160] = 0x7F7F                # largest finite BF16 everywhere
    h[3, 5] = 0x0001                      # smallest subnormal among normal values
    for act in (0, 1):
        b, q, e = _run_mx(h, act, fmt)
        r = O.quantize_mx(h, act, fmt)
        assert np.array_equal(bf16_np(b), r.bf16)
        assert np.array_equal(u8_np(e), r.scale)
        assert np.array_equal(u8_np(q), r.fp8)


def test_quantize_mx_every_exponent_boundary():
    """Block maxima at and around max * 2^k for every k the BF16 range reaches."""
    rows = []
    for fmt in (0, 1):
        for k in range(-133, 121):
            for frac in (0x5F, 0x60, 0x61, 0x7F, 0x00):
                ef = k + 127 + (8 if fmt == 0 else 15)
                if 1 <= ef <= 254:
                    blk = np.full(32, 0x3F80, np.uint16)
                    blk[7] = (ef << 7) | frac
                    rows.append(blk)
    h = np.stack(rows)
    for fmt in (0, 1):
        _, q, e = _run_mx(h, 0, fmt, want_bf16=False)
        r = O.quantize_mx(h, 0, fmt, want_bf16=False)
        assert np.array_equal(u8_np(e), r.scale)
        assert np.array_equal(u8_np(q), r.fp8)


def test_quantize_mx_gpt2_activation_full_size():
    w = workloads.get("gpt2")
    h = w.h0()
    b, q, e = _run_mx(h, sq.ACT_RELU2, sq.E4M3)
    r = _oracle_mx(h, O.ACT_RELU2, O.E4M3)
    assert np.array_equal(u8_np(e), r.scale)
    assert np.array_equal(u8_np(q), r.fp8)
    assert np.array_equal(bf16_np(b), r.bf16)


def test_quantize_mx_errors():
    h = torch.zeros((4, 48), dtype=torch.bfloat16, device=DEV)
    q = torch.empty((4, 48), dtype=torch.uint8, device=DEV)
    e = torch.empty((4, 2), dtype=torch.uint8, device=DEV)
    # cols not a multiple of 32
    assert sq.lib().quantize_mx(h.data_ptr(), 4, 48, 0, 0, None, q.data_ptr(), e.data_ptr(),
                                None) == -1
    # missing exponent output, unknown format
    assert sq.lib().quantize_mx(h.data_ptr(), 4, 32, 0, 0, None, q.data_ptr(), None, None) == -1
    assert sq.lib().quantize_mx(h.data_ptr(), 4, 32, 0, 7, None, q.data_ptr(), e.data_ptr(),
                                None) == -1
    torch.cuda.synchronize()


# ------------------------------------------------------------------ GEMM
EXACT, FP8 = sq.ACCUM_EXACT, sq.ACCUM_MFMA_FP8
BOTH = pytest.mark.parametrize("accum", [EXACT, FP8], ids=["exact", "fp8"])


def _check(y, ref, absref, allowance, what, accum):
    """The plain bound on every element.  Exact mode must meet it everywhere;
    in FP8 mode, elements the microscaled instruction's truncation takes
    outside it make the case an expected failure (after the allowance
    accounts for each of them)."""
    check_gemm(y, ref, absref, what, accum == EXACT, allowance)


def _gemm_case(rng, M, N, K, fa, fb, lo=-12, hi=12):
    ha = _spread(rng, M, K, lo, hi)
    hb = _spread(rng, N, K, lo, hi)
    ra = O.quantize_mx(ha, O.ACT_IDENTITY, fa, want_bf16=False)
    rb = O.quantize_mx(hb, O.ACT_IDENTITY, fb, want_bf16=False)
    return ra.fp8, ra.scale, rb.fp8, rb.scale


def _gemm_mx_dev(a8, fa, ea, b8, fb, eb, accum):
    M, N = a8.shape[0], b8.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    sq.fp8_gemm_mx(to_dev_u8(a8), fa, to_dev_u8(ea), to_dev_u8(b8), fb, to_dev_u8(eb), y, accum)
    return y.float().cpu().numpy()


def _span(e):
    """Largest per-row spread (max - min) of block exponent bytes."""
    e = e.astype(np.int32)
    return int((e.max(axis=1) - e.min(axis=1)).max())


# block exponent spreads: lo..hi binades of the inputs; rows of +-12 or less
# fold everywhere, rows of +-55 span more than 90 (E4M3) or 78 (E5M2) binades
# in some tiles, which take the per-block fallback
@BOTH
@pytest.mark.parametrize("M,N,K,fa,fb,spread", [(256, 128, 128, 0, 0, 12), (256, 384, 1024, 0, 0, 12),
                                                (512, 512, 512, 1, 0, 12), (256, 640, 256, 0, 1, 12),
                                                (768, 768, 3072, 0, 0, 12), (256, 256, 384, 1, 1, 12),
                                                (512, 384, 1024, 0, 0, 9), (256, 256, 1024, 1, 1, 3),
                                                (256, 384, 512, 0, 1, 3), (256, 384, 1024, 0, 0, 55),
                                                (512, 256, 512, 1, 0, 55), (256, 256, 384, 1, 1, 55)])
def test_gemm_mx_vs_oracle(M, N, K, fa, fb, spread, accum):
    rng = np.random.default_rng(M + 3 * N + 7 * K + fa + 2 * fb + spread)
    a8, ea, b8, eb = _gemm_case(rng, M, N, K, fa, fb, -spread, spread)
    y = _gemm_mx_dev(a8, fa, ea, b8, fb, eb, accum)
    rows = np.unique(np.concatenate([np.arange(0, M, max(1, M // 24)), [M - 1]]))
    ref, absref = O.gemm_mx_f64(a8, fa, ea, b8, fb, eb, rows)
    _check(y[rows], ref, absref,
           lambda sel: fp8_mfma_allowance_mx(a8, fa, ea, b8, fb, eb, rows[sel]),
           f"{M}x{N}x{K} spread {spread}", accum)


@pytest.mark.parametrize("N", [256, 384])
@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 1), (0, 1)])
def test_gemm_mx_exact_fold_and_fallback_tiles_in_one_launch(fa, fb, N):
    """Rows 0-255 (the first row tile) and columns 0-191 keep their blocks
    within the fold span; one A row of the second row tile and one B row of
    the second column tile (256 x 128 tiles at N = 256, 256 x 192 at N = 384)
    spread over 110 binades, so three of the four tiles take the per-block
    fallback and one folds.  Every output meets the plain bound."""
    M, K = 512, 1024
    rng = np.random.default_rng(31 + fa + 2 * fb + N)
    narrow = {0: 9, 1: 3}
    ha = _spread(rng, M, K, -narrow[fa], narrow[fa])
    hb = _spread(rng, N, K, -narrow[fb], narrow[fb])
    # the wide rows: blocks alternately near 2^-55 and 2^55 (a span of ~110)
    wide = np.exp2(np.where(np.arange(K // 32) % 2 == 0, -55.0, 55.0)).repeat(32).astype(np.float32)
    for h, r in ((ha, 300), (hb, 200)):
        x = rng.standard_normal(K).astype(np.float32) * wide
        h[r] = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ra = O.quantize_mx(ha, O.ACT_IDENTITY, fa, want_bf16=False)
    rb = O.quantize_mx(hb, O.ACT_IDENTITY, fb, want_bf16=False)
    span_a, span_b = {0: 90, 1: 78}[fa], {0: 90, 1: 78}[fb]
    assert _span(ra.scale[:256]) <= span_a and _span(rb.scale[:192]) <= span_b
    assert _span(ra.scale[300:301]) > span_a and _span(rb.scale[200:201]) > span_b
    y = _gemm_mx_dev(ra.fp8, fa, ra.scale, rb.fp8, fb, rb.scale, EXACT)
    rows = np.unique(np.concatenate([np.arange(0, M, 8), [255, 256, 300, M - 1]]))
    ref, absref = O.gemm_mx_f64(ra.fp8, fa, ra.scale, rb.fp8, fb, rb.scale, rows)
    check_gemm(y[rows], ref, absref, f"mixed tiles {fa}{fb} N={N}")


@pytest.mark.parametrize("a_lo", [-40, -100])
def test_gemm_mx_exact_full_range_codes(a_lo):
    """Every finite code equally likely; block exponents over -40 .. 40
    binades (A's rows span under 90 and fold, B's up to 80 and some take the
    per-block fallback), then A's over -100 .. 0 (every A row past 90: the
    fallback everywhere), results within BF16's range: every element meets
    the bound."""
    rng = np.random.default_rng(77 - a_lo)
    M, N, K = 256, 256, 2048
    ta = np.flatnonzero(np.isfinite(O.fp8_decode_table(O.E4M3)))
    tb = np.flatnonzero(np.isfinite(O.fp8_decode_table(O.E5M2)))
    a8 = rng.choice(ta, size=(M, K)).astype(np.uint8)
    b8 = rng.choice(tb, size=(N, K)).astype(np.uint8)
    ea = rng.integers(127 + a_lo, 127 + (40 if a_lo == -40 else 0), (M, K // 32)).astype(np.uint8)
    eb = rng.integers(127 - 40, 127 + 40, (N, K // 32)).astype(np.uint8)
    y = _gemm_mx_dev(a8, O.E4M3, ea, b8, O.E5M2, eb, EXACT)
    ref, absref = O.gemm_mx_f64(a8, O.E4M3, ea, b8, O.E5M2, eb)
    check_gemm(y, ref, absref, "full range")


@BOTH
@pytest.mark.parametrize("M,N,K", [(512, 384, 1536), (256, 256, 512)])
def test_gemm_mx_exponent_copy_paths_agree(M, N, K, accum):
    """With K a multiple of 512 and 16-byte aligned exponent arrays the kernel
    copies four stages' exponents per row at once; exponent arrays 4 bytes off
    that alignment take the per-stage copies.  Both read the same bytes, so the
    outputs are equal bit for bit, and both match the oracle."""
    rng = np.random.default_rng(K + N)
    a8, ea, b8, eb = _gemm_case(rng, M, N, K, 0, 0, -9, 9)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    sq.fp8_gemm_mx(to_dev_u8(a8), 0, to_dev_u8(ea), to_dev_u8(b8), 0, to_dev_u8(eb), y, accum)

    def off4(x):
        buf = torch.zeros(x.size + 16, dtype=torch.uint8, device=DEV)
        v = buf[4:4 + x.size].view(x.shape)
        v.copy_(torch.from_numpy(np.ascontiguousarray(x)).to(DEV))
        assert v.data_ptr() % 16 == 4
        return v

    y2 = torch.empty_like(y)
    sq.fp8_gemm_mx(to_dev_u8(a8), 0, off4(ea), to_dev_u8(b8), 0, off4(eb), y2, accum)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    rows = np.unique(np.concatenate([np.arange(0, M, 16), [M - 1]]))
    ref, absref = O.gemm_mx_f64(a8, 0, ea, b8, 0, eb, rows)
    _check(y.float().cpu().numpy()[rows], ref, absref,
           lambda sel: fp8_mfma_allowance_mx(a8, 0, ea, b8, 0, eb, rows[sel]), f"{M}x{N}x{K}",
           accum)


@BOTH
def test_gemm_mx_neutral_exponents_equal_per_tensor_gemm(accum):
    """Exponent bytes 127 + i (A) and 127 + j (B) everywhere equal per-tensor
    scales 2^i, 2^j: the MX GEMM then matches fp8_gemm_scaled in the same
    accumulation mode bit for bit (the fold scales every product by one power
    of two, which the epilogue takes back exactly)."""
    rng = np.random.default_rng(5)
    M, N, K = 512, 768, 1024
    t = O.fp8_decode_table(0)
    ok = np.flatnonzero(np.isfinite(t) & (np.abs(t) <= 16))
    a8 = rng.choice(ok, size=(M, K)).astype(np.uint8)
    b8 = rng.choice(ok, size=(N, K)).astype(np.uint8)
    for i, j in ((0, 0), (3, -5)):
        ea = np.full((M, K // 32), 127 + i, np.uint8)
        eb = np.full((N, K // 32), 127 + j, np.uint8)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        sq.fp8_gemm_mx(to_dev_u8(a8), 0, to_dev_u8(ea), to_dev_u8(b8), 0, to_dev_u8(eb), y, accum)
        y2 = torch.empty_like(y)
        sa = torch.tensor([2.0 ** i], dtype=torch.float32, device=DEV)
        sb = torch.tensor([2.0 ** j], dtype=torch.float32, device=DEV)
        sq.fp8_gemm_scaled(to_dev_u8(a8), 0, to_dev_u8(b8), 0, sq.PER_TENSOR, sa, sb, y2, accum)
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), (i, j)


@BOTH
def test_gemm_mx_gpt2_down_projection(accum):
    """The GPT-2 down-projection in MXFP8: H = relu2(H0) and W cast by
    quantize_mx on the GPU, checked byte for byte against the oracle's cast,
    then the GEMM on sampled rows against the oracle."""
    w = workloads.get("gpt2")
    h = w.h0()
    wt = w.weight()                          # [768, 3072]
    _, qa, ea = _run_mx(h, sq.ACT_RELU2, sq.E4M3, want_bf16=False)
    _, qb, eb = _run_mx(wt, sq.ACT_IDENTITY, sq.E4M3, want_bf16=False)
    rng = np.random.default_rng(17)
    rows = np.sort(rng.choice(h.shape[0], size=64, replace=False))
    ra = O.quantize_mx(h[rows], O.ACT_RELU2, O.E4M3, want_bf16=False)
    rb = O.quantize_mx(wt, O.ACT_IDENTITY, O.E4M3, want_bf16=False)
    assert np.array_equal(u8_np(qa)[rows], ra.fp8) and np.array_equal(u8_np(ea)[rows], ra.scale)
    assert np.array_equal(u8_np(qb), rb.fp8) and np.array_equal(u8_np(eb), rb.scale)
    M, N = h.shape[0], wt.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    sq.fp8_gemm_mx(qa, sq.E4M3, ea, qb, sq.E4M3, eb, y, accum)
    ref, absref = O.gemm_mx_f64(ra.fp8, O.E4M3, ra.scale, rb.fp8, O.E4M3, rb.scale)
    _check(y.float().cpu().numpy()[rows], ref, absref,
           lambda sel: fp8_mfma_allowance_mx(ra.fp8, 0, ra.scale, rb.fp8, 0, rb.scale, sel),
           "gpt2 mx", accum)


def test_gemm_mx_errors():
    a = torch.zeros((256, 128), dtype=torch.uint8, device=DEV)
    e = torch.zeros((256, 4), dtype=torch.uint8, device=DEV)
    y = torch.empty((256, 256), dtype=torch.bfloat16, device=DEV)
    b = torch.zeros((256, 128), dtype=torch.uint8, device=DEV)
    rc = sq.lib().fp8_gemm_mx(a.data_ptr(), 0, e.data_ptr(), b.data_ptr(), 0, e.data_ptr(),
                              128, 256, 128, EXACT, y.data_ptr(), None)
    assert rc == -1
    rc = sq.lib().fp8_gemm_mx(a.data_ptr(), 0, e.data_ptr(), b.data_ptr(), 0, e.data_ptr() + 1,
                              256, 256, 128, EXACT, y.data_ptr(), None)
    assert rc == -1
    rc = sq.lib().fp8_gemm_mx(a.data_ptr(), 0, e.data_ptr(), b.data_ptr(), 0, e.data_ptr(),
                              256, 256, 128, 7, y.data_ptr(), None)
    assert rc == -1 and b"accumulation" in sq.lib().fp8dp_last_error()
