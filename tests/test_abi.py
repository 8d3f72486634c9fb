"""The C-ABI library loads and exports every symbol include/fp8dp.h declares;
argument checks reject bad calls before anything is enqueued (CPU only: no
call here reaches a GPU)."""
import ctypes
import os
import re

import pytest

import scaled_quantization_amd as sq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8dp.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\*?\s+\*?([A-Za-z_]\w*)\s*\(",
                       text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(sq.LIB_PATH):
        pytest.skip("libfp8dp.so not built")
    return sq.lib()


def test_header_declares_the_named_entry_points():
    names = declared_functions()
    for n in ("quantize_fused", "amax_history_update", "fp8_gemm_scaled", "fp8dp_state_init",
              "quantize_weight", "gemm_bf16_quantize_fused", "fp8_gemm_scaled_splitk",
              "fp8_gemm_scaled_splitk_noalloc", "fp8_transpose", "quantize_fused_transposed", "quantize_mx", "fp8_gemm_mx", "quantize_recompute",
              "fp8_gemm_scaled_if", "relu2_backward_quantize", "fp8_gemm_relu2_backward",
              "fp8dp_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing


def test_state_layout_matches_binding(L):
    assert L.fp8dp_state_size() == sq.STATE_BYTES == 192 + 64 * sq.ACC_SLOTS


def test_argument_checks_reject_without_launching(L):
    # every call below fails its host-side checks, so nothing reaches HIP
    rc = L.quantize_fused(None, 4, 8, 0, 0, 0, None, None, None, None, None)
    assert rc == -1 and b"non-NULL" in L.fp8dp_last_error()
    rc = L.quantize_fused(16, 4, 8, 0, 0, 0, None, None, None, None, None)
    assert rc == -1 and b"scaling state" in L.fp8dp_last_error()
    rc = L.quantize_fused(16, 4, 100, 0, 0, 1, None, None, 32, None, None)
    assert rc == -1 and b"128" in L.fp8dp_last_error()
    rc = L.quantize_fused(18, 4, 8, 0, 0, 0, 16, None, None, None, None)
    assert rc == -1 and b"aligned" in L.fp8dp_last_error()
    rc = L.quantize_fused(16, 4, 8, 7, 0, 0, 16, None, None, None, None)
    assert rc == -1
    # empty inputs are refused, not launched
    for rows, cols in ((0, 8), (4, 0), (-1, 8)):
        rc = L.quantize_fused(16, rows, cols, 0, 0, 0, 16, None, 16, None, None)
        assert rc == -1 and b"rows" in L.fp8dp_last_error()
    rc = L.quantize_fused_update(16, 0, 8, 0, 0, 16, None, 16, None)
    assert rc == -1
    rc = L.fp8_gemm_scaled(16, 0, 16, 0, 128, 128, 100, 0, 0, 16, 16, 16, None)
    assert rc == -1 and b"multiples of 128" in L.fp8dp_last_error()
    rc = L.fp8_gemm_scaled(16, 0, 16, 0, 0, 128, 128, 0, 0, 16, 16, 16, None)
    assert rc == -1 and b"M must be positive" in L.fp8dp_last_error()
    rc = L.fp8_gemm_scaled(16, 0, 16, 3, 128, 128, 128, 0, 0, 16, 16, 16, None)
    assert rc == -1 and b"format" in L.fp8dp_last_error()
    rc = L.fp8_gemm_scaled(None, 0, 16, 0, 128, 128, 128, 0, 0, 16, 16, 16, None)
    assert rc == -1
    rc = L.fp8_gemm_scaled(16, 0, 16, 0, 128, 128, 128, 0, 5, 16, 16, 16, None)
    assert rc == -1 and b"accumulation" in L.fp8dp_last_error()
    rc = L.fp8dp_state_init(16, 0, 0, 1.25, 1.0, None)
    assert rc == -1 and b"hist_len" in L.fp8dp_last_error()
    rc = L.fp8dp_state_init(16, 0, 1, -1.0, 1.0, None)
    assert rc == -1 and b"margin" in L.fp8dp_last_error()
    rc = L.fp8dp_state_init(16, 2, 1, 1.0, 1.0, None)
    assert rc == -1
    rc = L.amax_history_update(None, None)
    assert rc == -1
    rc = L.quantize_weight(16, 100, 128, 0, 1, 16, 16, None)
    assert rc == -1 and b"128" in L.fp8dp_last_error()
    rc = L.fp8dp_convert_f32(16, 12, 0, 16, None)
    assert rc == -1
    rc = L.fp8dp_bench_copy(16, 16, 24, None)
    assert rc == -1
    # gemm_bf16_quantize_fused(x, w, M, N, K, act, fmt, st, h_out, bf16_out, fp8_out, stream)
    rc = L.gemm_bf16_quantize_fused(None, 16, 256, 128, 64, 1, 0, None, 16, None, None, None)
    assert rc == -1 and b"non-NULL" in L.fp8dp_last_error()
    rc = L.gemm_bf16_quantize_fused(16, 16, 128, 128, 64, 1, 0, None, 16, None, None, None)
    assert rc == -1 and b"256" in L.fp8dp_last_error()
    rc = L.gemm_bf16_quantize_fused(16, 16, 256, 128, 96, 1, 0, None, 16, None, None, None)
    assert rc == -1 and b"64" in L.fp8dp_last_error()
    rc = L.gemm_bf16_quantize_fused(16, 16, 256, 128, 64, 1, 0, None, None, None, None, None)
    assert rc == -1 and b"h_out" in L.fp8dp_last_error()
    rc = L.gemm_bf16_quantize_fused(16, 16, 256, 128, 64, 1, 0, None, None, None, 16, None)
    assert rc == -1 and b"state" in L.fp8dp_last_error()
    rc = L.gemm_bf16_quantize_fused(16, 16, 256, 128, 64, 5, 0, 16, None, None, 16, None)
    assert rc == -1 and b"activation" in L.fp8dp_last_error()
    rc = L.gemm_bf16_quantize_fused(16, 24, 256, 128, 64, 1, 0, 16, None, None, 16, None)
    assert rc == -1 and b"aligned" in L.fp8dp_last_error()
    # fp8_gemm_scaled_splitk(a, fa, b, fb, M, N, K, splits, accum, sa, sb, ws, y, stream)
    rc = L.fp8_gemm_scaled_splitk(16, 0, 16, 1, 256, 128, 512, 0, 1, 16, 16, 16, 16, None)
    assert rc == -1 and b"splits" in L.fp8dp_last_error()
    rc = L.fp8_gemm_scaled_splitk(16, 0, 16, 1, 256, 128, 128, 2, 1, 16, 16, 16, 16, None)
    assert rc == -1 and b"128 * splits" in L.fp8dp_last_error()
    rc = L.fp8_gemm_scaled_splitk(16, 0, 16, 1, 256, 128, 200, 1, 1, 16, 16, 16, 16, None)
    assert rc == -1 and b"of 128" in L.fp8dp_last_error()
    rc = L.fp8_gemm_scaled_splitk(16, 0, 16, 1, 256, 128, 512, 2, 1, 16, 16, None, 16, None)
    assert rc == -1 and b"NULL" in L.fp8dp_last_error()
    rc = L.fp8_gemm_scaled_splitk(16, 0, 16, 1, 256, 128, 512, 2, 1, 16, 16, 24, 16, None)
    assert rc == -1 and b"aligned" in L.fp8dp_last_error()
    rc = L.fp8_gemm_scaled_splitk(16, 0, 16, 1, 256, 128, 512, 2, 7, 16, 16, 16, 16, None)
    assert rc == -1 and b"accumulation" in L.fp8dp_last_error()
    # fp8_gemm_scaled_splitk_noalloc(a, fa, b, fb, M, N, K, splits, accum, sa, sb, y, stream):
    # the split-K checks, then the scratch limit (16 Mi floats), all before any HIP call
    rc = L.fp8_gemm_scaled_splitk_noalloc(16, 0, 16, 1, 256, 128, 512, 0, 1, 16, 16, 16, None)
    assert rc == -1 and b"splits" in L.fp8dp_last_error()
    rc = L.fp8_gemm_scaled_splitk_noalloc(16, 0, 16, 1, 256, 128, 512, 2, 7, 16, 16, 16, None)
    assert rc == -1 and b"accumulation" in L.fp8dp_last_error()
    rc = L.fp8_gemm_scaled_splitk_noalloc(16, 0, 16, 1, 4096, 4096, 1024, 2, 1, 16, 16, 16, None)
    assert rc == -1 and b"scratch" in L.fp8dp_last_error()
    rc = L.fp8_gemm_scaled_splitk_noalloc(16, 0, 16, 1, 256, 128, 512, 2, 1, 16, 16, None, None)
    assert rc == -1 and b"NULL" in L.fp8dp_last_error()
    # quantize_fused_transposed(h, rows, cols, act, fmt, st, bf16_out, fp8_out, fp8_t_out, stream)
    rc = L.quantize_fused_transposed(16, 96, 128, 1, 0, 16, None, None, 16, None)
    assert rc == -1 and b"multiple of 64" in L.fp8dp_last_error()
    rc = L.quantize_fused_transposed(16, 128, 128, 1, 0, 16, None, None, None, None)
    assert rc == -1 and b"non-NULL" in L.fp8dp_last_error()
    rc = L.quantize_fused_transposed(16, 128, 128, 1, 7, 16, None, None, 16, None)
    assert rc == -1 and b"format" in L.fp8dp_last_error()
    rc = L.quantize_fused_transposed(16, 128, 128, 1, 0, 16, None, None, 24, None)
    assert rc == -1 and b"aligned" in L.fp8dp_last_error()
    rc = L.fp8_transpose(16, 64, 96, 32, None)
    assert rc == -1 and b"64" in L.fp8dp_last_error()
    rc = L.fp8_transpose(16, 64, 64, 16, None)
    assert rc == -1 and b"same buffer" in L.fp8dp_last_error()


def test_switches_return_previous_value(L):
    prev = L.fp8dp_set_grid_limit(7)
    assert L.fp8dp_set_grid_limit(prev) == 7
    prev = L.fp8dp_set_codec(1)
    assert L.fp8dp_set_codec(prev) == 1


def test_binding_refuses_host_tensors(L):
    import torch
    h = torch.zeros(8, 128, dtype=torch.bfloat16)
    with pytest.raises(sq.Fp8dpError):
        sq.quantize_fused(h, sq.ACT_RELU2, sq.E4M3, sq.PER_GROUP128, None, None, None, None,
                          stream=0)


def test_binding_checks_weight_scale_buffer(L):
    # a per-tensor weight cast writes [1/s, s]; a one-float buffer is refused
    # before anything is launched
    import torch
    w = torch.zeros(128, 256, dtype=torch.bfloat16)
    w8 = torch.zeros(128, 256, dtype=torch.uint8)
    with pytest.raises(sq.Fp8dpError, match="2 float32"):
        sq.quantize_weight(w, sq.E4M3, sq.PER_TENSOR, w8, torch.zeros(1))
    with pytest.raises(sq.Fp8dpError, match="2 float32"):
        sq.quantize_weight(w, sq.E4M3, sq.PER_GROUP128, w8, torch.zeros(1))


def test_binding_checks_output_and_scale_sizes(L):
    # outputs and scale arrays smaller than the call would write or read are
    # refused before anything is launched
    import torch
    h = torch.zeros(4, 256, dtype=torch.bfloat16)
    with pytest.raises(sq.Fp8dpError, match="fp8_out"):
        sq.quantize_fused(h, sq.ACT_RELU2, sq.E4M3, sq.PER_TENSOR, None, None,
                          torch.zeros(1000, dtype=torch.uint8))
    with pytest.raises(sq.Fp8dpError, match="group_scale_inv"):
        sq.quantize_fused(h, sq.ACT_RELU2, sq.E4M3, sq.PER_GROUP128, None, None,
                          torch.zeros(1024, dtype=torch.uint8), torch.zeros(7))
    a8 = torch.zeros(256, 512, dtype=torch.uint8)
    w8 = torch.zeros(128, 512, dtype=torch.uint8)
    y = torch.zeros(256, 128, dtype=torch.bfloat16)
    with pytest.raises(sq.Fp8dpError, match="a_scale_inv"):
        sq.fp8_gemm_scaled(a8, 0, w8, 0, sq.PER_GROUP128, torch.zeros(4), torch.zeros(4), y)


def test_mx_argument_checks_reject_without_launching(L):
    rc = L.quantize_mx(16, 4, 48, 0, 0, None, 16, 16, None)
    assert rc == -1 and b"32" in L.fp8dp_last_error()
    rc = L.quantize_mx(16, 4, 64, 0, 0, None, 16, None, None)
    assert rc == -1 and b"NULL" in L.fp8dp_last_error()
    rc = L.quantize_mx(16, 4, 64, 0, 9, None, 16, 16, None)
    assert rc == -1 and b"format" in L.fp8dp_last_error()
    rc = L.quantize_mx(24, 4, 64, 0, 0, None, 16, 16, None)
    assert rc == -1 and b"aligned" in L.fp8dp_last_error()
    rc = L.fp8_gemm_mx(16, 0, 16, 16, 0, 16, 128, 128, 128, 1, 16, None)
    assert rc == -1 and b"256" in L.fp8dp_last_error()
    rc = L.fp8_gemm_mx(16, 0, 18, 16, 0, 16, 256, 128, 128, 1, 16, None)
    assert rc == -1 and b"aligned" in L.fp8dp_last_error()
    rc = L.fp8_gemm_mx(16, 3, 16, 16, 0, 16, 256, 128, 128, 1, 16, None)
    assert rc == -1 and b"format" in L.fp8dp_last_error()


def test_recompute_argument_checks_reject_without_launching(L):
    rc = L.quantize_recompute(16, 4, 8, 0, 0, None, 16, None)
    assert rc == -1 and b"non-NULL" in L.fp8dp_last_error()
    rc = L.quantize_recompute(16, 4, 8, 0, 0, 24, 16, None)
    assert rc == -1 and b"aligned" in L.fp8dp_last_error()
    rc = L.fp8_gemm_scaled_if(16, 0, 16, 0, 256, 128, 128, 1, 16, 16, 16, None, None)
    assert rc == -1 and b"NULL" in L.fp8dp_last_error()
    rc = L.fp8_gemm_scaled_if(16, 0, 16, 0, 0, 128, 128, 1, 16, 16, 16, 16, None)
    assert rc == -1 and b"M must be positive" in L.fp8dp_last_error()
    rc = L.fp8_gemm_scaled_if(16, 0, 16, 0, 128, 100, 128, 1, 16, 16, 16, 16, None)
    assert rc == -1 and b"multiples of 128" in L.fp8dp_last_error()
    rc = L.fp8_gemm_scaled_if(16, 0, 16, 0, 256, 128, 128, 1, 16, 16, 16, 18, None)
    assert rc == -1 and b"aligned" in L.fp8dp_last_error()
    rc = L.fp8_gemm_scaled_if(16, 0, 16, 0, 256, 128, 128, 2, 16, 16, 16, 16, None)
    assert rc == -1 and b"accumulation" in L.fp8dp_last_error()


def test_relu2_backward_argument_checks_reject_without_launching(L):
    rc = L.relu2_backward_quantize(16, 16, 0, None, 4, 8, 1, 16, None, 16, None)
    assert rc == -1 and b"inverse scale" in L.fp8dp_last_error()
    rc = L.relu2_backward_quantize(16, 16, 5, 16, 4, 8, 1, 16, None, 16, None)
    assert rc == -1 and b"cache" in L.fp8dp_last_error()
    rc = L.relu2_backward_quantize(16, 16, 2, None, 4, 8, 1, 24, None, 16, None)
    assert rc == -1 and b"aligned" in L.fp8dp_last_error()
    rc = L.relu2_backward_quantize(16, 16, 2, None, 4, 8, 1, 16, None, None, None)
    assert rc == -1 and b"NULL" in L.fp8dp_last_error()


def test_fused_dgrad_argument_checks_reject_without_launching(L):
    # fp8_gemm_relu2_backward(a, fa, b, fb, M, N, K, accum, sa, sb, cache, kind, sc, fmt, st,
    #                         out, stream)
    rc = L.fp8_gemm_relu2_backward(16, 1, 16, 0, 256, 128, 128, 1, 16, 16, None, 0, 16, 1, 16, 16, None)
    assert rc == -1 and b"NULL" in L.fp8dp_last_error()
    rc = L.fp8_gemm_relu2_backward(16, 1, 16, 0, 128, 128, 128, 1, 16, 16, 16, 0, 16, 1, 16, 16, None)
    assert rc == -1 and b"256" in L.fp8dp_last_error()
    rc = L.fp8_gemm_relu2_backward(16, 0, 16, 0, 256, 128, 128, 1, 16, 16, 16, 0, 16, 1, 16, 16, None)
    assert rc == -2
    rc = L.fp8_gemm_relu2_backward(16, 1, 16, 0, 256, 128, 128, 1, 16, 16, 16, 2, 16, 1, 16, 16, None)
    assert rc == -2
    rc = L.fp8_gemm_relu2_backward(16, 1, 16, 0, 256, 128, 128, 1, 16, 16, 24, 0, 16, 1, 16, 16, None)
    assert rc == -1 and b"aligned" in L.fp8dp_last_error()
    rc = L.fp8_gemm_relu2_backward(16, 1, 16, 0, 256, 128, 128, 4, 16, 16, 16, 0, 16, 1, 16, 16,
                                   None)
    assert rc == -1 and b"accumulation" in L.fp8dp_last_error()


def test_binding_checks_element_sizes(L):
    # a main tensor whose element size differs from what the kernel reads or
    # writes is refused before anything is launched (a uint8 y would be
    # written 2 bytes per element past its end)
    import torch
    a8 = torch.zeros(256, 512, dtype=torch.uint8)
    w8 = torch.zeros(128, 512, dtype=torch.uint8)
    one = torch.ones(1)
    with pytest.raises(sq.Fp8dpError, match="y: expected 2-byte"):
        sq.fp8_gemm_scaled(a8, 0, w8, 0, sq.PER_TENSOR, one, one,
                           torch.zeros(256, 128, dtype=torch.uint8))
    with pytest.raises(sq.Fp8dpError, match="a: expected 8-bit"):
        sq.fp8_gemm_scaled(a8.float(), 0, w8, 0, sq.PER_TENSOR, one, one,
                           torch.zeros(256, 128, dtype=torch.bfloat16))
    with pytest.raises(sq.Fp8dpError, match="b: expected 8-bit"):
        sq.fp8_gemm_scaled_if(a8, 0, w8.to(torch.int16), 0, one, one,
                              torch.zeros(256, 128, dtype=torch.bfloat16), one)
    with pytest.raises(sq.Fp8dpError, match="y: expected 2-byte"):
        sq.fp8_gemm_scaled_splitk(a8, 0, w8, 0, 2, one, one, torch.zeros(2 * 256 * 128),
                                  torch.zeros(256, 128, dtype=torch.float32))
    with pytest.raises(sq.Fp8dpError, match="h: expected 2-byte"):
        sq.quantize_fused(torch.zeros(4, 256), sq.ACT_RELU2, sq.E4M3, sq.PER_TENSOR, None)
    with pytest.raises(sq.Fp8dpError, match="bf16_out: expected 2-byte"):
        sq.quantize_fused(torch.zeros(4, 256, dtype=torch.bfloat16), sq.ACT_RELU2, sq.E4M3,
                          sq.PER_TENSOR, None, torch.zeros(4, 256, dtype=torch.uint8))
    with pytest.raises(sq.Fp8dpError, match="fp8_out: expected 8-bit"):
        sq.quantize_fused(torch.zeros(4, 256, dtype=torch.bfloat16), sq.ACT_RELU2, sq.E4M3,
                          sq.PER_TENSOR, None, None, torch.zeros(4, 256, dtype=torch.float16))


def test_binding_checks_every_entry_points_tensors(L):
    # the same refusals on the other entry points: inputs read at 2 bytes per
    # element, outputs written past the end of a smaller buffer
    import torch
    bf = lambda *s: torch.zeros(*s, dtype=torch.bfloat16)
    u8 = lambda *s: torch.zeros(*s, dtype=torch.uint8)
    with pytest.raises(sq.Fp8dpError, match="dA: expected 2-byte"):
        sq.relu2_backward_quantize(u8(4, 256), u8(4, 256), sq.CACHE_E4M3, None, sq.E5M2, None,
                                   u8(4, 256))
    with pytest.raises(sq.Fp8dpError, match="a_cache: expected 2-byte"):
        sq.relu2_backward_quantize(bf(4, 256), u8(4, 256), sq.CACHE_BF16, None, sq.E5M2, None,
                                   u8(4, 256))
    with pytest.raises(sq.Fp8dpError, match="bf16_out: needs"):
        sq.relu2_backward_quantize(bf(4, 256), u8(4, 256), sq.CACHE_E4M3, None, sq.E5M2, None,
                                   u8(4, 256), bf(4, 128))
    with pytest.raises(sq.Fp8dpError, match="quantize_recompute: fp8_out: needs"):
        sq.quantize_recompute(bf(4, 256), sq.ACT_RELU2, sq.E4M3, None, u8(4, 128))
    with pytest.raises(sq.Fp8dpError, match="quantize_recompute: h: expected 2-byte"):
        sq.quantize_recompute(u8(4, 256), sq.ACT_RELU2, sq.E4M3, None, u8(4, 256))
    with pytest.raises(sq.Fp8dpError, match="quantize_mx: h: expected 2-byte"):
        sq.quantize_mx(u8(4, 256), sq.ACT_RELU2, sq.E4M3, u8(4, 256), u8(4, 8))
    with pytest.raises(sq.Fp8dpError, match="quantize_mx: bf16_out: needs"):
        sq.quantize_mx(bf(4, 256), sq.ACT_RELU2, sq.E4M3, u8(4, 256), u8(4, 8), bf(2, 256))
    with pytest.raises(sq.Fp8dpError, match="quantize_weight: w8: needs"):
        sq.quantize_weight(bf(128, 256), sq.E4M3, sq.PER_TENSOR, u8(64, 256), torch.zeros(2))
    with pytest.raises(sq.Fp8dpError, match="quantize_weight: w: expected 2-byte"):
        sq.quantize_weight(torch.zeros(128, 256), sq.E4M3, sq.PER_TENSOR, u8(128, 256),
                           torch.zeros(2))
    with pytest.raises(sq.Fp8dpError, match="gemm_bf16_quantize_fused: x: expected 2-byte"):
        sq.gemm_bf16_quantize_fused(torch.zeros(256, 128), bf(128, 128))
    with pytest.raises(sq.Fp8dpError, match="gemm_bf16_quantize_fused: fp8_out: expected 8-bit"):
        sq.gemm_bf16_quantize_fused(bf(256, 128), bf(128, 128), fp8_out=bf(256, 128))
    with pytest.raises(sq.Fp8dpError, match="fp8_transpose: dst: expected 8-bit"):
        sq.fp8_transpose(u8(64, 128), bf(128, 64))
    with pytest.raises(sq.Fp8dpError, match="run_flag: needs"):
        sq.fp8_gemm_scaled_if(u8(256, 512), 0, u8(128, 512), 0, torch.ones(1), torch.ones(1),
                              bf(256, 128), u8(2))
    with pytest.raises(sq.Fp8dpError, match="fp8dp_bench_copy: dst: needs"):
        sq.fp8dp_bench_copy(u8(4096), u8(2048))
    with pytest.raises(sq.Fp8dpError, match="fp8dp_bench_cast: out: needs"):
        sq.fp8dp_bench_cast(bf(4096), sq.E4M3, None, u8(2048))
    with pytest.raises(sq.Fp8dpError, match="fp8dp_bench_act_bf16: out: needs"):
        sq.fp8dp_bench_act_bf16(bf(4096), sq.ACT_RELU2, bf(2048))
    with pytest.raises(sq.Fp8dpError, match="fp8dp_convert_f32: out: needs"):
        sq.fp8dp_convert_f32(torch.zeros(64), 5, u8(64))
    with pytest.raises(sq.Fp8dpError, match="fp8dp_scale_rule: scale: needs"):
        sq.fp8dp_scale_rule(torch.zeros(8), 1.0, sq.E4M3, torch.zeros(4))


def test_binding_refuses_a_tensor_on_another_device(monkeypatch):
    # the kernels run on the current device's stream; a tensor on another
    # device is refused before any launch
    class OnDevice1:
        is_cuda = True

        def is_contiguous(self):
            return True

        def get_device(self):
            return 1

        def data_ptr(self):
            return 4096

    monkeypatch.setattr(sq, "_current_device", lambda: 0)
    with pytest.raises(sq.Fp8dpError, match="tensor on device 1, the current device is 0"):
        sq._p(OnDevice1())
    monkeypatch.setattr(sq, "_current_device", lambda: 1)
    assert sq._p(OnDevice1()) == 4096


def test_rows_cols_of_a_tensor():
    # rows x cols as the element-wise calls read a tensor: 1-D is one row,
    # more dimensions are rows of their trailing elements; no view is built
    import torch
    cases = {(10,): (1, 10), (4, 6): (4, 6), (3, 2, 5): (3, 10), (0, 7): (0, 7), (0, 2, 3): (0, 6)}
    for shape, want in cases.items():
        assert sq._rows_cols(torch.empty(shape)) == want, shape
