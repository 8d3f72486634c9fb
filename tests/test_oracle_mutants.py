"""The oracle's pins catch plausible mistakes (CPU only).

Each mutant below is oracle.c with one plausible mistake planted -- a dropped
term, a wrong sign, bias, index or operand, a rounding or comparison changed.
It is compiled to a library of its own, and the oracle's pin tests
(tests/test_oracle_*.py, which check the oracle against the pages' worked
examples, closed forms, library routines and brute force) run against it in
a separate process (ORACLE_LIB names the library).  Every mutant must make at
least one pin fail.  The mistakes are planted only in temporary copies on
the CPU; the real oracle is untouched.
"""
import glob
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]

# (name, text in oracle.c, replacement); each text occurs exactly once
MUTANTS = [
    ("decode: normal exponent bias off by one",
     "v = ldexp(1.0 + (double)m / (1 << f.mbits), e - f.bias);",
     "v = ldexp(1.0 + (double)m / (1 << f.mbits), e - f.bias + 1);"),
    ("decode: subnormal scale off by one binade",
     "v = ldexp((double)m / (1 << f.mbits), f.emin);",
     "v = ldexp((double)m / (1 << f.mbits), f.emin - 1);"),
    ("decode: sign dropped",
     "return sign ? -v : v;",
     "return v;"),
    ("E4M3: largest finite code taken as the NaN code",
     "f.max_code = 0x7E;",
     "f.max_code = 0x7D;"),
    ("E5M2: largest finite code taken as infinity",
     "f.max_code = 0x7B;",
     "f.max_code = 0x7C;"),
    ("encode: ties away from zero instead of to even",
     "*n_out = nearbyint(ax / q);",
     "*n_out = floor(ax / q + 0.5);"),
    ("encode: truncation instead of rounding",
     "*n_out = nearbyint(ax / q);",
     "*n_out = floor(ax / q);"),
    ("encode: saturation loses the sign",
     "if (ax >= f.maxval) return sign | f.max_code;",
     "if (ax >= f.maxval) return f.max_code;"),
    ("encode: NaN loses its sign",
     "if (isnan(x)) return sign | 0x7F;",
     "if (isnan(x)) return 0x7F;"),
    ("encode: subnormal cell spacing from the wrong binade",
     "if (e < f->emin) e = f->emin;   /* subnormal cells share the emin spacing */",
     "if (e < f->emin) e = f->emin - 1;"),
    ("saturation: values that round to the maximum counted",
     "return ldexp(n, e - f.mbits) > f.maxval;",
     "return ldexp(n, e - f.mbits) >= f.maxval;"),
    ("saturation: NaN counted",
     "if (isnan(x)) return 0;\n  if (isinf(x)) return 1;",
     "if (isnan(x)) return 1;\n  if (isinf(x)) return 1;"),
    ("saturation: infinity not counted",
     "if (isnan(x)) return 0;\n  if (isinf(x)) return 1;",
     "if (isnan(x)) return 0;\n  if (isinf(x)) return 0;"),
    ("BF16: one fraction bit too many",
     "double q = ldexp(1.0, e - 7);             /* BF16 keeps 7 fraction bits */",
     "double q = ldexp(1.0, e - 8);"),
    ("BF16: ties away from zero",
     "double r = nearbyint(ax / q) * q;         /* exact in double */",
     "double r = floor(ax / q + 0.5) * q;"),
    ("scale rule: margin dropped",
     "float d = amax * margin;",
     "float d = amax;"),
    ("scale rule: E5M2 maximum taken as E4M3's",
     "float fmax = (fmt == ORC_E4M3) ? 448.0f : 57344.0f;",
     "float fmax = 448.0f;"),
    ("scale rule: zero amax gives scale 0 instead of 1",
     "if (!(d > 0.0f) || isinf(d) || !isfinite(s)) return 1.0f;",
     "if (!(d > 0.0f) || isinf(d) || !isfinite(s)) return 0.0f;"),
    ("squared ReLU: negative inputs pass through",
     "float a = (x > 0.0f) ? x * x : 0.0f;",
     "float a = (x > 0.0f) ? x * x : x;"),
    ("squared ReLU: not squared",
     "float a = (x > 0.0f) ? x * x : 0.0f;",
     "float a = (x > 0.0f) ? x : 0.0f;"),
    ("per-tensor amax: sign bit not masked",
     "      uint32_t mag = ((uint32_t)(b & 0x7FFF)) << 16;\n      if (mag > amax) amax = mag;\n"
     "      float v = oracle_bf16_to_f32(b) * scale;",
     "      uint32_t mag = ((uint32_t)b) << 16;\n      if (mag > amax) amax = mag;\n"
     "      float v = oracle_bf16_to_f32(b) * scale;"),
    ("per-tensor cast: scale not applied",
     "      float v = oracle_bf16_to_f32(b) * scale;\n      if (fp8_out) fp8_out[i]",
     "      float v = oracle_bf16_to_f32(b);\n      if (fp8_out) fp8_out[i]"),
    ("per-group: groups start 127 elements apart",
     "const uint16_t* hg = h + g * ORC_GROUP;",
     "const uint16_t* hg = h + g * (ORC_GROUP - 1);"),
    ("per-group: group scale with a margin",
     "float sg = oracle_scale_from_amax(u2f(gmax), 1.0f, fmt);",
     "float sg = oracle_scale_from_amax(u2f(gmax), 1.25f, fmt);"),
    ("per-group: stored scale not inverted",
     "if (group_scale_inv) group_scale_inv[g] = oracle_recip_f32(sg);",
     "if (group_scale_inv) group_scale_inv[g] = sg;"),
    ("weight blocks: block amax over one row only",
     "      for (int64_t r = 0; r < ORC_GROUP; ++r)\n        for (int64_t c = 0; c < ORC_GROUP; ++c) {\n"
     "          uint32_t mag",
     "      for (int64_t r = 0; r < 1; ++r)\n        for (int64_t c = 0; c < ORC_GROUP; ++c) {\n"
     "          uint32_t mag"),
    ("history: ring position never advances",
     "st->hist_pos = (st->hist_pos + 1) % st->hist_len;",
     "st->hist_pos = st->hist_pos % st->hist_len;"),
    ("history: newest amax left out of the maximum",
     "for (int i = 0; i < st->hist_len; ++i) {\n    uint32_t b = f2u(st->history[i]) & 0x7FFFFFFFu;",
     "for (int i = 0; i < st->hist_len - 1; ++i) {\n    uint32_t b = f2u(st->history[i]) & 0x7FFFFFFFu;"),
    ("history: used inverse scale published after the new scale",
     "  st->scale_inv_used = st->scale_inv;\n  st->scale = oracle_scale_from_amax(history_max(st), "
     "st->margin, st->fmt);\n  st->scale_inv = oracle_recip_f32(st->scale);",
     "  st->scale = oracle_scale_from_amax(history_max(st), st->margin, st->fmt);\n"
     "  st->scale_inv = oracle_recip_f32(st->scale);\n  st->scale_inv_used = st->scale_inv;"),
    ("history: overflow never flagged",
     "st->overflow = st->sat_acc > 0 ? 1u : 0u;",
     "st->overflow = 0u;"),
    ("accumulate: saturation counts replaced instead of added",
     "st->sat_acc += sat;",
     "st->sat_acc = sat;"),
    ("GEMM: one scale not divided out",
     "double denom = sa_v * sb_v;",
     "double denom = sa_v;"),
    ("GEMM: B decoded with A's format",
     "double p = da[arow[k]] * db[brow[k]];",
     "double p = da[arow[k]] * da[brow[k]];"),
    ("GEMM: per-group B block taken from the column within the block",
     "sb_v = sb[(nn / ORC_GROUP) * ngroups + g];",
     "sb_v = sb[(nn % 2) * ngroups + g];"),
    ("GEMM: per-group A scale of the wrong group",
     "sa_v = sa[m * ngroups + g];",
     "sa_v = sa[m * ngroups];"),
    ("GEMM: absolute sum signed",
     "          sabs += fabs(p);\n        }\n        double sa_v, sb_v;",
     "          sabs += p;\n        }\n        double sa_v, sb_v;"),
    ("BF16 GEMM: weight row read from the activation",
     "double p = (double)oracle_bf16_to_f32(xr[k]) * (double)oracle_bf16_to_f32(wr[k]);",
     "double p = (double)oracle_bf16_to_f32(xr[k]) * (double)oracle_bf16_to_f32(xr[k]);"),
    ("MX exponent: strict comparison",
     "if (amax <= ldexp(f.maxval, k)) return k;",
     "if (amax < ldexp(f.maxval, k)) return k;"),
    ("MX exponent: range starts at -126",
     "for (int k = -127; k <= 127; ++k)",
     "for (int k = -126; k <= 127; ++k)"),
    ("MX exponent: infinite block gets the smallest exponent",
     "if (nonfinite) return 127;",
     "if (nonfinite) return -127;"),
    ("MX cast: block scale applied the wrong way",
     "float v = (float)ldexp((double)oracle_bf16_to_f32(b[j]), -k);",
     "float v = (float)ldexp((double)oracle_bf16_to_f32(b[j]), k);"),
    ("MX cast: E8M0 bias off by one",
     "if (scale_e8m0) scale_e8m0[g] = (uint8_t)(k + 127);",
     "if (scale_e8m0) scale_e8m0[g] = (uint8_t)(k + 128);"),
    ("MX GEMM: B's block exponent bias off by one",
     "double x = ldexp(1.0, (int)ea[m * nb + j] - 127 + (int)eb[n * nb + j] - 127);",
     "double x = ldexp(1.0, (int)ea[m * nb + j] - 127 + (int)eb[n * nb + j] - 126);"),
    ("MX GEMM: A's exponent from the wrong block",
     "double x = ldexp(1.0, (int)ea[m * nb + j] - 127 + (int)eb[n * nb + j] - 127);",
     "double x = ldexp(1.0, (int)ea[m * nb] - 127 + (int)eb[n * nb + j] - 127);"),
    ("relu2 backward: factor 2 dropped",
     "float two_r = 2.0f * r;",
     "float two_r = r;"),
    ("relu2 backward: cache inverse scale not applied",
     "a = d * a_scale_inv;",
     "a = d;"),
    ("relu2 backward: gradient cast scale not applied",
     "    float v = oracle_bf16_to_f32(b) * scale;\n    if (fp8_out) fp8_out[i] = oracle_fp8_encode(v, fmt);\n"
     "    sat += (uint64_t)oracle_fp8_saturates(v, fmt);\n  }\n  if (amax_bits_out) *amax_bits_out = amax;\n"
     "  if (sat_out) *sat_out = sat;\n}\n\n/* ----",
     "    float v = oracle_bf16_to_f32(b);\n    if (fp8_out) fp8_out[i] = oracle_fp8_encode(v, fmt);\n"
     "    sat += (uint64_t)oracle_fp8_saturates(v, fmt);\n  }\n  if (amax_bits_out) *amax_bits_out = amax;\n"
     "  if (sat_out) *sat_out = sat;\n}\n\n/* ----"),
]

PIN_TESTS = sorted(p for p in glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py"))
                   if not p.endswith("test_oracle_mutants.py"))


def _run_mutant(args):
    i, (name, old, new), src, tmp = args
    if src.count(old) != 1:
        return name, "pattern", src.count(old), ""
    lib = os.path.join(tmp, f"mutant{i}.so")
    path = os.path.join(tmp, f"mutant{i}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    subprocess.run(["gcc", *CFLAGS, path, "-o", lib, "-lm"], check=True, capture_output=True)
    env = dict(os.environ, ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", *PIN_TESTS], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    return name, "ran", r.returncode, r.stdout[-400:]


@pytest.fixture(scope="module")
def outcomes():
    src = open(SRC).read()
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max(1, min(6, (os.cpu_count() or 2) - 1))) as ex:
            res = list(ex.map(_run_mutant, [(i, m, src, tmp) for i, m in enumerate(MUTANTS)]))
    return {name: (kind, rc, tail) for name, kind, rc, tail in res}


def test_unmutated_oracle_passes_its_pins():
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", *PIN_TESTS], cwd=ROOT, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stdout[-800:]


@pytest.mark.parametrize("name", [m[0] for m in MUTANTS])
def test_every_planted_mistake_fails_a_pin(outcomes, name):
    kind, rc, tail = outcomes[name]
    assert kind == "ran", f"{name}: the mutated text occurs {rc} times in oracle.c"
    assert rc == 1, f"{name}: survived the pins (pytest exit {rc})\n{tail}"
