/*
 * oracle.c -- plain, slow, single-threaded CPU reference for the scaled FP8
 * down-projection path (fused activation + BF16 copy + scaled FP8 cast +
 * running amax + saturation count, delayed-scaling history, scaled FP8 GEMM).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product path
 * never calls it, and it shares no code, header, table or constant generator
 * with the HIP library: every rule below is written out again from its
 * definition.
 *
 * Sources (page title -- section):
 *   [FP8T] "FP8 training: what it is and how it works"
 *          -- "FP8 training from first principles" (definitions of scaling
 *             factor and amax), "Step 1: Choose the 8-bit format",
 *             "Step 2: Scale the tensor into range", "Step 3: Multiply in FP8
 *             and add up in higher precision", "Trade-offs and edge cases".
 *   [FP8I] "FP8 Training & Inference"
 *          -- "FP8 Formats: E4M3 vs E5M2", "Per-Tensor Scaling for FP8",
 *             "Delayed Scaling".
 *   [PARA] "Paradigma Details FP8 and Optimizer Tricks Behind NanoGPT
 *          Records" -- the fused-kernel paragraph (BF16 copy, FP8 copy,
 *          running maxima, previous step's amax times a safety margin).
 *   [PRE]  "Pretraining at scale" -- 4a "What a floating-point number is"
 *          (sign/exponent/fraction value formula, round to nearest,
 *          subnormals, underflow below half the smallest subnormal).
 *
 * Precision: the formats are bit-exact definitions; the scale and the scaled
 * value are computed in IEEE binary32 with round-to-nearest-even (the
 * precision the kernel uses, one operation at a time, no fused multiply-add);
 * the GEMM reference is float64 over the dequantized codes.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC
 * (see oracle/build.py).  No threads, no SIMD intrinsics.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORC_E4M3 0
#define ORC_E5M2 1
#define ORC_ACT_IDENTITY 0
#define ORC_ACT_RELU2 1
#define ORC_PER_TENSOR 0
#define ORC_PER_GROUP128 1
#define ORC_GROUP 128
#define ORC_MAX_HIST 16

/* ------------------------------------------------------------------------ */
/* Format description.  [FP8T] Step 1 and [FP8I] "FP8 Formats": E4M3 is      */
/* 1 sign + 4 exponent + 3 mantissa bits, largest value 448, no infinity;    */
/* E5M2 is 1 + 5 + 2 bits, largest value 57344, with infinities.  Biases are */
/* the usual 2^(ebits-1) - 1.                                               */
/* ------------------------------------------------------------------------ */
typedef struct {
  int ebits, mbits, bias;
  int emin;          /* exponent of the smallest normal binade: 1 - bias    */
  double maxval;     /* largest finite magnitude                             */
  uint8_t max_code;  /* code (without sign) of the largest finite magnitude  */
} orc_format;

static orc_format orc_fmt(int fmt) {
  orc_format f;
  if (fmt == ORC_E4M3) {
    f.ebits = 4; f.mbits = 3; f.bias = 7;
    /* 0x7F is the NaN pattern, so the largest finite code is 0x7E:
       exponent field 15, mantissa 6 -> 2^8 * 1.75 = 448. */
    f.max_code = 0x7E;
  } else {
    f.ebits = 5; f.mbits = 2; f.bias = 15;
    /* exponent field 31 is infinity/NaN, so the largest finite code is
       exponent 30, mantissa 3 -> 2^15 * 1.75 = 57344. */
    f.max_code = 0x7B;
  }
  f.emin = 1 - f.bias;
  /* both maxima are 1.75 * 2^(top exponent field - bias): 2^8 and 2^15 */
  f.maxval = ldexp(1.75, (fmt == ORC_E4M3 ? 15 : 30) - f.bias);
  return f;
}

static uint32_t f2u(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float u2f(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/* Value of an FP8 code: (-1)^S * 2^(E - bias) * (1 + M / 2^mbits) for a
   normal code, (-1)^S * 2^(1 - bias) * (M / 2^mbits) for a subnormal one
   ([PRE] 4a gives the formula; [FP8T]/[FP8I] give the bit counts). */
double oracle_fp8_decode(uint8_t code, int fmt) {
  orc_format f = orc_fmt(fmt);
  int sign = code >> 7;
  int e = (code >> f.mbits) & ((1 << f.ebits) - 1);
  int m = code & ((1 << f.mbits) - 1);
  double v;
  if (fmt == ORC_E4M3 && e == 15 && m == 7) return NAN;      /* S.1111.111 */
  if (fmt == ORC_E5M2 && e == 31) {
    if (m != 0) return NAN;
    return sign ? -INFINITY : INFINITY;
  }
  if (e == 0)
    v = ldexp((double)m / (1 << f.mbits), f.emin);
  else
    v = ldexp(1.0 + (double)m / (1 << f.mbits), e - f.bias);
  return sign ? -v : v;
}

/* Round |x| (finite, double, exactly a binary32 value) to the format's grid,
   ignoring the upper range limit: returns the grid multiple n and the
   exponent e of the grid cell, so the rounded magnitude is n * 2^(e-mbits).
   Round to nearest, ties to even n ([PRE] 4a: "rounds ... to the nearest
   value"; ties to even is the IEEE default). */
static void round_to_grid(double ax, const orc_format* f, int* e_out, double* n_out) {
  int e;
  if (ax == 0.0) {
    e = f->emin;
  } else {
    (void)frexp(ax, &e);   /* ax = frac * 2^e, frac in [0.5, 1) */
    e -= 1;                /* ax in [2^e, 2^(e+1)) */
    if (e < f->emin) e = f->emin;   /* subnormal cells share the emin spacing */
  }
  double q = ldexp(1.0, e - f->mbits);
  *n_out = nearbyint(ax / q);       /* exact division by a power of two */
  *e_out = e;
}

/* Saturating round-to-nearest-even cast of a binary32 value to FP8.
   NaN -> 0x7F with the sign kept; |x| >= max (infinity included) -> +-max;
   otherwise the nearest grid value, which also gives signed zero for
   |x| <= half the smallest subnormal (a tie there goes to the even code 0). */
uint8_t oracle_fp8_encode(float x, int fmt) {
  orc_format f = orc_fmt(fmt);
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return sign | 0x7F;
  double ax = fabs((double)x);
  if (ax >= f.maxval) return sign | f.max_code;
  int e; double n;
  round_to_grid(ax, &f, &e, &n);
  int full = 1 << f.mbits;
  int ni = (int)n;                  /* 0 .. 2*full */
  if (e == f.emin && ni < full) return sign | (uint8_t)ni;   /* subnormal or zero */
  if (ni == 2 * full) { e += 1; ni = full; }                  /* carried into next binade */
  int efield = e + f.bias;
  return sign | (uint8_t)((efield << f.mbits) | (ni - full));
}

/* Saturation predicate: the value is counted when a cast that does NOT
   saturate would have produced a non-finite result, i.e. when |x| is infinite
   or its unbounded round-to-nearest-even rounding lies above the format
   maximum.  NaN inputs are not counted ([FP8I] "Delayed Scaling": overflow is
   what the safety check must detect). */
int oracle_fp8_saturates(float x, int fmt) {
  orc_format f = orc_fmt(fmt);
  if (isnan(x)) return 0;
  if (isinf(x)) return 1;
  double ax = fabs((double)x);
  if (ax <= f.maxval) return 0;
  int e; double n;
  round_to_grid(ax, &f, &e, &n);
  return ldexp(n, e - f.mbits) > f.maxval;
}

/* BF16 (1 sign + 8 exponent + 7 fraction bits, [PRE] 4a) round to nearest,
   ties to even, from binary32.  NaN keeps its sign and top payload bits and
   is made quiet; overflow rounds to infinity as IEEE rounding does. */
uint16_t oracle_bf16_rne(float x) {
  uint32_t u = f2u(x);
  if (isnan(x)) return (uint16_t)((u >> 16) | 0x0040);
  double ax = fabs((double)x);
  int sign = (u >> 31) != 0;
  if (isinf(x)) return (uint16_t)(sign ? 0xFF80 : 0x7F80);
  int e;
  if (ax == 0.0) {
    e = -126;
  } else {
    (void)frexp(ax, &e);
    e -= 1;
    if (e < -126) e = -126;                 /* binary32/BF16 subnormal range */
  }
  double q = ldexp(1.0, e - 7);             /* BF16 keeps 7 fraction bits */
  double r = nearbyint(ax / q) * q;         /* exact in double */
  float rf = (float)r;                      /* exact, or +inf past the top */
  uint16_t out = (uint16_t)(f2u(rf) >> 16);
  return sign ? (uint16_t)(out | 0x8000) : out;
}

float oracle_bf16_to_f32(uint16_t b) { return u2f((uint32_t)b << 16); }

/* Scale rule ([FP8T] Step 2: scaling factor = format maximum / amax;
   [PARA]: the amax used is the previous step's value times a safety
   margin).  binary32 arithmetic: d = amax * margin, s = max / d.  A value of
   d that is not a positive finite number, or a quotient that is not finite,
   leaves nothing to scale by: the scale falls back to 1. */
float oracle_scale_from_amax(float amax, float margin, int fmt) {
  float fmax = (fmt == ORC_E4M3) ? 448.0f : 57344.0f;
  float d = amax * margin;
  float s = fmax / d;
  if (!(d > 0.0f) || isinf(d) || !isfinite(s)) return 1.0f;
  return s;
}

float oracle_recip_f32(float s) { float r = 1.0f / s; return r; }

/* Activation applied to one BF16 input value, result rounded to BF16.
   Identity keeps the input bits unchanged (no rounding step happens).
   Squared ReLU: a = h*h when h > 0, else +0 (NaN and -0 give +0); the
   product of two BF16 values is computed in binary32 and then rounded to
   BF16 -- the copy written for the backward pass ([PARA]). */
static uint16_t act_bf16(uint16_t h, int act) {
  if (act == ORC_ACT_IDENTITY) return h;
  float x = oracle_bf16_to_f32(h);
  float a = (x > 0.0f) ? x * x : 0.0f;
  return oracle_bf16_rne(a);
}

/* One quantization call over a row-major [rows x cols] BF16 tensor.
 *   act  : ORC_ACT_IDENTITY / ORC_ACT_RELU2
 *   mode : ORC_PER_TENSOR  -> every element is multiplied by `scale`
 *          ORC_PER_GROUP128 -> each run of 128 consecutive elements of a row
 *                              gets s_g = max / amax_g (current scaling,
 *                              margin 1) and group_scale_inv[g] = 1 / s_g
 *                              ([FP8T] "Fine-grained quantization"; the
 *                              1-by-128 activation tile of "Trade-offs").
 *   bf16_out, fp8_out, group_scale_inv, group_scale (the multipliers s_g
 *   themselves) may be NULL.
 * Outputs amax as the binary32 bit pattern of max |b| (the maximum of the
 * magnitude bit patterns, compared as unsigned integers), and the number of
 * saturating elements.
 */
void oracle_quantize(const uint16_t* h, int64_t rows, int64_t cols, int act, int fmt, int mode,
                     float scale, uint16_t* bf16_out, uint8_t* fp8_out, float* group_scale_inv,
                     float* group_scale, uint32_t* amax_bits_out, uint64_t* sat_out) {
  int64_t n = rows * cols;
  uint32_t amax = 0;
  uint64_t sat = 0;
  if (mode == ORC_PER_TENSOR) {
    for (int64_t i = 0; i < n; ++i) {
      uint16_t b = act_bf16(h[i], act);
      if (bf16_out) bf16_out[i] = b;
      uint32_t mag = ((uint32_t)(b & 0x7FFF)) << 16;
      if (mag > amax) amax = mag;
      float v = oracle_bf16_to_f32(b) * scale;
      if (fp8_out) fp8_out[i] = oracle_fp8_encode(v, fmt);
      sat += (uint64_t)oracle_fp8_saturates(v, fmt);
    }
  } else {
    int64_t groups = n / ORC_GROUP;
    for (int64_t g = 0; g < groups; ++g) {
      const uint16_t* hg = h + g * ORC_GROUP;
      uint32_t gmax = 0;
      for (int j = 0; j < ORC_GROUP; ++j) {
        uint32_t mag = ((uint32_t)(act_bf16(hg[j], act) & 0x7FFF)) << 16;
        if (mag > gmax) gmax = mag;
      }
      if (gmax > amax) amax = gmax;
      float sg = oracle_scale_from_amax(u2f(gmax), 1.0f, fmt);
      if (group_scale_inv) group_scale_inv[g] = oracle_recip_f32(sg);
      if (group_scale) group_scale[g] = sg;
      for (int j = 0; j < ORC_GROUP; ++j) {
        uint16_t b = act_bf16(hg[j], act);
        if (bf16_out) bf16_out[g * ORC_GROUP + j] = b;
        float v = oracle_bf16_to_f32(b) * sg;
        if (fp8_out) fp8_out[g * ORC_GROUP + j] = oracle_fp8_encode(v, fmt);
        sat += (uint64_t)oracle_fp8_saturates(v, fmt);
      }
    }
  }
  if (amax_bits_out) *amax_bits_out = amax;
  if (sat_out) *sat_out = sat;
}

/* Weight cast with current scaling over 128 x 128 blocks of a row-major
   [N x K] BF16 weight ([FP8T] "Trade-offs": DeepSeek-V3 gives each 128 by
   128 weight block its own scale).  Block (i, j) covers rows 128i..128i+127
   and columns 128j..128j+127; its multiplier is max / amax_block (margin 1)
   and scale_inv[i * (K/128) + j] = 1 / that multiplier (scale[] receives the
   multiplier itself when given).  Per-tensor weights
   use oracle_quantize with the multiplier from the tensor's amax. */
void oracle_quantize_weight_blocks(const uint16_t* w, int64_t N, int64_t K, int fmt, uint8_t* w8,
                                   float* scale_inv, float* scale) {
  int64_t kb = K / ORC_GROUP;
  for (int64_t bi = 0; bi < N / ORC_GROUP; ++bi) {
    for (int64_t bj = 0; bj < kb; ++bj) {
      uint32_t m = 0;
      for (int64_t r = 0; r < ORC_GROUP; ++r)
        for (int64_t c = 0; c < ORC_GROUP; ++c) {
          uint32_t mag = ((uint32_t)(w[(bi * ORC_GROUP + r) * K + bj * ORC_GROUP + c] & 0x7FFF)) << 16;
          if (mag > m) m = mag;
        }
      float s = oracle_scale_from_amax(u2f(m), 1.0f, fmt);
      scale_inv[bi * kb + bj] = oracle_recip_f32(s);
      if (scale) scale[bi * kb + bj] = s;
      for (int64_t r = 0; r < ORC_GROUP; ++r)
        for (int64_t c = 0; c < ORC_GROUP; ++c) {
          int64_t idx = (bi * ORC_GROUP + r) * K + bj * ORC_GROUP + c;
          float v = oracle_bf16_to_f32(w[idx]) * s;
          w8[idx] = oracle_fp8_encode(v, fmt);
        }
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Delayed scaling state ([PARA]: previous step's amax times a safety margin; */
/* [FP8T] "Trade-offs": delayed scaling keeps a stored history of earlier    */
/* amax values; [FP8I] "Delayed Scaling": detect overflow).                   */
/* The history holds hist_len amax values; the scale for the next step uses  */
/* the largest of them.                                                      */
/* ------------------------------------------------------------------------ */
typedef struct {
  float scale;            /* multiplier for the next step's cast             */
  float scale_inv;        /* 1/scale                                          */
  float scale_inv_used;   /* 1/scale of the step most recently consumed       */
  uint32_t amax_acc;      /* running amax bits of the current step            */
  uint64_t sat_acc;       /* running saturation count of the current step     */
  uint64_t sat_last;      /* saturation count of the step most recently consumed */
  uint32_t overflow;      /* 1 when that step saturated                       */
  float margin;
  int32_t hist_len;
  int32_t hist_pos;
  uint32_t steps;
  int32_t fmt;
  float history[ORC_MAX_HIST];
} oracle_state;

int64_t oracle_state_size(void) { return (int64_t)sizeof(oracle_state); }

static float history_max(const oracle_state* st) {
  uint32_t m = 0;
  for (int i = 0; i < st->hist_len; ++i) {
    uint32_t b = f2u(st->history[i]) & 0x7FFFFFFFu;
    if (b > m) m = b;
  }
  return u2f(m);
}

int oracle_state_init(oracle_state* st, int fmt, int hist_len, float margin, float initial_amax) {
  if (hist_len < 1 || hist_len > ORC_MAX_HIST) return -1;
  memset(st, 0, sizeof(*st));
  st->fmt = fmt;
  st->margin = margin;
  st->hist_len = hist_len;
  for (int i = 0; i < hist_len; ++i) st->history[i] = initial_amax;
  st->scale = oracle_scale_from_amax(history_max(st), margin, fmt);
  st->scale_inv = oracle_recip_f32(st->scale);
  st->scale_inv_used = st->scale_inv;
  return 0;
}

/* Consume the step: record its amax in the history, publish the inverse of
   the scale that step was cast with, derive the next scale, flag overflow,
   and clear the running accumulators. */
void oracle_history_update(oracle_state* st) {
  st->history[st->hist_pos] = u2f(st->amax_acc);
  st->hist_pos = (st->hist_pos + 1) % st->hist_len;
  st->scale_inv_used = st->scale_inv;
  st->scale = oracle_scale_from_amax(history_max(st), st->margin, st->fmt);
  st->scale_inv = oracle_recip_f32(st->scale);
  st->sat_last = st->sat_acc;
  st->overflow = st->sat_acc > 0 ? 1u : 0u;
  st->amax_acc = 0;
  st->sat_acc = 0;
  st->steps += 1;
}

/* Fold one quantization call's amax bits and saturation count into the state. */
void oracle_state_accumulate(oracle_state* st, uint32_t amax_bits, uint64_t sat) {
  if (amax_bits > st->amax_acc) st->amax_acc = amax_bits;
  st->sat_acc += sat;
}

/* ------------------------------------------------------------------------ */
/* Reference GEMM ([FP8T] Step 3: FP8 inputs, wide accumulation; [FP8I]      */
/* "Per-Tensor Scaling": the scales are factored out of the product and the  */
/* output is rescaled).                                                      */
/*   a : [M x K] codes, b : [N x K] codes (row-major, K contiguous)           */
/*   mode PER_TENSOR : sa[0], sb[0] are the cast multipliers s_a, s_b          */
/*   mode PER_GROUP128: sa is [M x K/128] (one per 1x128 activation tile),    */
/*                     sb is [N/128 x K/128] (one per 128x128 weight block)   */
/* ref[m,n] = sum over 128-wide K blocks g (one block = all of K per tensor)  */
/*            of S_g / (s_a * s_b), S_g = sum_k dec(a[m,k]) * dec(b[n,k]);   */
/* absref likewise with |dec * dec|.  Rows listed in `rows` (nrows of them)  */
/* are computed; rows == NULL means all M rows.                              */
/* ------------------------------------------------------------------------ */
void oracle_gemm_f64(const uint8_t* a, int fa, const uint8_t* b, int fb, int64_t M, int64_t N,
                     int64_t K, int mode, const float* sa, const float* sb, const int64_t* rows,
                     int64_t nrows, double* ref, double* absref) {
  double da[256], db[256];
  for (int c = 0; c < 256; ++c) {
    da[c] = oracle_fp8_decode((uint8_t)c, fa);
    db[c] = oracle_fp8_decode((uint8_t)c, fb);
  }
  int64_t count = rows ? nrows : M;
  int64_t kg = (mode == ORC_PER_TENSOR) ? K : ORC_GROUP;
  int64_t ngroups = K / kg;
  for (int64_t r = 0; r < count; ++r) {
    int64_t m = rows ? rows[r] : r;
    const uint8_t* arow = a + m * K;
    for (int64_t nn = 0; nn < N; ++nn) {
      const uint8_t* brow = b + nn * K;
      double total = 0.0, total_abs = 0.0;
      for (int64_t g = 0; g < ngroups; ++g) {
        double s = 0.0, sabs = 0.0;
        for (int64_t k = g * kg; k < (g + 1) * kg; ++k) {
          double p = da[arow[k]] * db[brow[k]];
          s += p;
          sabs += fabs(p);
        }
        double sa_v, sb_v;
        if (mode == ORC_PER_TENSOR) {
          sa_v = sa[0];
          sb_v = sb[0];
        } else {
          sa_v = sa[m * ngroups + g];
          sb_v = sb[(nn / ORC_GROUP) * ngroups + g];
        }
        double denom = sa_v * sb_v;
        total += s / denom;
        total_abs += sabs / denom;
      }
      ref[r * N + nn] = total;
      if (absref) absref[r * N + nn] = total_abs;
    }
  }
}

/* BF16 x BF16 GEMM reference for an up-projection whose epilogue carries the
   quantizer ("Paradigma Details FP8 and Optimizer Tricks Behind NanoGPT
   Records", FP8 paragraph: the fused kernel works on the preceding
   computation's results while they are still in registers, so the
   pre-activation H never goes through memory).  ref[r, n] = sum over k of
   x[m, k] * w[n, k] with m = rows[r] (or r), summed in float64 in k order;
   every product of two BF16 values is exact in float64 (8 + 8 significant
   bits).  absref[r, n] = the same sum of |x w|. */
void oracle_gemm_bf16_f64(const uint16_t* x, const uint16_t* w, int64_t M, int64_t N, int64_t K,
                          const int64_t* rows, int64_t nrows, double* ref, double* absref) {
  int64_t count = rows ? nrows : M;
  for (int64_t r = 0; r < count; ++r) {
    int64_t m = rows ? rows[r] : r;
    const uint16_t* xr = x + m * K;
    for (int64_t n = 0; n < N; ++n) {
      const uint16_t* wr = w + n * K;
      double s = 0.0, sabs = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        double p = (double)oracle_bf16_to_f32(xr[k]) * (double)oracle_bf16_to_f32(wr[k]);
        s += p;
        sabs += fabs(p);
      }
      ref[r * N + n] = s;
      if (absref) absref[r * N + n] = sabs;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* MXFP8 ([FP8T] "Trade-offs and edge cases": the microscaling recipe gives */
/* each block of 32 adjacent values its own scale, and every scale is a     */
/* power of two).                                                            */
/* ------------------------------------------------------------------------ */
#define ORC_MX_BLOCK 32

/* Exponent k of a block's decode scale 2^k.  The pages fix only "power of
   two"; the reading taken is the Step 2 rule (scale = format max / amax)
   held to powers of two without letting the block's largest magnitude
   overflow: k is the smallest integer in the E8M0 range [-127, 127] with
   amax <= max * 2^k (a zero block gets -127).  When no k qualifies (an
   infinity or a NaN in the block) k = 127.  The comparison is exact in
   float64. */
int oracle_mx_exponent(double amax, int nonfinite, int fmt) {
  orc_format f = orc_fmt(fmt);
  if (nonfinite) return 127;
  for (int k = -127; k <= 127; ++k)
    if (amax <= ldexp(f.maxval, k)) return k;
  return 127;
}

/* One MXFP8 cast of a row-major [rows x cols] BF16 tensor, cols % 32 == 0.
   Block j of a row is elements 32 j .. 32 j + 31 of that row.  For every
   element: b = act(h) rounded to BF16 (the copy, as in oracle_quantize);
   for every block: k from the largest |b| (oracle_mx_exponent), stored as
   the E8M0 byte k + 127 in scale_e8m0[row * cols/32 + j]; each code is the
   saturating RNE cast of b * 2^-k.  The product is formed exactly in
   float64 and then narrowed to binary32, which is exact unless it lies
   below the binary32 normal range, where every FP8 code is a signed zero
   anyway.  bf16_out, fp8_out and scale_e8m0 may each be NULL. */
void oracle_quantize_mx(const uint16_t* h, int64_t rows, int64_t cols, int act, int fmt,
                        uint16_t* bf16_out, uint8_t* fp8_out, uint8_t* scale_e8m0) {
  int64_t nblocks = rows * (cols / ORC_MX_BLOCK);
  for (int64_t g = 0; g < nblocks; ++g) {
    uint16_t b[ORC_MX_BLOCK];
    double amax = 0.0;
    int nonfinite = 0;
    for (int j = 0; j < ORC_MX_BLOCK; ++j) {
      b[j] = act_bf16(h[g * ORC_MX_BLOCK + j], act);
      double v = fabs((double)oracle_bf16_to_f32(b[j]));
      if (isnan(v) || isinf(v)) nonfinite = 1;
      else if (v > amax) amax = v;
    }
    int k = oracle_mx_exponent(amax, nonfinite, fmt);
    if (scale_e8m0) scale_e8m0[g] = (uint8_t)(k + 127);
    for (int j = 0; j < ORC_MX_BLOCK; ++j) {
      if (bf16_out) bf16_out[g * ORC_MX_BLOCK + j] = b[j];
      if (fp8_out) {
        float v = (float)ldexp((double)oracle_bf16_to_f32(b[j]), -k);
        fp8_out[g * ORC_MX_BLOCK + j] = oracle_fp8_encode(v, fmt);
      }
    }
  }
}

/* Float64 reference of the MXFP8 GEMM y = a b^T, a [M x K] and b [N x K]
   codes, each with its E8M0 block bytes ([M x K/32], [N x K/32]); every
   32-wide block product is multiplied by both decode scales:
     ref[r, n] = sum_j 2^(ea[m, j] - 127) 2^(eb[n, j] - 127)
                       sum_{k in block j} dec(a[m, k]) dec(b[n, k])
   absref the same with |products|.  rows selects output rows (NULL: all). */
void oracle_gemm_mx_f64(const uint8_t* a, int fa, const uint8_t* ea, const uint8_t* b, int fb,
                        const uint8_t* eb, int64_t M, int64_t N, int64_t K, const int64_t* rows,
                        int64_t nrows, double* ref, double* absref) {
  double da[256], db[256];
  for (int c = 0; c < 256; ++c) {
    da[c] = oracle_fp8_decode((uint8_t)c, fa);
    db[c] = oracle_fp8_decode((uint8_t)c, fb);
  }
  int64_t count = rows ? nrows : M;
  int64_t nb = K / ORC_MX_BLOCK;
  for (int64_t r = 0; r < count; ++r) {
    int64_t m = rows ? rows[r] : r;
    for (int64_t n = 0; n < N; ++n) {
      double total = 0.0, total_abs = 0.0;
      for (int64_t j = 0; j < nb; ++j) {
        double s = 0.0, sabs = 0.0;
        for (int64_t k = j * ORC_MX_BLOCK; k < (j + 1) * ORC_MX_BLOCK; ++k) {
          double p = da[a[m * K + k]] * db[b[n * K + k]];
          s += p;
          sabs += fabs(p);
        }
        double x = ldexp(1.0, (int)ea[m * nb + j] - 127 + (int)eb[n * nb + j] - 127);
        total += s * x;
        total_abs += sabs * x;
      }
      ref[r * N + n] = total;
      if (absref) absref[r * N + n] = total_abs;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Backward of the squared ReLU from a cached activation ([FP8T] Step 3:    */
/* the activations kept for the backward pass may be stored in FP8 to save  */
/* memory, except a few sensitive ones).                                    */
/* ------------------------------------------------------------------------ */
#define ORC_CACHE_BF16 2

/* For A = relu(H)^2 the derivative is dA/dH = 2 relu(H) = 2 sqrt(A), so the
   backward pass needs only the cached activation a (the tensor the weight
   gradient of the next layer reads anyway), either its BF16 copy or its FP8
   codes with the inverse scale they were cast with.  Per element, binary32
   with round-to-nearest-even, one operation at a time:
     a  = cache_kind == ORC_CACHE_BF16 ? bf16(cache) : dec(code) * a_scale_inv
     r  = sqrt(a)                      (IEEE square root: NaN below zero, -0 kept)
     g  = (2 r) * dA                   (2 r is exact)
     b  = bf16_rne(g)                  -> bf16_out
     code = sat_rne(b * scale)         -> fp8_out, the gradient's delayed scale
   amax is the largest |b| (bit patterns compared as unsigned integers) and
   sat the number of saturating elements, as in oracle_quantize. */
void oracle_relu2_backward(const uint16_t* dA, const void* cache, int cache_kind,
                           float a_scale_inv, int64_t n, int fmt, float scale,
                           uint16_t* bf16_out, uint8_t* fp8_out, uint32_t* amax_bits_out,
                           uint64_t* sat_out) {
  uint32_t amax = 0;
  uint64_t sat = 0;
  for (int64_t i = 0; i < n; ++i) {
    float a;
    if (cache_kind == ORC_CACHE_BF16) {
      a = oracle_bf16_to_f32(((const uint16_t*)cache)[i]);
    } else {
      float d = (float)oracle_fp8_decode(((const uint8_t*)cache)[i], cache_kind);
      a = d * a_scale_inv;
    }
    float r = sqrtf(a);
    float two_r = 2.0f * r;
    float g = two_r * oracle_bf16_to_f32(dA[i]);
    uint16_t b = oracle_bf16_rne(g);
    if (bf16_out) bf16_out[i] = b;
    uint32_t mag = ((uint32_t)(b & 0x7FFF)) << 16;
    if (mag > amax) amax = mag;
    float v = oracle_bf16_to_f32(b) * scale;
    if (fp8_out) fp8_out[i] = oracle_fp8_encode(v, fmt);
    sat += (uint64_t)oracle_fp8_saturates(v, fmt);
  }
  if (amax_bits_out) *amax_bits_out = amax;
  if (sat_out) *sat_out = sat;
}

/* ------------------------------------------------------------------------ */
/* Batch helpers (the per-element functions above applied to arrays).        */
/* ------------------------------------------------------------------------ */
void oracle_fp8_encode_batch(const float* x, int64_t n, int fmt, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_fp8_encode(x[i], fmt);
}

void oracle_fp8_saturates_batch(const float* x, int64_t n, int fmt, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)oracle_fp8_saturates(x[i], fmt);
}

void oracle_bf16_rne_batch(const float* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_rne(x[i]);
}

void oracle_scale_batch(const float* amax, int64_t n, float margin, int fmt, float* scale,
                        float* scale_inv) {
  for (int64_t i = 0; i < n; ++i) {
    scale[i] = oracle_scale_from_amax(amax[i], margin, fmt);
    if (scale_inv) scale_inv[i] = oracle_recip_f32(scale[i]);
  }
}

/* Encode every binary32 bit pattern in [lo, hi) (as uint32 values) and
   write the codes; used to compare a device cast against all 2^32 inputs
   in chunks. */
void oracle_fp8_encode_range(uint64_t lo, uint64_t hi, int fmt, uint8_t* out) {
  for (uint64_t u = lo; u < hi; ++u) out[u - lo] = oracle_fp8_encode(u2f((uint32_t)u), fmt);
}

void oracle_bf16_rne_range(uint64_t lo, uint64_t hi, uint16_t* out) {
  for (uint64_t u = lo; u < hi; ++u) out[u - lo] = oracle_bf16_rne(u2f((uint32_t)u));
}
