/*
 * fp8dp.h -- C ABI of libfp8dp.so: scaled FP8 quantization for an MLP
 * down-projection on AMD Instinct MI355X (gfx950).
 *
 * What the library computes (pages cited by title and section):
 *
 *  - "Paradigma Details FP8 and Optimizer Tricks Behind NanoGPT Records",
 *    the FP8 section: one fused kernel applies the activation, writes the BF16
 *    copy the backward pass needs, emits the FP8 copy and keeps small running
 *    maxima, so the large tensor is never read again; the scale uses the
 *    previous step's maximum times a safety margin (delayed scaling); the
 *    down-projection then runs in FP8 in the forward pass only.
 *  - "FP8 training: what it is and how it works", Step 1 (E4M3 max 448,
 *    E5M2 max 57344), Step 2 (scale = format max / amax, applied before
 *    rounding and divided out afterwards), Step 3 (FP8 inputs, wide
 *    accumulation), Trade-offs (delayed scaling keeps a history of amaxes;
 *    1 x 128 activation tiles and 128 x 128 weight blocks).
 *  - "FP8 Training & Inference", FP8 Formats (E4M3 for weights/activations,
 *    E5M2 for gradients), Per-Tensor Scaling (scales factored out of the
 *    matmul, output rescaled), Delayed Scaling (detect overflow).
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless marked (host).  The caller owns all
 *    memory; the library never allocates device memory.
 *  - Every call is enqueued on `stream` and returns without waiting for the
 *    GPU; outputs are valid once the stream reaches the call.
 *  - Return value: 0 on success, FP8DP_EINVAL (-1) for an invalid argument,
 *    FP8DP_EUNSUPPORTED (-2) for an unsupported combination, FP8DP_EHIP (-3)
 *    when a HIP launch fails.  fp8dp_last_error() describes the last failure
 *    of the calling thread.  Nothing is enqueued when a call fails argument
 *    checks.
 *  - BF16 values are passed as uint16_t bit patterns, FP8 values as uint8_t
 *    codes (OCP E4M3 "fn" or OCP E5M2), scales as IEEE binary32.
 *  - Matrices are row-major.  Vector I/O needs every tensor pointer to be
 *    16-byte aligned.
 */
#ifndef FP8DP_H
#define FP8DP_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8DP_OK 0
#define FP8DP_EINVAL (-1)
#define FP8DP_EUNSUPPORTED (-2)
#define FP8DP_EHIP (-3)

/* OCP E4M3 (1/4/3 bits, bias 7, max 448, no infinity, NaN = S.1111.111) and
   OCP E5M2 (1/5/2 bits, bias 15, max 57344, with infinities). */
typedef enum { FP8DP_E4M3 = 0, FP8DP_E5M2 = 1 } fp8dp_format;

/* Activation applied before the copies are written.  RELU2: a = h*h for
   h > 0, else +0 (NaN and -0 give +0), rounded to BF16 nearest-even.
   IDENTITY: the input value unchanged. */
typedef enum { FP8DP_ACT_IDENTITY = 0, FP8DP_ACT_RELU2 = 1 } fp8dp_act;

/* PER_TENSOR: one multiplier for the whole tensor, read from the delayed-
   scaling state.  PER_GROUP128: each run of 128 consecutive elements of a row
   gets its own multiplier max / amax_group computed in the kernel (current
   scaling, no margin); weights use 128 x 128 blocks. */
typedef enum { FP8DP_PER_TENSOR = 0, FP8DP_PER_GROUP128 = 1 } fp8dp_scale_mode;

/* How the GEMM sums products.
   MFMA_FP8: the FP8 matrix instructions.  Measured on gfx950, they sum
   products in groups of 8 consecutive k, each product truncated toward zero
   to a multiple of 2^(E-13), where E is the largest exponent sum e_a + e_b in
   its group.  Products within 7 binades of the group's largest are exact.
   Group sums and the FP32 accumulator are combined at FP32 precision.  This
   is the same kind of limited tensor-core accumulation that "FP8 training:
   what it is and how it works", Step 3, reports for another GPU.
   EXACT: FP8 operands are widened to FP16 in registers (every E4M3 and E5M2
   value is exact in FP16) and summed by the FP16 matrix instructions with
   FP32-accurate accumulation, at the FP16 instruction rate. */
typedef enum { FP8DP_ACCUM_MFMA_FP8 = 0, FP8DP_ACCUM_EXACT = 1 } fp8dp_accum;

#define FP8DP_MAX_HIST 16
#define FP8DP_ACC_SLOTS 64

/* One running-accumulator slot (64 bytes).  Quantization calls fold their
   results into slot (block index % FP8DP_ACC_SLOTS) with one atomic max and
   one atomic add per thread block; amax_history_update reduces the slots. */
typedef struct fp8dp_acc_slot {
  uint32_t amax;      /* binary32 bits of the running max |b| (unsigned compare) */
  uint32_t ticket;    /* quantize_fused_update: workgroups folded into this slot so far */
  uint64_t sat;       /* running count of saturating elements */
  uint8_t reserved[48];
} fp8dp_acc_slot;

/* Delayed-scaling state of one tensor (4288 bytes, 64-byte aligned, in
   device memory; allocate it, e.g. as a uint8 tensor, and initialise it with
   fp8dp_state_init).  It is plain data: copying it out and back resumes the
   scaling sequence exactly. */
typedef struct fp8dp_tensor_state {
  float scale;            /* multiplier the next PER_TENSOR cast uses            */
  float scale_inv;        /* binary32 1/scale                                     */
  float scale_inv_used;   /* 1/scale of the step most recently consumed           */
  uint32_t overflow;      /* 1 when the step most recently consumed saturated     */
  uint64_t sat_last;      /* saturation count of that step                        */
  float amax_last;        /* amax of that step                                    */
  float margin;           /* safety margin (1.0 = plain current-style scale)      */
  int32_t hist_len;       /* 1 .. FP8DP_MAX_HIST amax values kept                  */
  int32_t hist_pos;       /* ring position of the next history write              */
  uint32_t steps;         /* steps consumed so far                                */
  int32_t fmt;            /* fp8dp_format the state was initialised for           */
  float history[FP8DP_MAX_HIST];
  uint32_t ticket;        /* quantize_fused_update: slots whose workgroups have all folded */
  uint8_t reserved[76];   /* pads the header to 192 bytes: acc starts on a 64-byte line */
  fp8dp_acc_slot acc[FP8DP_ACC_SLOTS];   /* running accumulators of the current step */
} fp8dp_tensor_state;

/* Size in bytes of fp8dp_tensor_state (for callers allocating raw bytes). */
int64_t fp8dp_state_size(void);

/* Initialise a state for delayed scaling ("Paradigma ...": each step casts
   with the scale derived from the previous step's amax times a safety margin;
   "FP8 training ...", Trade-offs and edge cases: the amax kept over a stored
   history window).  The pages leave the first step's amax open; it is taken
   as initial_amax here: history filled with initial_amax, accumulators
   zeroed, scale = max / (initial_amax * margin) (1.0 if that is not a
   positive finite number), scale_inv = 1/scale.  Runs as a one-thread kernel
   on `stream`.
   Errors: EINVAL for st == NULL, misaligned st, bad fmt, hist_len outside
   1..FP8DP_MAX_HIST, or a margin that is not positive and finite. */
int fp8dp_state_init(fp8dp_tensor_state* st, fp8dp_format fmt, int32_t hist_len, float margin,
                     float initial_amax, hipStream_t stream);

/* The fused quantizer (the Paradigma FP8 kernel; "FP8 training ...", Step 2).
 *   h        [rows x cols] BF16 input (pre-activation), contiguous
 *   act      activation applied first
 *   fmt      FP8 output format
 *   mode     PER_TENSOR: every element b is cast as sat_rne(b * st->scale)
 *            PER_GROUP128: cols % 128 == 0; group g (128 consecutive elements
 *            of a row) is cast with s_g = max / amax_g and
 *            group_scale_inv[g] = 1/s_g is written, [rows x cols/128] row-major
 *   st       PER_TENSOR: required (its scale is read); PER_GROUP128: optional.
 *            When given, the call folds max |b| and the number of saturating
 *            elements into st's running accumulators (consumed by
 *            amax_history_update), so several calls may form one step.
 *   bf16_out [rows x cols] BF16 copy of the activation output, or NULL
 *   fp8_out  [rows x cols] FP8 codes, or NULL (an amax-only scan)
 * The cast is binary32 b * s rounded to nearest-even, then FP8 rounding to
 * nearest-even with saturation to +-max (infinity included); NaN stays NaN
 * (0x7F | sign).  An element "saturates" when a cast without saturation would
 * have overflowed (E4M3: |b*s| > 464; E5M2: |b*s| >= 61440).
 * Errors: EINVAL for NULL h, rows or cols < 1, misaligned pointers, missing
 * st in PER_TENSOR mode, cols % 128 != 0 or a NULL group_scale_inv in
 * PER_GROUP128 mode with fp8_out given. */
int quantize_fused(const uint16_t* h, int64_t rows, int64_t cols, fp8dp_act act,
                   fp8dp_format fmt, fp8dp_scale_mode mode, fp8dp_tensor_state* st,
                   uint16_t* bf16_out, uint8_t* fp8_out, float* group_scale_inv,
                   hipStream_t stream);

/* Close a step of delayed scaling ("Paradigma ...": previous step's amax times
 * a safety margin; "FP8 training ...", Trade-offs: a stored amax history;
 * "FP8 Training & Inference", Delayed Scaling: detect overflow).  One
 * single-wave kernel, no host round trip:
 *   amax_t = max of the accumulator slots; history[hist_pos] = amax_t;
 *   scale_inv_used = scale_inv (the inverse of the scale step t was cast with);
 *   scale = max / (max(history) * margin) (1.0 when not a positive finite
 *   number), scale_inv = 1/scale; sat_last = sum of the slots;
 *   overflow = sat_last > 0; amax_last = amax_t; slots cleared; steps += 1.
 * Errors: EINVAL for a NULL or misaligned st. */
int amax_history_update(fp8dp_tensor_state* st, hipStream_t stream);

/* quantize_fused in PER_TENSOR mode followed by amax_history_update, in one
 * launch: the workgroup that folds its (amax, count) last -- counted with one
 * atomic per workgroup on the slot's ticket and one per slot on st->ticket --
 * closes the step ("Paradigma ...": the scale for the next step comes from
 * this step's amax; delayed scaling removes the wait for it).  Outputs and
 * the state after the call are bit for bit those of the two calls in
 * sequence; a GEMM on this step's codes then takes &st->scale_inv_used (the
 * inverse of the scale the codes were cast with).  The call ends the step:
 * amax and counts folded by earlier quantize_fused calls of the same step are
 * included.  Tickets are left at zero for the next call; calls that overlap
 * on one state race.
 * Errors: as quantize_fused in PER_TENSOR mode (st is required). */
int quantize_fused_update(const uint16_t* h, int64_t rows, int64_t cols, fp8dp_act act,
                          fp8dp_format fmt, fp8dp_tensor_state* st, uint16_t* bf16_out,
                          uint8_t* fp8_out, hipStream_t stream);

/* Scaled FP8 x FP8 GEMM with FP32 accumulation and BF16 output ("FP8
 * training ...", Step 3; "FP8 Training & Inference", Per-Tensor Scaling):
 *   a [M x K] codes (format fa), b [N x K] codes (format fb), the weight in
 *   the layout of a linear layer (K contiguous), y [M x N] BF16.
 *   PER_TENSOR : y = bf16_rne(sum_k dec(a) dec(b) * a_scale_inv[0] * b_scale_inv[0])
 *   PER_GROUP128: y = bf16_rne(sum_g (sum_{k in g} dec(a) dec(b))
 *                              * a_scale_inv[m, g] * b_scale_inv[n/128, g]),
 *                 a_scale_inv [M x K/128], b_scale_inv [N/128 x K/128]
 *                 (each 128-wide partial sum is promoted into the FP32
 *                 accumulator with its scales, as the FP32 promotion every
 *                 128 elements of Step 3 describes).
 * accum selects how products are summed (fp8dp_accum above).
 * For delayed scaling, pass &st_a->scale_inv when the GEMM is enqueued before
 * amax_history_update of that step, or &st_a->scale_inv_used after it.
 * M is any positive row count (the number of tokens need not fill a tile);
 * N and K are multiples of 128.  Only rows 0 .. M-1 of y are written.
 * Errors: EINVAL for NULL pointers, M < 1, N or K not positive multiples of
 * 128, misaligned pointers, bad formats, mode or accum. */
int fp8_gemm_scaled(const uint8_t* a, fp8dp_format fa, const uint8_t* b, fp8dp_format fb,
                    int64_t M, int64_t N, int64_t K, fp8dp_scale_mode mode, fp8dp_accum accum,
                    const float* a_scale_inv, const float* b_scale_inv, uint16_t* y,
                    hipStream_t stream);

/* The same GEMM (per-tensor scales) with K split
 * over `splits` workgroups per output tile, for outputs too small to fill the
 * GPU on their own -- the weight-gradient GEMM of the FP8 recipe ("FP8
 * Training & Inference", FP8 Training Recipe) has a [N x K] output and a
 * contraction over all tokens.  With KS = K/128 blocks of 128 k, split s
 * sums the blocks [floor(s KS/splits), floor((s+1) KS/splits)) into
 * workspace[s][m][n] (FP32, unscaled); a second kernel adds
 * the splits in order s = 0, 1, ... and writes
 *   y = bf16_rne((sum_s workspace[s]) * a_scale_inv[0] * b_scale_inv[0]),
 * so the result is deterministic; with splits = 1 it equals fp8_gemm_scaled
 * with the same accum bit for bit.  accum as in fp8_gemm_scaled.
 * workspace: caller-owned device memory of splits * M * N floats, 16-byte
 * aligned; its contents are overwritten.
 * Errors: EINVAL for NULL pointers, splits outside 1..64, M not a positive
 * multiple of 256, N or K not of 128, K < 128 * splits, misaligned pointers,
 * a bad format or accum. */
int fp8_gemm_scaled_splitk(const uint8_t* a, fp8dp_format fa, const uint8_t* b, fp8dp_format fb,
                           int64_t M, int64_t N, int64_t K, int32_t splits, fp8dp_accum accum,
                           const float* a_scale_inv, const float* b_scale_inv, float* workspace,
                           uint16_t* y, hipStream_t stream);

/* fp8_gemm_scaled_splitk without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * The split partials go to a device array of 16 Mi floats (64 MiB) inside
 * the library, one per GPU, held until the process ends; its device address
 * is resolved on the first call on each device (hipGetSymbolAddress, no
 * allocation).  Same arguments, kernels and result as fp8_gemm_scaled_splitk
 * (bit for bit), minus the workspace.  Nothing in the array needs clearing:
 * each call writes every partial it reads.  Every call on a GPU shares that
 * GPU's array: calls that overlap on one GPU (on different streams, or from
 * several threads) race and must be serialized by the caller.
 * The stream must belong to the current device (the array's address is
 * that device's).
 * Errors: those of fp8_gemm_scaled_splitk; EINVAL when splits * M * N
 * exceeds 16 Mi floats or the stream belongs to another device; EHIP when
 * no device is current or the array's address cannot be resolved. */
int fp8_gemm_scaled_splitk_noalloc(const uint8_t* a, fp8dp_format fa, const uint8_t* b,
                                   fp8dp_format fb, int64_t M, int64_t N, int64_t K,
                                   int32_t splits, fp8dp_accum accum, const float* a_scale_inv,
                                   const float* b_scale_inv, uint16_t* y, hipStream_t stream);

/* quantize_fused in PER_TENSOR mode (delayed scale from st, accumulators into
 * st's slots, amax_history_update closes the step as usual) that also writes
 * its codes transposed: fp8_t_out[c * rows + r] = code(r, c), the [cols x rows]
 * operand layout of the weight-gradient GEMM ("FP8 Training & Inference", FP8
 * Training Recipe: dW = dY^T X; this GEMM contracts along the contiguous
 * dimension of both operands).  One more byte written per element replaces a
 * separate fp8_transpose pass.  The codes, BF16 copy, amax and saturation
 * count are quantize_fused's, bit for bit.
 *   fp8_t_out: required, [cols x rows] bytes; bf16_out, fp8_out: optional
 *   ([rows x cols], as in quantize_fused).
 * Errors: EINVAL for NULL h, st or fp8_t_out, rows not a positive multiple
 * of 64 or cols of 128, misaligned (16 bytes) pointers, a bad format or
 * activation. */
int quantize_fused_transposed(const uint16_t* h, int64_t rows, int64_t cols, fp8dp_act act,
                              fp8dp_format fmt, fp8dp_tensor_state* st, uint16_t* bf16_out,
                              uint8_t* fp8_out, uint8_t* fp8_t_out, hipStream_t stream);

/* dst [cols x rows] = src [rows x cols] transposed, bytes (FP8 codes): the
 * operand layouts of the backward GEMMs (dgrad needs W^T, wgrad dY^T and
 * X^T).  The codes and their scale are unchanged.
 * Errors: EINVAL for NULL or misaligned (16 bytes) pointers, src == dst, or
 * rows / cols not positive multiples of 64 (or more than 2^31 - 1 tiles of
 * 64 x 64). */
int fp8_transpose(const uint8_t* src, int64_t rows, int64_t cols, uint8_t* dst,
                  hipStream_t stream);

/* Which form the activation kept for the backward pass takes: FP8 codes
 * (with the inverse scale they were cast with) or the BF16 copy. */
typedef enum { FP8DP_CACHE_E4M3 = 0, FP8DP_CACHE_E5M2 = 1, FP8DP_CACHE_BF16 = 2 } fp8dp_cache;

/* Backward of the squared ReLU from the cached activation, fused with the
 * gradient's FP8 cast ("FP8 training ...", Step 3: the activations kept for
 * the backward pass may be stored in FP8, except a few sensitive ones).
 * For A = relu(H)^2, dH = dA * 2 relu(H) = dA * 2 sqrt(A):
 *   dA        [rows x cols] BF16, the gradient of A (e.g. the dgrad GEMM's output)
 *   a_cache   [rows x cols] the cached A: FP8 codes (cache = E4M3 / E5M2) or
 *             BF16 (cache = BF16)
 *   a_scale_inv  device pointer to the inverse scale the codes were cast
 *             with (FP8 caches; e.g. &st_a->scale_inv_used after the forward
 *             step's amax_history_update), ignored for BF16
 *   per element, binary32 nearest-even one operation at a time:
 *     a = BF16 ? bf16(a_cache) : dec(code) * a_scale_inv; g = (2 sqrt(a)) * dA
 *     (IEEE square root: a negative or NaN a gives NaN, whose sign is not
 *     specified); b = bf16_rne(g) -> bf16_out (may be NULL);
 *     fp8_out = sat_rne(b * st->scale) in format fmt (E5M2 in the FP8
 *     recipe), max |b| and the saturation count folded into st's
 *     accumulators (consumed by amax_history_update), as quantize_fused.
 * Errors: EINVAL for NULL dA / a_cache / st / fp8_out, a NULL a_scale_inv with
 * an FP8 cache, rows or cols < 1, misaligned pointers (16 bytes; the scale 4),
 * or an unknown cache kind or format. */
int relu2_backward_quantize(const uint16_t* dA, const void* a_cache, fp8dp_cache cache,
                            const float* a_scale_inv, int64_t rows, int64_t cols,
                            fp8dp_format fmt, fp8dp_tensor_state* st, uint16_t* bf16_out,
                            uint8_t* fp8_out, hipStream_t stream);

/* The FP8 recipe's dgrad GEMM with the squared ReLU's backward in its
 * epilogue ("FP8 training ...", Step 3: activations kept for the backward
 * pass in FP8; "FP8 Training & Inference", FP8 Training Recipe: E5M2
 * gradients x E4M3 weights).  Equal, bit for bit, to
 *   fp8_gemm_scaled(a, E5M2, b, E4M3, M, N, K, PER_TENSOR, accum,
 *                   a_scale_inv, b_scale_inv, dA)           (dA [M x N] BF16)
 *   relu2_backward_quantize(dA, act_cache, cache, act_scale_inv, M, N, fmt,
 *                           st, NULL, dh_out)
 * without dA's write and read: dh_out [M x N] codes in format fmt cast with
 * st->scale, amax and saturation count folded into st.  a [M x K] is dY8, b
 * [N x K] the weight codes transposed (W8^T), act_cache [M x N] the FP8 codes
 * of the activation A with act_scale_inv the inverse scale they were cast
 * with.
 * Errors: EINVAL for NULL pointers, M not a positive multiple of 256, N or K
 * not of 128, misaligned pointers (16 bytes; scales 4), unknown formats or
 * accum; EUNSUPPORTED for operand formats other than E5M2 x E4M3 or a BF16
 * cache. */
int fp8_gemm_relu2_backward(const uint8_t* a, fp8dp_format fa, const uint8_t* b, fp8dp_format fb,
                            int64_t M, int64_t N, int64_t K, fp8dp_accum accum,
                            const float* a_scale_inv,
                            const float* b_scale_inv, const uint8_t* act_cache, fp8dp_cache cache,
                            const float* act_scale_inv, fp8dp_format fmt, fp8dp_tensor_state* st,
                            uint8_t* dh_out, hipStream_t stream);

/* Recompute after an overflow ("FP8 Training & Inference", Delayed Scaling:
 * a step whose delayed scale was too large is detected and recomputed with a
 * corrected scale).  Enqueue after amax_history_update of the step: when that
 * update set st->overflow, fp8_out = sat_rne(b * st->scale) for every element
 * (b = bf16_rne(act(h)), st->scale now computed from a history that includes
 * the step's own amax); when it did not, the kernel returns at once and
 * fp8_out is untouched.  The decision is taken on the GPU (no host round
 * trip).  The BF16 copy is not rewritten (it does not depend on the scale),
 * and nothing is folded into st.  Same shapes and alignment as
 * quantize_fused in PER_TENSOR mode.
 * Errors: EINVAL for NULL h / st / fp8_out, rows or cols < 1, misaligned
 * pointers, or an unknown act / fmt. */
int quantize_recompute(const uint16_t* h, int64_t rows, int64_t cols, fp8dp_act act,
                       fp8dp_format fmt, const fp8dp_tensor_state* st, uint8_t* fp8_out,
                       hipStream_t stream);

/* fp8_gemm_scaled (PER_TENSOR, the given accum) that runs only when
 * *run_flag != 0, read on the GPU -- the GEMM half of the recompute above:
 * pass &st->overflow of the operand whose cast overflowed and
 * &st->scale_inv (the corrected scale's inverse).  With *run_flag == 0 y is
 * untouched.  Any M >= 1, as fp8_gemm_scaled; N and K multiples of 128.
 * Errors: EINVAL for NULL pointers, M < 1, N or K not positive multiples of
 * 128, misaligned pointers (operands 16 bytes, scales and flag 4), or a bad
 * format or accum. */
int fp8_gemm_scaled_if(const uint8_t* a, fp8dp_format fa, const uint8_t* b, fp8dp_format fb,
                       int64_t M, int64_t N, int64_t K, fp8dp_accum accum,
                       const float* a_scale_inv,
                       const float* b_scale_inv, uint16_t* y, const uint32_t* run_flag,
                       hipStream_t stream);

/* MXFP8 cast ("FP8 training ...", Trade-offs and edge cases: the
 * microscaling recipe gives each block of 32 adjacent values its own scale,
 * a power of two).  h [rows x cols] BF16 (cols % 32 == 0); block j of a row
 * is its elements 32 j .. 32 j + 31.
 *   b = bf16_rne(act(h)) -> bf16_out (may be NULL)
 *   per block: k = the smallest integer in [-127, 127] with
 *     |b| <= max * 2^k for all 32 elements (zero blocks: -127; a block with
 *     an infinity or NaN: 127), written as the E8M0 byte k + 127 to
 *     scale_out[row * cols/32 + j] (decode scale 2^(byte - 127))
 *   codes: fp8_out = sat_rne(b * 2^-k) (finite values never saturate).
 * No scaling state is read or written.  Pointers are device pointers owned
 * by the caller; nothing is allocated.
 * Errors: EINVAL for NULL h / fp8_out / scale_out, rows < 1, cols not a
 * positive multiple of 32, h, bf16_out or fp8_out not 16-byte aligned, or an
 * unknown act / fmt. */
int quantize_mx(const uint16_t* h, int64_t rows, int64_t cols, fp8dp_act act, fp8dp_format fmt,
                uint16_t* bf16_out, uint8_t* fp8_out, uint8_t* scale_out, hipStream_t stream);

/* quantize_mx with the blocks of 32 running down the columns, its codes and
 * exponents written transposed ("FP8 training: what it is and how it works",
 * Trade-offs and edge cases, for the GEMMs that contract along the token
 * dimension or along a weight's output features: the weight gradient
 * dW = dY^T X takes dY and X this way, the input gradient dX = dY W takes W).
 * h [rows x cols] BF16; block j of column c is its rows 32 j .. 32 j + 31:
 *   b = bf16_rne(act(h)) -> bf16_out [rows x cols], row-major (may be NULL)
 *   per block: k by quantize_mx's rule, E8M0 byte k + 127 ->
 *     scale_t_out[c * rows/32 + j]
 *   codes: fp8_t_out[c * rows + r] = sat_rne(b[r][c] * 2^-k)
 * i.e. exactly quantize_mx applied to act(h) transposed.  Device pointers
 * owned by the caller; nothing is allocated.
 * Errors: EINVAL for NULL h / fp8_t_out / scale_t_out, rows not a positive
 * multiple of 64 or cols of 128, h, bf16_out or fp8_t_out not 16-byte
 * aligned, or an unknown act / fmt. */
int quantize_mx_transposed(const uint16_t* h, int64_t rows, int64_t cols, fp8dp_act act,
                           fp8dp_format fmt, uint16_t* bf16_out, uint8_t* fp8_t_out,
                           uint8_t* scale_t_out, hipStream_t stream);

/* MXFP8 GEMM: a [M x K] codes (format fa) with E8M0 block exponents a_scale
 * [M x K/32], b [N x K] codes (format fb) with b_scale [N x K/32] (the output
 * of quantize_mx on each operand), y [M x N] BF16:
 *   y = bf16_rne( sum_j 2^(a_scale[m, j] - 127) 2^(b_scale[n, j] - 127)
 *                       sum_{k in block j} dec(a[m, k]) dec(b[n, k]) )
 * with FP32 accumulation, one scale pair per 32-value block.
 * accum = ACCUM_EXACT: each row's block exponents are folded into the FP16
 *   widening of its codes, relative to the row's largest exponent (exact while
 *   a tile's rows span at most 22 binades, E4M3, or 8, E5M2, which a scan of
 *   the tile's exponents checks); a tile past that takes a fallback that sums
 *   each block on its own and adds it scaled by its two exponents (exact for
 *   any exponents, slower).  FP16 products, FP32 sums: |err| <= 2^-8 |ref| +
 *   1e-5 sum|ab| on every output.
 * accum = ACCUM_MFMA_FP8: the block scales are applied by gfx950's microscaled
 *   FP8 matrix instructions, which truncate small products as the unscaled
 *   ones do (see fp8dp_accum).
 * Errors: EINVAL for NULL pointers, M not a positive multiple of 256, N or K
 * not of 128, a, b or y not 16-byte aligned, exponent arrays not 4-byte
 * aligned, or a bad format or accum. */
int fp8_gemm_mx(const uint8_t* a, fp8dp_format fa, const uint8_t* a_scale, const uint8_t* b,
                fp8dp_format fb, const uint8_t* b_scale, int64_t M, int64_t N, int64_t K,
                fp8dp_accum accum, uint16_t* y, hipStream_t stream);

/* fp8_gemm_mx with K split over `splits` workgroups per output tile, for the
 * shapes whose output has too few tiles to fill the GPU: the MX weight
 * gradient dW [N x K] = dY^T X contracts along the tokens ("FP8 Training &
 * Inference", FP8 Training Recipe; blocks along the tokens from
 * quantize_mx_transposed).  Split s sums the 128-wide K blocks
 * floor(s KS / splits) .. floor((s + 1) KS / splits) - 1 (KS = K / 128) into
 * FP32 partials in workspace (at least splits * M * N floats, caller-owned,
 * 16-byte aligned), with the block scales already applied; a second kernel
 * adds the partials in split order and rounds to BF16 (deterministic).  The
 * accumulation modes are fp8_gemm_mx's (exact mode: each split folds the
 * block exponents of its own range); one split gives fp8_gemm_mx's output
 * bit for bit.
 * Errors: those of fp8_gemm_scaled_splitk (shapes: M a positive multiple of
 * 256, N and K of 128, K >= 128 * splits, 1 <= splits <= 64), plus NULL or
 * misaligned (4 bytes) exponent arrays. */
int fp8_gemm_mx_splitk(const uint8_t* a, fp8dp_format fa, const uint8_t* a_scale,
                       const uint8_t* b, fp8dp_format fb, const uint8_t* b_scale, int64_t M,
                       int64_t N, int64_t K, int32_t splits, fp8dp_accum accum, float* workspace,
                       uint16_t* y, hipStream_t stream);

/* Weight cast with current scaling ("FP8 training ...", Step 4: the 8-bit
 * copies are cast from the master weights at every step; Trade-offs: 128 x
 * 128 weight blocks).  w [N x K] BF16 -> w8 [N x K] codes.
 *   PER_TENSOR : scale_out is 2 floats: [0] = 1/s, [1] = s, s = max / amax(w)
 *   PER_GROUP128: N % 128 == K % 128 == 0; block (i, j) = rows 128i.., cols
 *                 128j.. is cast with s_ij = max / amax_ij and
 *                 scale_out[i * (K/128) + j] = 1/s_ij.
 * Errors: EINVAL for NULL pointers, bad sizes or alignment. */
int quantize_weight(const uint16_t* w, int64_t N, int64_t K, fp8dp_format fmt,
                    fp8dp_scale_mode mode, uint8_t* w8, float* scale_out, hipStream_t stream);

/* Up-projection BF16 GEMM with the quantizer in its epilogue ("Paradigma
 * Details FP8 and Optimizer Tricks Behind NanoGPT Records", FP8 paragraph:
 * the fused kernel handles the preceding computation's results while they
 * are still in registers, so the intermediate is neither written out nor
 * read back).
 *   x [M x K] BF16 (the MLP input), w [N x K] BF16 (the up-projection weight
 *   in linear-layer layout); H = bf16_rne(x w^T) with FP32 accumulation
 *   (the BF16 matrix instructions; products are exact in FP32).
 *   fp8_out != NULL: the epilogue applies quantize_fused(H, act, fmt,
 *     PER_TENSOR, st, bf16_out, fp8_out) element for element: b =
 *     bf16_rne(act(H)) to bf16_out (may be NULL), fp8_out [M x N] codes cast
 *     with st->scale, running amax of |b| and the saturation count folded
 *     into st's accumulator slots (amax_history_update consumes them).
 *     h_out [M x N] BF16 receives H when non-NULL.
 *   fp8_out == NULL: the plain GEMM, H to h_out (required); bf16_out and st
 *     must be NULL.
 * All pointers are device pointers owned by the caller; nothing is allocated.
 * Errors: EINVAL for NULL x or w, M not a positive multiple of 256, N of 128
 * or K of 64, misaligned pointers (16 bytes), a missing state with fp8_out,
 * or an unknown act / fmt. */
int gemm_bf16_quantize_fused(const uint16_t* x, const uint16_t* w, int64_t M, int64_t N,
                             int64_t K, fp8dp_act act, fp8dp_format fmt, fp8dp_tensor_state* st,
                             uint16_t* h_out, uint16_t* bf16_out, uint8_t* fp8_out,
                             hipStream_t stream);

/* (host) Message for the last failing call on this thread ("" if none). */
const char* fp8dp_last_error(void);

/* ---------------------------------------------------------------------------
 * Comparison and diagnostic entry points.
 *
 * The naive three-pass quantizer the Paradigma page contrasts with the fused
 * kernel (write the whole intermediate, scan it for the max, read it again to
 * convert): a caller runs fp8dp_bench_act_bf16, fp8dp_bench_amax,
 * amax_history_update (margin 1, history 1: current scaling) and
 * fp8dp_bench_cast.  n is the element count; all pointers 16-byte aligned.
 * ------------------------------------------------------------------------- */
/* Pass 1: out = bf16(act(h)); no amax. */
int fp8dp_bench_act_bf16(const uint16_t* h, int64_t n, fp8dp_act act, uint16_t* out,
                         hipStream_t stream);
/* Pass 2: fold max |x| into st's accumulators (x read once). */
int fp8dp_bench_amax(const uint16_t* x, int64_t n, fp8dp_tensor_state* st, hipStream_t stream);
/* Pass 3: out = sat_rne(x * st->scale), saturation count folded into st. */
int fp8dp_bench_cast(const uint16_t* x, int64_t n, fp8dp_format fmt, fp8dp_tensor_state* st,
                     uint8_t* out, hipStream_t stream);
/* Plain 16-byte-vector device copy (bandwidth ceiling and counter
   calibration); bytes % 16 == 0. */
int fp8dp_bench_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);

/* Device conversion routines applied to arbitrary binary32 inputs, for
 * exhaustive comparison with a reference.  target 0: E4M3 codes (uint8 out),
 * 1: E5M2 codes (uint8 out), 2: BF16 round-to-nearest-even (uint16 out).
 * 3: saturation predicate for E4M3, 4: for E5M2 (uint8 0/1 out), 5: the
 * binary32 square root the activation backward uses (float out). */
int fp8dp_convert_f32(const float* x, int64_t n, int32_t target, void* out, hipStream_t stream);

/* Device scale rule on n amax values: scale[i] = max / (amax[i] * margin)
   with the fallback to 1, scale_inv[i] = 1/scale[i]. */
int fp8dp_scale_rule(const float* amax, int64_t n, float margin, fp8dp_format fmt, float* scale,
                     float* scale_inv, hipStream_t stream);

/* (host) Process-wide tuning and diagnostic switches; they change how the
   work is scheduled or which bit-exact conversion routine runs, never the
   results.  grid_limit: maximum thread blocks of the element-wise kernels
   (0 = automatic).  codec: 0 = hardware conversion instructions, 1 = integer
   bit-manipulation routines.  Return the previous value. */
int32_t fp8dp_set_grid_limit(int32_t blocks);
int32_t fp8dp_set_codec(int32_t codec);

#ifdef __cplusplus
}
#endif
#endif /* FP8DP_H */
