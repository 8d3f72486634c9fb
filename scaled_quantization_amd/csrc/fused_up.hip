// fused_up.hip -- BF16 GEMM of the MLP up-projection with the quantizer in its
// epilogue.
//
// "Paradigma Details FP8 and Optimizer Tricks Behind NanoGPT Records", FP8
// paragraph: instead of writing the intermediate tensor out and reading it
// back to scan its maximum and to convert it, one kernel produces the BF16
// copy the backward pass needs, the FP8 copy and the running maxima while the
// preceding computation's results are still in registers.  Here the preceding
// computation is the up-projection H = X W1^T, so H itself never goes to
// memory: each output tile leaves the MFMA accumulators as
//   h = bf16_rne(acc)            (the value H would have had in memory)
//   b = bf16_rne(act(h))         -> BF16 copy
//   v = fp32(b * s); q = sat_rne_fp8(v)  -> FP8 copy, s the delayed scale
//   amax = max |b|, count of saturating v  -> the state's accumulator slots
// which is, element for element, quantize_fused applied to bf16(X W1^T).
//
// Kernel (gfx950): the large-tile pipeline of the FP8 GEMM (gemm_core.hpp)
// with BF16 operands: a 128-byte LDS row holds 64 BF16 values of K, and each
// 64-value half stage is two k steps of v_mfma_f32_32x32x16_bf16, which take
// the same MFMA cycles per stage as the FP8 instruction.  512 threads (8
// waves, two per SIMD) own a 256 x BN tile (BN = 128, 192, or 256 for the
// plain GEMM); wave w owns 64 x BN/2 as 2 x TN MFMA tiles.  The grid is
// persistent: a workgroup runs its tiles back to back in one pipeline.
#include <hip/hip_runtime.h>

#include "codec.hpp"
#include "common.hpp"
#include "gemm_core.hpp"
#include "quant_core.hpp"

namespace fp8dp {

typedef __bf16 v8bf_t __attribute__((ext_vector_type(8)));

// Output path.  The MFMA is issued with the weight fragment first, so a
// 32 x 32 accumulator tile holds Y^T: lane l has row l % 32 of the tile and
// register r column 8 (r / 4) + 4 (l / 32) + r % 4 -- runs of four
// consecutive columns.  Each wave stages one 32 x 32 tile at a time in a
// private LDS area (one 8-byte write per run of BF16 values, one 4-byte write
// per run of codes) and writes it out by rows, 16 bytes per lane.  Row pitches
// of 72 and 40 bytes put the 32 rows of a column run on distinct banks.
// (Storing the runs straight from registers touches 32 rows per store
// instruction, and pairing columns across lanes with DPP costs ~27 vector
// instructions per two elements; both were measured slower.)
constexpr int kPitch16 = 72, kPitch8 = 40;
constexpr int kStage16 = 32 * kPitch16, kStage8 = 32 * kPitch8;

// Writes the staged 32 x 32 BF16 tile to out (row-major, leading dimension
// ld) at (row0, col0): 64 bytes per row, 4 lanes per row, 16 rows per pass.
__device__ __forceinline__ void flush16(const uint8_t* st, uint16_t* out, int row0, int col0,
                                        int ld, int lane) {
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int r = (lane >> 2) + 16 * k, c = lane & 3;
    const uint2 lo = *reinterpret_cast<const uint2*>(st + r * kPitch16 + c * 16);
    const uint2 hi = *reinterpret_cast<const uint2*>(st + r * kPitch16 + c * 16 + 8);
    *reinterpret_cast<uint4*>(out + (size_t)(row0 + r) * ld + col0 + c * 8) =
        make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
}

// The same for the staged 32 x 32 tile of codes: 32 bytes per row, 2 lanes per row.
__device__ __forceinline__ void flush8(const uint8_t* st, uint8_t* out, int row0, int col0,
                                       int ld, int lane) {
  const int r = lane >> 1, c = lane & 1;
  const uint2 lo = *reinterpret_cast<const uint2*>(st + r * kPitch8 + c * 16);
  const uint2 hi = *reinterpret_cast<const uint2*>(st + r * kPitch8 + c * 16 + 8);
  *reinterpret_cast<uint4*>(out + (size_t)(row0 + r) * ld + col0 + c * 16) =
      make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// QUANT = false: plain BF16 GEMM, H = bf16(X W^T) to h_out.
// QUANT = true: the quantizing epilogue; h_out and b_out may be null.
template <int TN, int ACT, int FMT, bool QUANT, bool SPL>
__global__ __launch_bounds__(512, 1) void k_gemm_bf16(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, int M, int N, int K,
    const float* __restrict__ scale_ptr, fp8dp_acc_slot* __restrict__ slots,
    uint16_t* __restrict__ h_out, uint16_t* __restrict__ b_out, uint8_t* __restrict__ q_out) {
  constexpr int BM = 256, BN = 64 * TN, TM = 2;
  constexpr int ASZ = BM * kBK, SLOT = (BM + BN) * kBK;
  constexpr int LA = BM / 64, LB = BN / 64;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * SLOT + 8 * (kStage16 + kStage8)];

  const int tiles_n = N / BN;
  const int ntiles = (M / BM) * tiles_n;
  const int G = gridDim.x;
  const int passes = tiles_of_block(blockIdx.x, G, ntiles);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = (wave >> 1) * 64;
  const int wc = (wave & 1) * (BN / 2);
  const size_t rowbytes = (size_t)K * 2;
  const int KT = (int)(rowbytes / kBK);
  const int GS = passes * KT;   // stages this workgroup runs, tile after tile

  // copies: as in the FP8 kernel, over rows of K * 2 bytes; stage g is
  // k-stage g % KT of the tile of pass g / KT
  const int lrow = lane >> 3;
  const int lchunk = (lane & 7) ^ ((4 * wave + (lrow >> 1)) & 7);
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(X) + (size_t)(wave * 8 + lrow) * rowbytes + lchunk * 16;
  const uint8_t* wb = reinterpret_cast<const uint8_t*>(W) + (size_t)(wave * 8 + lrow) * rowbytes + lchunk * 16;
  const size_t rstep = (size_t)64 * rowbytes;
  // SPL: only waves 0-3 copy (row groups w + 4 i: the LDS swizzle depends on
  // w % 2 alone, so the layout is the same), and only waves 4-7 store the
  // epilogue's outputs.  The vector-memory counter is per wave and counts
  // loads and stores together: a wave that stores and copies must wait for
  // its stores whenever it waits for its copies, which after each tile's
  // epilogue drained ~144 KiB of stores per CU before the next stage could
  // start.  Split this way, the copying waves never have stores in flight
  // and the storing waves never wait on the counter.
  auto issue = [&](int g) {
    const int tile = tile_of_pass(blockIdx.x, g / KT, G, ntiles);
    const size_t k0 = (size_t)(g % KT) * kBK;
    const uint8_t* gA = xb + (size_t)((tile / tiles_n) * BM) * rowbytes + k0;
    const uint8_t* gB = wb + (size_t)((tile % tiles_n) * BN) * rowbytes + k0;
    uint8_t* base = lds + (g & 1) * SLOT + wave * 1024;
    if constexpr (SPL) {
      if (wave < 4) {
#pragma unroll
        for (int i = 0; i < 2 * LA; ++i) copy16_to_lds(gA + i * (rstep / 2), base + i * 4096);
#pragma unroll
        for (int i = 0; i < 2 * LB; ++i) copy16_to_lds(gB + i * (rstep / 2), base + ASZ + i * 4096);
      }
    } else {
#pragma unroll
      for (int i = 0; i < LA; ++i) copy16_to_lds(gA + i * rstep, base + i * 8192);
#pragma unroll
      for (int i = 0; i < LB; ++i) copy16_to_lds(gB + i * rstep, base + ASZ + i * 8192);
    }
  };

  // fragments of half stage h: k steps q = 2h, 2h + 1 of 16 values; the lane
  // reads chunk 2q + lane / 32 (8 BF16 values) of its row.  A and B use the
  // same k assignment, which is all a dot product needs.
  const int frow = lane & 31;
  const int fsel = lane >> 5;
  auto load_frags = [&](int g, int h, v8bf_t fa[][2], v8bf_t fb[][2]) {
    const uint8_t* sA = lds + (g & 1) * SLOT;
    const uint8_t* sB = sA + ASZ;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const int c = 2 * (2 * h + qq) + fsel;
#pragma unroll
      for (int t = 0; t < TM; ++t)
        fa[t][qq] = __builtin_bit_cast(
            v8bf_t, *reinterpret_cast<const u32x4_t*>(sA + swz(wr + t * 32 + frow, c)));
#pragma unroll
      for (int t = 0; t < TN; ++t)
        fb[t][qq] = __builtin_bit_cast(
            v8bf_t, *reinterpret_cast<const u32x4_t*>(sB + swz(wc + t * 32 + frow, c)));
    }
  };

  v16f_t acc[TM][TN];
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  };
  auto mfmas = [&](v8bf_t fa[][2], v8bf_t fb[][2]) {
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j][qq], fa[i][qq], acc[i][j], 0, 0, 0);
  };

  const float s = QUANT ? *scale_ptr : 1.0f;
  uint32_t amax16 = 0, sat = 0;
  // epilogue of one tile, through this wave's staging area
  uint8_t* st16 = lds + 2 * SLOT + wave * (kStage16 + kStage8);
  uint8_t* st8 = st16 + kStage16;
  const int srow = lane & 31, scol = 4 * (lane >> 5);
  // SPL: store wave w (4-7) also writes out the staging area of wave w - 4;
  // a barrier after the staging writes hands the sub-tile over, a second one
  // frees the areas for the next sub-tile (neither touches the memory counters)
  const int pw = wave - 4;
  const int wr_p = (pw >> 1) * 64, wc_p = (pw & 1) * (BN / 2);
  const uint8_t* pst16 = lds + 2 * SLOT + (pw & 3) * (kStage16 + kStage8);
  const uint8_t* pst8 = pst16 + kStage16;
  auto handoff = [&]() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS accesses are done
    stage_barrier();
  };
  auto epilogue = [&](int tile) {
    const int m0 = (tile / tiles_n) * BM;
    const int n0 = (tile % tiles_n) * BN;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row0 = m0 + wr + i * 32;
        const int col0 = n0 + wc + j * 32;
        const int prow0 = m0 + wr_p + i * 32;
        const int pcol0 = n0 + wc_p + j * 32;
        uint32_t hb[8];   // run g = pairs 2g, 2g + 1: columns 8 g + scol .. +3
#pragma unroll
        for (int p = 0; p < 8; ++p) hb[p] = pack2_bf16_hw(acc[i][j][2 * p], acc[i][j][2 * p + 1]);
        if (!QUANT || h_out != nullptr) {
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<uint2*>(st16 + srow * kPitch16 + (8 * g + scol) * 2) =
                make_uint2(hb[2 * g], hb[2 * g + 1]);
          if constexpr (SPL) {
            handoff();
            if (wave >= 4) {
              flush16(st16, h_out, row0, col0, N, lane);
              flush16(pst16, h_out, prow0, pcol0, N, lane);
            }
            handoff();
          } else {
            flush16(st16, h_out, row0, col0, N, lane);
          }
        }
        if constexpr (QUANT) {
          uint32_t b[8];
#pragma unroll
          for (int p = 0; p < 8; ++p) b[p] = act_pair<ACT, true>(hb[p]);
          if (b_out != nullptr) {
#pragma unroll
            for (int g = 0; g < 4; ++g)
              *reinterpret_cast<uint2*>(st16 + srow * kPitch16 + (8 * g + scol) * 2) =
                  make_uint2(b[2 * g], b[2 * g + 1]);
            if constexpr (!SPL) flush16(st16, b_out, row0, col0, N, lane);
          }
          const uint32_t mx0 = vec_absmax16<ACT == FP8DP_ACT_IDENTITY>(b);
          const uint32_t mx1 = vec_absmax16<ACT == FP8DP_ACT_IDENTITY>(b + 4);
          const uint32_t mx = mx0 > mx1 ? mx0 : mx1;
          amax16 = mx > amax16 ? mx : amax16;
          const uint2 q0 = cast8<FMT, true>(b, mx0, s, sat);       // runs 0, 1
          const uint2 q1 = cast8<FMT, true>(b + 4, mx1, s, sat);   // runs 2, 3
          const uint32_t q[4] = {q0.x, q0.y, q1.x, q1.y};
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<uint32_t*>(st8 + srow * kPitch8 + 8 * g + scol) = q[g];
          if constexpr (SPL) {
            handoff();
            if (wave >= 4) {
              if (b_out != nullptr) {
                flush16(st16, b_out, row0, col0, N, lane);
                flush16(pst16, b_out, prow0, pcol0, N, lane);
              }
              flush8(st8, q_out, row0, col0, N, lane);
              flush8(pst8, q_out, prow0, pcol0, N, lane);
            }
            handoff();
          } else {
            flush8(st8, q_out, row0, col0, N, lane);
          }
        }
      }
  };

  // One pipeline over all of this workgroup's stages: the copies of the next
  // tile's first stages are in flight while a tile finishes and its epilogue
  // runs.  (The copy-completion waits also wait for the epilogue's stores:
  // the vector memory counter covers both.)
  zero_acc();
  if (GS > 0) {
    issue(0);
    if (GS > 1) {
      issue(1);
      if (!SPL) wait_vmcnt<LA + LB>();
      else if (wave < 4) wait_vmcnt<2 * (LA + LB)>();
    } else {
      if (!SPL || wave < 4) wait_vmcnt<0>();
    }
    stage_barrier();
    v8bf_t fa0[TM][2], fb0[TN][2], fa1[TM][2], fb1[TN][2];
    load_frags(0, 0, fa0, fb0);
    int kt = 0;
    for (int g = 0; g < GS; ++g) {
      load_frags(g, 1, fa1, fb1);
      mfmas(fa0, fb0);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      if (!SPL || wave < 4) wait_vmcnt<0>();   // (storing waves have no copies to wait for)
      stage_barrier();
      if (g + 2 < GS) issue(g + 2);
      if (g + 1 < GS) load_frags(g + 1, 0, fa0, fb0);
      mfmas(fa1, fb1);
      if (++kt == KT) {
        epilogue(tile_of_pass(blockIdx.x, g / KT, G, ntiles));
        zero_acc();
        kt = 0;
      }
    }
  }
  if constexpr (QUANT) {
    // the staging areas hold the fold's scratch (one LDS array, see
    // block_fold_in); every wave is past its last staging access
    __builtin_amdgcn_s_waitcnt(0xC07F);
    stage_barrier();
    block_fold_in<512>(amax16, sat, slots, reinterpret_cast<uint32_t*>(lds + 2 * SLOT));
  }
}

template <int TN, int ACT, int FMT, bool QUANT>
static int launch_bf16(const uint16_t* x, const uint16_t* w, int64_t M, int64_t N, int64_t K,
                       fp8dp_tensor_state* st, uint16_t* h_out, uint16_t* b_out, uint8_t* q_out,
                       hipStream_t stream) {
  // persistent: at most one workgroup per compute unit (the LDS ring takes
  // more than half of a CU's 160 KiB), a multiple of 8 for the XCD order
  const int64_t ntiles = (M / 256) * (N / (64 * TN));
  int64_t grid = ntiles;
  const int64_t cus = num_cus() & ~7;
  if (cus >= 8 && grid > cus) grid = cus;
  // the split of copy and store duties pays with the quantizing epilogue's
  // 144 KiB of stores per tile (117.6 vs 120.0 us at the GPT-2 up-projection),
  // not with the plain GEMM's 96 KiB (89.6 vs 87.5 us)
  hipLaunchKernelGGL((k_gemm_bf16<TN, ACT, FMT, QUANT, QUANT>),
                     dim3((unsigned)grid), dim3(512), 0, stream, x, w,
                     (int)M, (int)N, (int)K, QUANT ? &st->scale : nullptr,
                     QUANT ? st->acc : nullptr, h_out, b_out, q_out);
  return check_launch("gemm_bf16_quantize_fused");
}

template <int ACT, int FMT, bool QUANT>
static int launch_bf16_tile(const uint16_t* x, const uint16_t* w, int64_t M, int64_t N, int64_t K,
                            fp8dp_tensor_state* st, uint16_t* h_out, uint16_t* b_out,
                            uint8_t* q_out, hipStream_t stream) {
  // (the quantizing epilogue does not fit the 256-wide tile's registers)
  if (N % 192 == 0) return launch_bf16<3, ACT, FMT, QUANT>(x, w, M, N, K, st, h_out, b_out, q_out, stream);
  if constexpr (!QUANT) {
    if (N % 256 == 0) return launch_bf16<4, ACT, FMT, QUANT>(x, w, M, N, K, st, h_out, b_out, q_out, stream);
  }
  return launch_bf16<2, ACT, FMT, QUANT>(x, w, M, N, K, st, h_out, b_out, q_out, stream);
}

}  // namespace fp8dp

using namespace fp8dp;

extern "C" int gemm_bf16_quantize_fused(const uint16_t* x, const uint16_t* w, int64_t M, int64_t N,
                                        int64_t K, fp8dp_act act, fp8dp_format fmt,
                                        fp8dp_tensor_state* st, uint16_t* h_out,
                                        uint16_t* bf16_out, uint8_t* fp8_out,
                                        hipStream_t stream) {
  if (x == nullptr || w == nullptr) {
    set_error("gemm_bf16_quantize_fused: x and w must be non-NULL");
    return FP8DP_EINVAL;
  }
  if (M < 256 || N < 128 || K < 64 || M % 256 || N % 128 || K % 64) {
    set_error("gemm_bf16_quantize_fused: M must be a positive multiple of 256, N of 128 and K of "
              "64 (got %lld, %lld, %lld)", (long long)M, (long long)N, (long long)K);
    return FP8DP_EINVAL;
  }
  if (M > (int64_t)1 << 30 || N > (int64_t)1 << 30 || K > (int64_t)1 << 29 ||
      (M / 256) * (N / 128) > (int64_t)0x7FFFFFFF) {
    set_error("gemm_bf16_quantize_fused: shape too large");
    return FP8DP_EINVAL;
  }
  if (!aligned16(x) || !aligned16(w) || !aligned16(h_out) || !aligned16(bf16_out) ||
      !aligned16(fp8_out)) {
    set_error("gemm_bf16_quantize_fused: tensors must be 16-byte aligned");
    return FP8DP_EINVAL;
  }
  if (fp8_out == nullptr) {
    if (h_out == nullptr || bf16_out != nullptr || st != nullptr) {
      set_error("gemm_bf16_quantize_fused: without fp8_out it is the plain GEMM: h_out required, "
                "bf16_out and st must be NULL");
      return FP8DP_EINVAL;
    }
    return launch_bf16_tile<FP8DP_ACT_IDENTITY, 0, false>(x, w, M, N, K, nullptr, h_out, nullptr,
                                                           nullptr, stream);
  }
  if (st == nullptr || reinterpret_cast<uintptr_t>(st) & 15u) {
    set_error("gemm_bf16_quantize_fused: fp8_out needs a 16-byte aligned scaling state");
    return FP8DP_EINVAL;
  }
  if ((act != FP8DP_ACT_IDENTITY && act != FP8DP_ACT_RELU2) ||
      (fmt != FP8DP_E4M3 && fmt != FP8DP_E5M2)) {
    set_error("gemm_bf16_quantize_fused: unknown activation or format");
    return FP8DP_EINVAL;
  }
  if (act == FP8DP_ACT_RELU2) {
    if (fmt == FP8DP_E4M3)
      return launch_bf16_tile<FP8DP_ACT_RELU2, 0, true>(x, w, M, N, K, st, h_out, bf16_out, fp8_out, stream);
    return launch_bf16_tile<FP8DP_ACT_RELU2, 1, true>(x, w, M, N, K, st, h_out, bf16_out, fp8_out, stream);
  }
  if (fmt == FP8DP_E4M3)
    return launch_bf16_tile<FP8DP_ACT_IDENTITY, 0, true>(x, w, M, N, K, st, h_out, bf16_out, fp8_out, stream);
  return launch_bf16_tile<FP8DP_ACT_IDENTITY, 1, true>(x, w, M, N, K, st, h_out, bf16_out, fp8_out, stream);
}
