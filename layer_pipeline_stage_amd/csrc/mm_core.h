// One 256 x 256 tile of C = A B^T (bf16 operands, f32 accumulators) on the
// matrix cores of a gfx950 CU: the main loop shared by the prefill GEMMs (the MoE
// grouped GEMMs and the dense layer GEMMs).  The caller maps its rows (gathered
// token rows, chunk rows, weight rows) to byte offsets; this file stages and
// multiplies them.
//
// Four waves (2 x 2, one per SIMD), each 128 x 128 as 4 x 4 MFMA 32x32x16 blocks
// with the accumulators in the accumulation registers: per 16-deep sub-step a wave
// reads 8 KiB of operands from LDS for 16 products, half a KiB per product.
// The operands go from global memory straight into LDS by the LDS DMA path (buffer
// loads with the LDS as destination: no registers, no LDS store instructions) in
// K steps of MM_BK through rings of MM_SA stages for A and MM_SB for B.  A staged
// row is one step of K (whole 128-byte lines); its 16-byte k chunk c sits at slot
// c ^ mm_swz(r).  The LDS has 64 four-byte banks and serves a ds_read_b128 16 lanes
// (256 bytes) at a time; an operand read is 16 consecutive rows at one chunk, so
// rows of the same parity (two 128-byte rows per 256 bytes) take 8 distinct slots.
// Order of issue, pinned with scheduling-group barriers because with one wave per
// SIMD the wave's own instruction order decides what overlaps the products and its
// loads queue at the CU's one address unit: each sub-step's 16 products go out one
// by one with the next sub-step's 8 operand reads between the first eight (their
// LDS latency is covered by the last eight) and a share of the A loads of step
// t + MM_SA - 1 between the last eight; after step t's barrier (every wave has read
// step t's stages and every wave's loads of step t + 1 have landed) the B loads of
// step t + MM_SB go between the last sub-step's products.  The last steps' loads
// repeat the last step into stages that are not read again.
#pragma once

#include "dev.h"

namespace lps {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int MM_TILE = 256;                 // rows of A and of B per tile
constexpr int MM_THREADS = 256;
constexpr int MM_BK = 64;                    // K per step
constexpr int MM_SA = 3, MM_SB = 2;          // LDS stages of A and of B
constexpr int MM_NS = MM_BK / 16;            // sub-steps per step
constexpr int MM_CH = MM_BK / 8;             // 16-byte chunks per staged row
constexpr int MM_ROWB = MM_BK * 2;           // bytes of a staged row
constexpr int MM_OPB = MM_TILE * MM_ROWB;    // bytes per operand stage
constexpr int MM_RPI = 64 / MM_CH;           // staged rows per load instruction
constexpr int MM_NI = 64 / MM_RPI;           // load instructions per wave, operand and step
constexpr int MM_LDS = (MM_SA + MM_SB) * MM_OPB;
static_assert(MM_NS == 4 && MM_SA == MM_SB + 1 && MM_SB >= 2, "staging shape");
static_assert(MM_LDS <= 160 * 1024, "staging exceeds the LDS");
// Loads return in order, so at step t's wait (A and B of step t + 1 landed) the
// loads issued after B of step t + 1 may still be out: step t's A loads and MM_SB - 2
// steps of A and B.
constexpr int MM_VM_MID = MM_NI + (MM_SB - 2) * 2 * MM_NI;
constexpr int MM_VM_PRO = (MM_SB - 1) * 2 * MM_NI;
static_assert(MM_VM_PRO < 64 && MM_VM_MID < 64, "vmcnt range");

// slot of chunk c in staged row r is c ^ mm_swz(r)
__device__ __forceinline__ int mm_swz(int r) { return (r >> 1) & 7; }
// the tile row this lane stages with its load j (j < MM_NI), and the k chunk it loads
__device__ __forceinline__ int mm_stage_row(int wv, int lane, int j) {
  return 64 * wv + MM_RPI * j + lane / MM_CH;
}
__device__ __forceinline__ int mm_stage_chunk(int row, int lane) {
  return (lane % MM_CH) ^ mm_swz(row);
}
// s_waitcnt immediates (gfx9 encoding): vmcnt bits [3:0] and [15:14], lgkmcnt [11:8]
constexpr int mm_wait(int vm, int lgkm) {
  return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | ((vm >> 4) << 14);
}

// acc[i][j] += the tile's products: acc[i][j][r] is C[128 wm + 32 i + 8 (r / 4) +
// 4 (lane / 32) + r % 4][128 wn + 32 j + lane % 32] with wave (wm, wn) = (wv / 2, wv % 2).
// aoff / boff: the byte offset, in ares / bres, of the k chunk that staged row
// mm_stage_row(wv, lane, j) loads at step 0 (mm_stage_chunk of that row); step t adds
// t * MM_ROWB.  AUXA / AUXB: the loads' cache policy bits.  nk >= 2 steps.  lds:
// MM_LDS bytes, 16-byte aligned.  Returns with every load landed and a barrier
// passed, so the caller may reuse the LDS.
template <int AUXA, int AUXB>
__device__ __forceinline__ void mm_tile(__amdgpu_buffer_rsrc_t ares, __amdgpu_buffer_rsrc_t bres,
                                        const int (&aoff)[MM_NI], const int (&boff)[MM_NI], int nk,
                                        char* lds, f32x16 (&acc)[4][4]) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int wm = wv >> 1, wn = wv & 1;
  char* ldsA = lds;                          // [MM_SA][MM_TILE][MM_ROWB]
  char* ldsB = lds + MM_SA * MM_OPB;         // [MM_SB][MM_TILE][MM_ROWB]
  // operand reads: A rows 128 wm + 32 i + lane % 32, B rows 128 wn + 32 j + lane % 32
  // (their swizzle is lane % 32's); sub-step ks takes k chunk 2 ks + lane / 32
  const int fr = lane & 31, fsw = mm_swz(fr), fh = lane >> 5;
  const int ard = (128 * wm + fr) * MM_ROWB, brd = (128 * wn + fr) * MM_ROWB;

#define MM_DMA_B(S, T)                                                                         \
  _Pragma("unroll") for (int j = 0; j < MM_NI; ++j)                                            \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                  \
        bres, (lds_ptr_t)(ldsB + (S) * MM_OPB + (64 * wv + MM_RPI * j) * MM_ROWB), 16, boff[j], \
        (T) * MM_ROWB, 0, AUXB);
#define MM_DMA_A1(S, T, J)                                                                     \
  __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                    \
      ares, (lds_ptr_t)(ldsA + (S) * MM_OPB + (64 * wv + MM_RPI * (J)) * MM_ROWB), 16, aoff[J], \
      (T) * MM_ROWB, 0, AUXA);
#define MM_READ(R, SA_, SB_, KS)                                                               \
  {                                                                                            \
    const int sl = 16 * ((2 * (KS) + fh) ^ fsw);                                               \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                            \
      R[i] = *reinterpret_cast<const bf16x8*>(ldsA + (SA_) * MM_OPB + ard + 32 * i * MM_ROWB + sl); \
      R[4 + i] = *reinterpret_cast<const bf16x8*>(ldsB + (SB_) * MM_OPB + brd + 32 * i * MM_ROWB + sl); \
    }                                                                                          \
  }
#define MM_MMA(R)                                                                              \
  _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                                              \
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(R[i], R[4 + j], acc[i][j], 0, 0, 0);
#define MM_PACE_READS()                                                                        \
  _Pragma("unroll") for (int q = 0; q < 8; ++q) {                                              \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                         \
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                         \
  }

  // prologue: the loads of steps before 0 in the loop's order (during step s the A
  // loads of step s + MM_SB, after it the B loads of the same step, s = -MM_SB .. -1);
  // with fewer steps than stages the extra stages get the last step again and are
  // never read
#pragma unroll
  for (int s = 0; s < MM_SB; ++s) {
#pragma unroll
    for (int j = 0; j < MM_NI; ++j) MM_DMA_A1(s, min(s, nk - 1), j)
    MM_DMA_B(s, min(s, nk - 1))
  }
  bf16x8 r0[8], r1[8];
  __builtin_amdgcn_s_waitcnt(mm_wait(MM_VM_PRO, 15));   // this wave's loads of step 0
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  MM_READ(r0, 0, 0, 0)
  int sa = 0, sb = 0;                        // stages of step kt
  int fa = MM_SA - 1;                        // the A stage freed by the previous step
  for (int kt = 0; kt < nk; ++kt) {
    const int ta = min(kt + MM_SA - 1, nk - 1);   // A loads of this step's spread
    // sub-step KS: read sub-step KS into RN, issue A loads [J0, J1), multiply RC
#define MM_SUB(KS, RN, RC)                                                                     \
    {                                                                                          \
      constexpr int J0 = ((KS) - 1) * MM_NI / (MM_NS - 1), J1 = (KS) * MM_NI / (MM_NS - 1);    \
      MM_READ(RN, sa, sb, KS)                                                                  \
      _Pragma("unroll") for (int j = J0; j < J1; ++j) MM_DMA_A1(fa, ta, j)                     \
      MM_MMA(RC)                                                                               \
      MM_PACE_READS()                                                                          \
      _Pragma("unroll") for (int q = 0; q < J1 - J0; ++q) {                                    \
        __builtin_amdgcn_sched_group_barrier(0x008, 8 / (J1 - J0), 0);                         \
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                                     \
      }                                                                                        \
      __builtin_amdgcn_sched_group_barrier(0x008, 8 - (8 / (J1 - J0)) * (J1 - J0), 0);         \
      __builtin_amdgcn_sched_barrier(0);                                                       \
    }
    MM_SUB(1, r1, r0)
    MM_SUB(2, r0, r1)
    MM_SUB(3, r1, r0)
#undef MM_SUB
    // the reads above are done and this wave's loads of step kt + 1 have landed
    __builtin_amdgcn_s_waitcnt(mm_wait(MM_VM_MID, 0));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const int na = sa + 1 == MM_SA ? 0 : sa + 1, nb = sb + 1 == MM_SB ? 0 : sb + 1;
    MM_READ(r0, na, nb, 0)
    MM_DMA_B(sb, min(kt + MM_SB, nk - 1))
    MM_MMA(r1)                               // the last sub-step (3) is in r1
    MM_PACE_READS()
#pragma unroll
    for (int q = 0; q < MM_NI; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 8 / MM_NI, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    fa = sa;
    sa = na;
    sb = nb;
  }
#undef MM_DMA_A1
#undef MM_DMA_B
#undef MM_READ
#undef MM_MMA
#undef MM_PACE_READS
  // the loads still out only repeat the last step into unread stages: drain them
  // before the stages are reused
  __builtin_amdgcn_s_waitcnt(mm_wait(0, 0));
  __syncthreads();
}

}  // namespace lps
