// Device helpers for the gfx950 kernels (wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace lps {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

// Streaming 16-byte load of weights that are read once per token: the
// nontemporal hint keeps them from evicting the activations and KV tiles.
__device__ __forceinline__ u32x4 ld_stream16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// bf16 halves of a 32-bit word, widened exactly to f32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// f32 -> bf16 bits, round to nearest, ties to even (finite values).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Cross-lane steps.  Inside a 16-lane row: DPP permutations (a VALU operand
// modifier, no LDS).  Across rows: DPP row broadcasts for whole-wave totals, and
// LDS-crossbar shuffles (ds_bpermute) where every lane needs its own partner.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float v, float old = 0.f) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                               __builtin_bit_cast(int, v), CTRL,
                                                               ROW_MASK, 0xF, false));
}
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <-> 7 - i within 8
constexpr int DPP_MIRROR = 0x140;      // lane i <-> 15 - i within 16
constexpr int DPP_ROR8 = 0x128;        // lane i <- (i + 8) % 16, i.e. i ^ 8
constexpr int DPP_BCAST15 = 0x142;     // rows 1, 3 <- lane 15 of rows 0, 2
constexpr int DPP_BCAST31 = 0x143;     // rows 2, 3 <- lane 31

// A workgroup barrier for LDS traffic only: this wave's LDS operations complete
// (lgkmcnt 0), then s_barrier.  Unlike __syncthreads it does not wait for the
// wave's outstanding global loads, so weight loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt 63, expcnt 7, lgkmcnt 0
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ float lane63(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Sum over aligned groups of W lanes (W a power of two <= 64).  Every lane of a
// group receives the same total: each step adds two partial sums that are
// equal on both partner lanes, and a + b == b + a exactly, so one fixed tree.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (W >= 2) v += dpp<DPP_XOR1>(v);
  if constexpr (W >= 4) v += dpp<DPP_XOR2>(v);
  if constexpr (W >= 8) v += dpp<DPP_HALF_MIRROR>(v);
  if constexpr (W >= 16) v += dpp<DPP_MIRROR>(v);
  if constexpr (W == 32) v += __shfl_xor(v, 16, WAVE);
  if constexpr (W == 64) {
    // row sums -> rows 1, 3 hold S0 + S1, S2 + S3 -> row 3 holds the total
    v += dpp<DPP_BCAST15, 0xA>(v);
    v += dpp<DPP_BCAST31, 0xC>(v);
    v = lane63(v);
  }
  return v;
}
__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<DPP_XOR1>(v));
  v = fmaxf(v, dpp<DPP_XOR2>(v));
  v = fmaxf(v, dpp<DPP_HALF_MIRROR>(v));
  v = fmaxf(v, dpp<DPP_MIRROR>(v));
  v = fmaxf(v, dpp<DPP_BCAST15, 0xA>(v, v));   // rows left unwritten keep their own value
  v = fmaxf(v, dpp<DPP_BCAST31, 0xC>(v, v));
  return lane63(v);
}
// Sum over the lanes l, l + S, l + 2S, ... (S a power of two >= 8): the
// per-row partial sums of lanes that own the same columns.
template <int S>
__device__ __forceinline__ float strided_sum(float v) {
  if constexpr (S <= 8) v += dpp<DPP_ROR8>(v);
  if constexpr (S <= 16) v += __shfl_xor(v, 16, WAVE);
  if constexpr (S <= 32) v += __shfl_xor(v, 32, WAVE);
  return v;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }
// e^x as one v_exp_f32 of x log2(e) (a few ulps from the correctly rounded expf, which
// takes ~10 instructions): for softmax weights, whose selections never depend on it
__device__ __forceinline__ float exp_native(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}
// silu from the native base-2 exponential and reciprocal (v_exp_f32, v_rcp_f32: about
// one ulp each, a few ulp together): for epilogues that round the product to bf16
// right after, where the correctly rounded expf and division cost ~20 VALU
// instructions per value.  z -> -inf: exp2 -> inf, rcp -> 0, result -0.
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}

}  // namespace lps
