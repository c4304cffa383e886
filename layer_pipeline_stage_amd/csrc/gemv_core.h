// Shared pieces of the weight-streaming kernels: chunk formats, the per-chunk
// multiply-accumulate for f32 / bf16 / MXFP4 weights, and the LDS staging of the
// (optionally RMS-normalised) activation vector.
#pragma once

#include "dev.h"
#include "../../include/lps.h"

namespace lps {

template <int WT> struct Fmt;
template <> struct Fmt<LPS_F32> { static constexpr int CH = 4; };
template <> struct Fmt<LPS_BF16> { static constexpr int CH = 8; };
template <> struct Fmt<LPS_MXFP4> { static constexpr int CH = 32; };

constexpr int GEMV_THREADS = 256;

// e8m0 byte -> f32 scale 2^(s-127) (0 -> 2^-127 subnormal, 255 -> NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  if (s == 0) return __uint_as_float(0x00400000u);
  if (s == 255) return __uint_as_float(0x7FC00000u);
  return __uint_as_float(s << 23);
}

template <int WT>
__device__ __forceinline__ void acc_chunk(const u32x4 v, uint32_t sb, const float* xs, float& a) {
  if constexpr (WT == LPS_F32) {
    const f32x4 xv = *reinterpret_cast<const f32x4*>(xs);
    a = fmaf(__uint_as_float(v.x), xv.x, a);
    a = fmaf(__uint_as_float(v.y), xv.y, a);
    a = fmaf(__uint_as_float(v.z), xv.z, a);
    a = fmaf(__uint_as_float(v.w), xv.w, a);
  } else if constexpr (WT == LPS_BF16) {
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(xs);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(xs + 4);
    a = fmaf(bf16_lo(v.x), x0.x, a);
    a = fmaf(bf16_hi(v.x), x0.y, a);
    a = fmaf(bf16_lo(v.y), x0.z, a);
    a = fmaf(bf16_hi(v.y), x0.w, a);
    a = fmaf(bf16_lo(v.z), x1.x, a);
    a = fmaf(bf16_hi(v.z), x1.y, a);
    a = fmaf(bf16_lo(v.w), x1.z, a);
    a = fmaf(bf16_hi(v.w), x1.w, a);
  } else {
    const float sc = e8m0_to_f32(sb);
    const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 xa = *reinterpret_cast<const f32x4*>(xs + 8 * q);
      const f32x4 xb = *reinterpret_cast<const f32x4*>(xs + 8 * q + 4);
      // each call converts the two codes of one byte: element 2b (low nibble)
      // then 2b+1 (high nibble), already multiplied by the group scale
      const f32x2 e0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[q], sc, 0);
      const f32x2 e1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[q], sc, 1);
      const f32x2 e2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[q], sc, 2);
      const f32x2 e3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[q], sc, 3);
      a = fmaf(e0.x, xa.x, a);
      a = fmaf(e0.y, xa.y, a);
      a = fmaf(e1.x, xa.z, a);
      a = fmaf(e1.y, xa.w, a);
      a = fmaf(e2.x, xb.x, a);
      a = fmaf(e2.y, xb.y, a);
      a = fmaf(e3.x, xb.z, a);
      a = fmaf(e3.y, xb.w, a);
    }
  }
}

// Stage the activation vector in LDS; with NORM, as RMSNorm(x) * g.
template <bool NORM, int NT = GEMV_THREADS>
__device__ __forceinline__ void stage_x(const float* x, const float* g, float eps, int K, float* xs) {
  const int tid = threadIdx.x;
  float ss = 0.f;
  for (int k = tid * 4; k < K; k += NT * 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(x + k);
    *reinterpret_cast<f32x4*>(xs + k) = v;
    if (NORM) ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  if (NORM) {
    __shared__ float red[NT / WAVE];
    ss = wave_sum(ss);
    if ((tid & (WAVE - 1)) == 0) red[tid / WAVE] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < NT / WAVE; ++i) tot += red[i];
    const float r = 1.0f / sqrtf(tot / float(K) + eps);
    for (int k = tid * 4; k < K; k += NT * 4) {
      f32x4 v = *reinterpret_cast<f32x4*>(xs + k);
      const f32x4 gg = *reinterpret_cast<const f32x4*>(g + k);
      v.x = v.x * r * gg.x;
      v.y = v.y * r * gg.y;
      v.z = v.z * r * gg.z;
      v.w = v.w * r * gg.w;
      *reinterpret_cast<f32x4*>(xs + k) = v;
    }
  }
  __syncthreads();
}

}  // namespace lps
