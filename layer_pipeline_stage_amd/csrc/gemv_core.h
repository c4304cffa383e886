// Shared pieces of the weight-streaming kernels: chunk formats, the per-chunk
// multiply-accumulate for f32 / bf16 weights (f32 activations) and MXFP4 weights
// (f16 activations), and the LDS staging of the (optionally RMS-normalised)
// activation vector.
#pragma once

#include "dev.h"
#include "../../include/lps.h"

namespace lps {

template <int WT> struct Fmt;
template <> struct Fmt<LPS_F32> { static constexpr int CH = 4; };
template <> struct Fmt<LPS_BF16> { static constexpr int CH = 8; };
template <> struct Fmt<LPS_MXFP4> { static constexpr int CH = 32; };

constexpr int GEMV_THREADS = 256;

// e8m0 byte -> f32 scale 2^(s-127) (0 -> 2^-127 subnormal, 255 -> NaN), without
// branches: s << 23 is the exponent field; bit 22 turns 0 into the subnormal
// 2^-127 and the all-ones exponent into a quiet NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  const uint32_t edge = ((s + 1u) & 0xFFu) < 2u ? 0x00400000u : 0u;
  return __uint_as_float((s << 23) | edge);
}

// one chunk of f32 or bf16 weights against its staged f32 activations (sb unused)
template <int WT>
__device__ __forceinline__ void acc_chunk(const u32x4 v, uint32_t sb, const float* xs, float& a) {
  static_assert(WT == LPS_F32 || WT == LPS_BF16, "MXFP4 chunks: acc_chunk_mx16");
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
  }
}

constexpr int GPRE = 8;   // norm-gain float4s per thread held in registers

// v = v * r * g, in that order (the rounding the oracle's RMSNorm reading fixes)
__device__ __forceinline__ void scale4(float* px, float r, const f32x4 gg) {
  f32x4 v = *reinterpret_cast<f32x4*>(px);
  v.x = v.x * r * gg.x;
  v.y = v.y * r * gg.y;
  v.z = v.z * r * gg.z;
  v.w = v.w * r * gg.w;
  *reinterpret_cast<f32x4*>(px) = v;
}

// gfx9 s_waitcnt immediate that waits until at most vm vector-memory loads are
// outstanding (lgkmcnt and expcnt left at their maxima)
constexpr int vm_wait(int vm) { return (vm & 15) | (7 << 4) | (15 << 8) | ((vm >> 4) << 14); }

// Stage the activation vector in LDS; with NORM, as RMSNorm(x) * g.  The copy
// uses the LDS DMA path (global_load_lds_dwordx4: each lane's 16 bytes land at
// the wave's LDS base + 16 * lane, no VGPRs): every wave issues all of its
// 1 KiB pieces back to back, so staging costs one L2 round trip rather than one
// per piece.  x must be 16-byte aligned and K a multiple of 4.
// In two parts: stage_x_issue sends the gain's loads and the copy; stage_x_finish
// waits until at most VM later loads are outstanding (loads complete in issue order,
// so a caller that issues VM weight loads in between has them in flight while the
// staging completes), then normalises.
template <bool NORM, int NT = GEMV_THREADS>
__device__ __forceinline__ void stage_x_issue(const float* x, const float* g, int K, float* xs,
                                              f32x4 (&gpre)[GPRE]) {
  constexpr int NW = NT / WAVE;
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1);
  const int wv = tid / WAVE;
  // the norm gain goes out with the copy (same wait), for K <= NT * 4 * GPRE
  if (NORM) {
#pragma unroll
    for (int i = 0; i < GPRE; ++i) {
      const int k = (tid + i * NT) * 4;
      gpre[i] = k < K ? *reinterpret_cast<const f32x4*>(g + k) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  for (int b = wv * 256; b < K; b += NW * 256) {
    if (b + 4 * lane < K)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(x + b + 4 * lane),
                                       (__attribute__((address_space(3))) void*)(xs + b), 16, 0, 0);
  }
}
template <bool NORM, int NT, int VM>
__device__ __forceinline__ void stage_x_finish(const float* g, float eps, int K, float* xs,
                                               const f32x4 (&gpre)[GPRE]) {
  constexpr int NW = NT / WAVE;
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1);
  const int wv = tid / WAVE;
  // the copy has landed (at most VM later loads outstanding) and this wave's LDS
  // stores are done; the barrier leaves the later loads in flight
  __builtin_amdgcn_s_waitcnt(vm_wait(VM) & ~(15 << 8));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (NORM) {
    __shared__ float red[NW];
    float ss = 0.f;
    for (int k = tid * 4; k < K; k += NT * 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(xs + k);
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = wave_sum(ss);
    if (lane == 0) red[wv] = ss;
    lds_barrier();
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) tot += red[i];
    const float r = 1.0f / sqrtf(tot / float(K) + eps);
#pragma unroll
    for (int i = 0; i < GPRE; ++i) {
      const int k = (tid + i * NT) * 4;
      if (k < K) scale4(xs + k, r, gpre[i]);
    }
    for (int k = (tid + GPRE * NT) * 4; k < K; k += NT * 4)
      scale4(xs + k, r, *reinterpret_cast<const f32x4*>(g + k));
    lds_barrier();
  }
}
template <bool NORM, int NT = GEMV_THREADS>
__device__ __forceinline__ void stage_x(const float* x, const float* g, float eps, int K, float* xs) {
  f32x4 gpre[GPRE];
  stage_x_issue<NORM, NT>(x, g, K, xs, gpre);
  stage_x_finish<NORM, NT, 0>(g, eps, K, xs, gpre);
}

// MXFP4 rows against f16 activations.  The activation vector is staged in LDS as
// f16 (rounded once, to nearest even, after the optional RMSNorm in f32), 32-value
// chunks at a pitch of 40 halves (80 bytes: lane l reads the x of its own weight
// chunk, so lanes are a chunk apart; at 80 bytes sixteen consecutive lanes cover
// distinct 16-byte bank groups).  Each byte of codes becomes two f16 weights in
// one scaled conversion (exact: an e2m1 value times a power of two); the products
// with f32 accumulation run on the matrix cores (below).  The chunk after the last
// (index K / 32) is zero.
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
constexpr int MX16_XS = 40;     // halves per staged MXFP4 chunk (32 values + 8 pad)
// x float4 groups per thread held across the norm's sum: a launch with U chunks per
// lane covers rows of up to U * 64 chunks (512 U groups); U = 4 is the launch for
// longer rows, which holds 12 groups per thread
constexpr int mx16_maxr(int U, int NT) { return U == 4 ? 12 : (512 * U + NT - 1) / NT; }

// A chunk's products on the matrix cores: v_mfma_f32_16x16x32_f16
// takes the A operand of row m = l % 16, k = 8 (l / 16) .. + 7 from lane l and the B
// operand of column n = l % 16 at the same k from lane l, so when every lane gives
// 8 of its own chunk's weights as A and the same 8 staged activations as B, the
// diagonal element D[m][m] sums those products of lanes m, m + 16, m + 32, m + 48
// (the other elements mix lanes and are not used).  Four products (the chunk's
// words q = 0..3: values 8q .. 8q + 7) cover the 32 values; the conversions stay on
// the vector ALUs, the dot products leave them.  A zero chunk adds exactly +0.
typedef float f32x4m __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void acc_chunk_mx16(const u32x4 v, uint32_t sb, const _Float16* xh, f32x4m& d) {
  const float sc = e8m0_to_f32(sb);
  const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const h8 xv = *reinterpret_cast<const h8*>(xh + 8 * q);
    const h2 w0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd[q], sc, 0);
    const h2 w1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd[q], sc, 1);
    const h2 w2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd[q], sc, 2);
    const h2 w3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd[q], sc, 3);
    const h8 wv = {w0[0], w0[1], w1[0], w1[1], w2[0], w2[1], w3[0], w3[1]};
    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv, xv, d, 0, 0, 0);
  }
}
// this lane's share of the row: its diagonal element of D (lanes 20 q .. 20 q + 3 hold
// D[4 q + i][4 q + i] as element i), zero on the other lanes; a wave sum then gives
// the row's dot product
__device__ __forceinline__ float acc_value(float a) { return a; }
__device__ __forceinline__ float acc_value(f32x4m d) {
  const int l = threadIdx.x & 63;
  if ((l >> 4) != ((l & 15) >> 2)) return 0.f;
  const int i = l & 3;
  return i == 0 ? d[0] : i == 1 ? d[1] : i == 2 ? d[2] : d[3];
}

// Stage x as f16 chunks (see above); with NORM, as RMSNorm(x) * g computed in f32
// (the same v * r * g order as stage_x) before the rounding.  K % 32 == 0 and
// K / 4 <= MAXR * NT (the launch checks it).
// Without NORM the vector's magnitude is not bounded (the attention output, the
// SwiGLU output): when its largest |x| passes 2^15 the staged values are x * 2^-e,
// e the smallest power that brings it to at most 2^15, so none rounds to an f16
// infinity; the return value 2^e scales the products back (exact powers of two,
// and 1 for every vector below 2^15, where the staging is unchanged).
// The staging in two parts, so that a caller can issue the vector's loads (and the
// norm gain's) before its first weight loads: loads return in issue order, so a
// staging whose loads follow the weight batch would wait for that whole batch.
template <bool NORM, int MAXR>
struct Mx16Vec {
  f32x4 v[MAXR];
  f32x4 g[NORM ? MAXR : 1];
};
template <bool NORM, int NT, int MAXR>
__device__ __forceinline__ void stage_x_mx16_load(const float* x, const float* g, int K,
                                                  Mx16Vec<NORM, MAXR>& s) {
  const int tid = threadIdx.x;
  const int ng = K / 4;
#pragma unroll
  for (int i = 0; i < MAXR; ++i) {
    const int G = tid + i * NT;
    s.v[i] = G < ng ? *reinterpret_cast<const f32x4*>(x + 4 * G) : f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (NORM)
      s.g[i] = G < ng ? *reinterpret_cast<const f32x4*>(g + 4 * G) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
}
template <bool NORM, int NT, int MAXR>
__device__ __forceinline__ float stage_x_mx16_store(const Mx16Vec<NORM, MAXR>& s, const float* x,
                                                   float eps, int K, _Float16* xs) {
  constexpr int NW = NT / WAVE;
  const int tid = threadIdx.x;
  const int ng = K / 4;
  float r = 1.f;
  if (NORM) {
    __shared__ float red[NW];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < MAXR; ++i)
      ss += s.v[i].x * s.v[i].x + s.v[i].y * s.v[i].y + s.v[i].z * s.v[i].z + s.v[i].w * s.v[i].w;
    ss = wave_sum(ss);
    if ((tid & (WAVE - 1)) == 0) red[tid / WAVE] = ss;
    lds_barrier();
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) tot += red[i];
    r = 1.0f / sqrtf(tot / float(K) + eps);
  }
  // without NORM each wave records its largest |x| (read after the staging barrier)
  __shared__ float mx[NW];
  if (!NORM) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < MAXR; ++i)
      m = fmaxf(m, fmaxf(fmaxf(fabsf(s.v[i].x), fabsf(s.v[i].y)), fmaxf(fabsf(s.v[i].z), fabsf(s.v[i].w))));
    m = wave_max(m);
    if ((tid & (WAVE - 1)) == 0) mx[tid / WAVE] = m;
  }
#pragma unroll
  for (int i = 0; i < MAXR; ++i) {
    const int G = tid + i * NT;
    if (G < ng) {
      f32x4 y = s.v[i];
      if constexpr (NORM) {
        const f32x4 gg = s.g[i];
        y.x = y.x * r * gg.x;
        y.y = y.y * r * gg.y;
        y.z = y.z * r * gg.z;
        y.w = y.w * r * gg.w;
      }
      // float4 G = values 4G .. 4G + 3: chunk G / 8, halves 4 (G % 8) ..
      _Float16* dst = xs + (G >> 3) * MX16_XS + 4 * (G & 7);
      *reinterpret_cast<h2*>(dst) = h2{(_Float16)y.x, (_Float16)y.y};
      *reinterpret_cast<h2*>(dst + 2) = h2{(_Float16)y.z, (_Float16)y.w};
    }
  }
  if (tid < 16) *reinterpret_cast<h2*>(xs + (K / 32) * MX16_XS + 2 * tid) = h2{0, 0};   // zero chunk
  lds_barrier();
  float back = 1.f;
  if (!NORM) {
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) am = fmaxf(am, mx[i]);
    // the same value on every thread: the restaging below (x read again, scaled)
    // is taken by the whole workgroup or by none of it
    if (am > 32768.f && am <= 3.0e38f) {   // finite and past 2^15 (inf passes as is)
      const int e = ilogbf(am) - 14;         // am * 2^-e < 2^15
      const float sc = ldexpf(1.f, -e);
      back = ldexpf(1.f, e);
      for (int G = tid; G < ng; G += NT) {
        const f32x4 y = *reinterpret_cast<const f32x4*>(x + 4 * G);
        _Float16* dst = xs + (G >> 3) * MX16_XS + 4 * (G & 7);
        *reinterpret_cast<h2*>(dst) = h2{(_Float16)(y.x * sc), (_Float16)(y.y * sc)};
        *reinterpret_cast<h2*>(dst + 2) = h2{(_Float16)(y.z * sc), (_Float16)(y.w * sc)};
      }
      lds_barrier();
    }
  }
  return back;
}

}  // namespace lps
