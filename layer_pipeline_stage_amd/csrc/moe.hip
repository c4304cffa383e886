// MoE FFN layer for gfx950: router + top-k, batch-1 expert GEMVs over the
// selected and shared experts, and the fixed-order combine.
//
// strata PR #3648 (Problem and result; Approach): the experts' per-token sums
// are split into a "local" half and a "remote" half whose sums travel as FP16;
// the FP16 -> FP32 widening is exact and the combine keeps the order of its
// additions, so the result does not depend on how the remote sums were moved.
// At decode (one token) the down projection and the combine run in one kernel:
// every output row's selected-expert terms are added in ascending expert id
// within each half, and y = (shared + local) + f32(f16(remote)).
#include "dev.h"
#include "gemv_core.h"
#include "internal.h"

#include <cmath>

namespace lps {

constexpr int MOE_MAXK = 16;
constexpr int MOE_MAXE = 256;

// ---- A10: router logits, softmax, top-k ------------------------------------------
// grid (ceil(E / 8), T): each workgroup computes 8 experts' logits for one token
// (2 per wave); the last workgroup of that token selects the top k.
struct RouteP {
  const float* x;      // [T, d]
  const float* g;
  float eps;
  const uint16_t* wr;  // [E, d] bf16
  int d, E, k;
  float* logits;       // scratch [T, E]
  int* cnt;            // scratch [T], zero on entry, left zero
  int32_t* idx;        // [T, k]
  float* w;            // [T, k]
};

__device__ __forceinline__ float bf16_dot_row(const uint16_t* row, const float* xs, int d, int lane) {
  float a = 0.f;
  const int nck = d / 8;
  for (int c = lane; c < nck; c += WAVE) {
    const u32x4 v = ld16(row + (long long)c * 8);
    acc_chunk<LPS_BF16>(v, 0, xs + c * 8, a);
  }
  return wave_sum(a);
}

__global__ __launch_bounds__(256) void k_route(RouteP p) {
  extern __shared__ float xs[];
  const int t = blockIdx.y;
  stage_x<true>(p.x + (long long)t * p.d, p.g, p.eps, p.d, xs);
  const int lane = threadIdx.x & 63, wv = threadIdx.x / 64;
  for (int q = 0; q < 2; ++q) {
    const int e = blockIdx.x * 8 + wv * 2 + q;
    if (e < p.E) {
      const float r = bf16_dot_row(p.wr + (long long)e * p.d, xs, p.d, lane);
      if (lane == 0) p.logits[(long long)t * p.E + e] = r;
    }
  }
  __shared__ int is_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) is_last = atomicAdd(p.cnt + t, 1) == int(gridDim.x) - 1;
  __syncthreads();
  if (!is_last || wv != 0) return;
  __threadfence();
  // one wave: lane holds logits e = lane + 64 q
  float r[MOE_MAXE / 64];
#pragma unroll
  for (int q = 0; q < MOE_MAXE / 64; ++q) {
    const int e = lane + 64 * q;
    r[q] = e < p.E ? __hip_atomic_load(p.logits + (long long)t * p.E + e, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT)
                   : -INFINITY;
  }
  float m = -INFINITY;
#pragma unroll
  for (int q = 0; q < MOE_MAXE / 64; ++q) m = fmaxf(m, r[q]);
  m = wave_max(m);
  float z = 0.f;
#pragma unroll
  for (int q = 0; q < MOE_MAXE / 64; ++q) z += (lane + 64 * q < p.E) ? expf(r[q] - m) : 0.f;
  z = wave_sum(z);
  // k rounds of argmax over the logits (ties -> lower id); softmax is monotone
  __shared__ float sel_pi[MOE_MAXK];
  __shared__ int sel_id[MOE_MAXK];
  float ssum = 0.f;
  for (int j = 0; j < p.k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < MOE_MAXE / 64; ++q) {
      const int e = lane + 64 * q;
      if (e < p.E && (r[q] > bv || (r[q] == bv && e < bi))) { bv = r[q]; bi = e; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    // non-finite router inputs leave nothing selectable: fall back to slot id j
    // with a NaN weight, so the step is poisoned loudly but every index stays valid
    const bool none = bi >= p.E;
    if (none) bi = j;
#pragma unroll
    for (int q = 0; q < MOE_MAXE / 64; ++q)
      if (lane + 64 * q == bi) r[q] = -INFINITY;
    const float pi = none ? __uint_as_float(0x7FC00000u) : expf(bv - m) / z;
    if (lane == 0) {
      sel_pi[j] = pi;
      sel_id[j] = bi;
    }
    ssum += pi;
  }
  if (lane == 0) {
    for (int j = 0; j < p.k; ++j) {
      p.idx[(long long)t * p.k + j] = sel_id[j];
      p.w[(long long)t * p.k + j] = sel_pi[j] / ssum;
    }
    p.cnt[t] = 0;
  }
}

static int launch_route(const lps_moe_desc* m, const float* x, int T, int32_t* idx, float* w,
                        float* logits, int* cnt, hipStream_t st) {
  RouteP p{};
  p.x = x;
  p.g = m->g_ffn;
  p.eps = m->eps;
  p.wr = static_cast<const uint16_t*>(m->w_r);
  p.d = m->d;
  p.E = m->n_experts;
  p.k = m->top_k;
  p.logits = logits;
  p.cnt = cnt;
  p.idx = idx;
  p.w = w;
  hipLaunchKernelGGL(k_route, dim3((m->n_experts + 7) / 8, T), dim3(256), size_t(m->d) * 4, st, p);
  LPS_HIP(hipGetLastError());
  return LPS_OK;
}

// ---- A11: gate/up + SwiGLU for the k selected experts and the shared one ----------
// unit u = (slot j, i): rows i and ff + i of slot j's fused gate/up matrix.
struct MoeGuP {
  const float* x;
  const float* g;
  float eps;
  const uint16_t* w_e;   // [E, 2ff, d]
  const uint16_t* w_s;   // [2ff, d]
  const int32_t* idx;    // [k]
  int d, ff, k, units, E;
  float* mbuf;           // [(k+1), ff]
};

template <int U>
__global__ __launch_bounds__(256) void k_moe_gu(MoeGuP p) {
  extern __shared__ float xs[];
  stage_x<true>(p.x, p.g, p.eps, p.d, xs);
  const int lane = threadIdx.x & 63, wv = threadIdx.x / 64;
  const int nck = p.d / 8;
  for (int u = blockIdx.x * 4 + wv; u < p.units; u += gridDim.x * 4) {
    const int j = u / p.ff, i = u - j * p.ff;
    const int e = j < p.k ? min(max(p.idx[j], 0), p.E - 1) : 0;   // indices are device data
    const uint16_t* base = j < p.k ? p.w_e + (long long)e * 2 * p.ff * p.d : p.w_s;
    const uint16_t* w0 = base + (long long)i * p.d;
    const uint16_t* w1 = base + (long long)(p.ff + i) * p.d;
    float a0 = 0.f, a1 = 0.f;
    for (int j0 = lane; j0 < nck; j0 += 64 * U) {
      u32x4 v0[U], v1[U];
#pragma unroll
      for (int q = 0; q < U; ++q) {
        const int c = j0 + 64 * q;
        if (c < nck) {
          v0[q] = ld_stream16(w0 + (long long)c * 8);
          v1[q] = ld_stream16(w1 + (long long)c * 8);
        }
      }
#pragma unroll
      for (int q = 0; q < U; ++q) {
        const int c = j0 + 64 * q;
        if (c < nck) {
          acc_chunk<LPS_BF16>(v0[q], 0, xs + c * 8, a0);
          acc_chunk<LPS_BF16>(v1[q], 0, xs + c * 8, a1);
        }
      }
    }
    a0 = wave_sum(a0);
    a1 = wave_sum(a1);
    if (lane == 0) p.mbuf[(long long)j * p.ff + i] = silu(a0) * a1;
  }
}

// ---- A11 + A12: down projections of all slots and the fixed-order combine ----------
struct MoeDownP {
  const uint16_t* w_e;   // [E, d, ff]
  const uint16_t* w_s;   // [d, ff]
  const int32_t* idx;    // [k]
  const float* wts;      // [k]
  const float* mbuf;     // [(k+1), ff]
  float* x;              // [d] residual, updated
  int d, ff, k, remote_from, E;
};

__global__ __launch_bounds__(256) void k_moe_down(MoeDownP p) {
  extern __shared__ float ms[];  // (k+1) * ff
  __shared__ int ids[MOE_MAXK];
  __shared__ float wts[MOE_MAXK];
  __shared__ int order[MOE_MAXK];   // slots sorted by ascending expert id
  __shared__ float accs[4][MOE_MAXK + 1];
  const int nm = (p.k + 1) * p.ff;
  for (int i = threadIdx.x * 4; i < nm; i += 256 * 4)
    *reinterpret_cast<f32x4*>(ms + i) = *reinterpret_cast<const f32x4*>(p.mbuf + i);
  if (threadIdx.x < p.k) {
    ids[threadIdx.x] = min(max(p.idx[threadIdx.x], 0), p.E - 1);   // indices are device data
    wts[threadIdx.x] = p.wts[threadIdx.x];
  }
  __syncthreads();
  if (threadIdx.x < p.k) {
    // rank of this slot by (expert id, slot): a permutation even if ids repeat
    int rank = 0;
    for (int j = 0; j < p.k; ++j)
      rank += ids[j] < ids[threadIdx.x] || (ids[j] == ids[threadIdx.x] && j < int(threadIdx.x));
    order[rank] = threadIdx.x;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wv = threadIdx.x / 64;
  const int nck = p.ff / 8;
  for (int r = blockIdx.x * 4 + wv; r < p.d; r += gridDim.x * 4) {
    for (int j = 0; j <= p.k; ++j) {
      const uint16_t* row = (j < p.k ? p.w_e + (long long)ids[j] * p.d * p.ff : p.w_s) +
                            (long long)r * p.ff;
      float a = 0.f;
      for (int c = lane; c < nck; c += 64) {
        const u32x4 v = ld_stream16(row + (long long)c * 8);
        acc_chunk<LPS_BF16>(v, 0, ms + j * p.ff + c * 8, a);
      }
      a = wave_sum(a);
      if (lane == 0) accs[wv][j] = a;
    }
    if (lane == 0) {
      // ascending expert id within each half
      float local = 0.f, remote = 0.f;
      for (int n = 0; n < p.k; ++n) {
        const int j = order[n];
        const float term = wts[j] * accs[wv][j];
        if (ids[j] < p.remote_from) local += term;
        else remote += term;
      }
      const float r32 = static_cast<float>(static_cast<_Float16>(remote));
      const float y = (accs[wv][p.k] + local) + r32;
      p.x[r] = p.x[r] + y;
    }
  }
}

struct MoeScratch {
  size_t logits, cnt, idx, w, mbuf, total;
};
static MoeScratch moe_scratch(const lps_moe_desc* m) {
  MoeScratch s{};
  s.cnt = 0;
  s.logits = align256(4);
  s.idx = s.logits + align256(size_t(m->n_experts) * 4);
  s.w = s.idx + align256(size_t(m->top_k) * 4);
  s.mbuf = s.w + align256(size_t(m->top_k) * 4);
  s.total = s.mbuf + align256(size_t(m->top_k + 1) * m->ff * 4);
  return s;
}

static int check_moe(const lps_moe_desc* m, const char* who) {
  LPS_REQUIRE(m, LPS_EINVAL, "%s: null MoE descriptor", who);
  LPS_REQUIRE(m->d > 0 && m->d % 8 == 0 && m->ff > 0 && m->ff % 8 == 0, LPS_EINVAL,
              "%s: d %d and ff %d must be positive multiples of 8", who, m->d, m->ff);
  LPS_REQUIRE(m->n_experts >= 1 && m->n_experts <= MOE_MAXE, LPS_EUNSUP,
              "%s: n_experts %d outside [1, %d]", who, m->n_experts, MOE_MAXE);
  LPS_REQUIRE(m->top_k >= 1 && m->top_k <= MOE_MAXK && m->top_k <= m->n_experts, LPS_EUNSUP,
              "%s: top_k %d outside [1, min(%d, n_experts)]", who, m->top_k, MOE_MAXK);
  LPS_REQUIRE(m->remote_from >= 0 && m->remote_from <= m->n_experts, LPS_EINVAL,
              "%s: remote_from %d outside [0, n_experts]", who, m->remote_from);
  LPS_REQUIRE(size_t(m->d) * 4 <= 160 * 1024 && size_t(m->top_k + 1) * m->ff * 4 <= 160 * 1024,
              LPS_EUNSUP, "%s: activations exceed 160 KiB of LDS", who);
  LPS_REQUIRE(m->g_ffn && m->w_r && m->w_gu_e && m->w_d_e && m->w_gu_s && m->w_d_s, LPS_EINVAL,
              "%s: null weight pointer", who);
  return LPS_OK;
}


}  // namespace lps

using namespace lps;

extern "C" size_t lps_moe_route_scratch_bytes(const lps_moe_desc* m, int32_t T) {
  if (check_moe(m, "lps_moe_route_scratch_bytes") || T < 0) return 0;
  return align256(size_t(T) * 4) + align256(size_t(T) * m->n_experts * 4);
}

extern "C" int lps_moe_route(const lps_moe_desc* m, const float* x, int32_t T, int32_t* idx,
                             float* w, void* scratch, size_t scratch_bytes, void* stream) {
  int rc = check_moe(m, "lps_moe_route");
  if (rc) return rc;
  LPS_REQUIRE(T >= 0 && T <= 65535, LPS_EINVAL, "lps_moe_route: T %d outside [0, 65535]", T);
  if (T == 0) return LPS_OK;
  LPS_REQUIRE(x && idx && w && scratch, LPS_EINVAL, "lps_moe_route: null pointer");
  LPS_REQUIRE(scratch_bytes >= lps_moe_route_scratch_bytes(m, T), LPS_EINVAL,
              "lps_moe_route: scratch %zu < %zu", scratch_bytes, lps_moe_route_scratch_bytes(m, T));
  rc = ensure_lds((const void*)k_route, size_t(m->d) * 4);
  if (rc) return rc;
  char* s = static_cast<char*>(scratch);
  return launch_route(m, x, T, idx, w, reinterpret_cast<float*>(s + align256(size_t(T) * 4)),
                      reinterpret_cast<int*>(s), as_stream(stream));
}

extern "C" size_t lps_moe_layer_scratch_bytes(const lps_moe_desc* m) {
  if (check_moe(m, "lps_moe_layer_scratch_bytes")) return 0;
  return moe_scratch(m).total;
}

extern "C" int lps_moe_layer_decode(const lps_moe_desc* m, float* x, void* scratch,
                                    size_t scratch_bytes, void* stream) {
  int rc = check_moe(m, "lps_moe_layer_decode");
  if (rc) return rc;
  LPS_REQUIRE(x && scratch, LPS_EINVAL, "lps_moe_layer_decode: null x or scratch");
  const MoeScratch s = moe_scratch(m);
  LPS_REQUIRE(scratch_bytes >= s.total, LPS_EINVAL, "lps_moe_layer_decode: scratch %zu < %zu",
              scratch_bytes, s.total);
  hipStream_t st = as_stream(stream);
  char* sc = static_cast<char*>(scratch);
  int32_t* idx = reinterpret_cast<int32_t*>(sc + s.idx);
  float* wts = reinterpret_cast<float*>(sc + s.w);
  float* mbuf = reinterpret_cast<float*>(sc + s.mbuf);
  if ((rc = ensure_lds((const void*)k_route, size_t(m->d) * 4)) ||
      (rc = ensure_lds((const void*)k_moe_gu<4>, size_t(m->d) * 4)) ||
      (rc = ensure_lds((const void*)k_moe_down, size_t(m->top_k + 1) * m->ff * 4)))
    return rc;
  rc = launch_route(m, x, 1, idx, wts, reinterpret_cast<float*>(sc + s.logits),
                    reinterpret_cast<int*>(sc + s.cnt), st);
  if (rc) return rc;
  MoeGuP g{};
  g.x = x;
  g.g = m->g_ffn;
  g.eps = m->eps;
  g.w_e = static_cast<const uint16_t*>(m->w_gu_e);
  g.w_s = static_cast<const uint16_t*>(m->w_gu_s);
  g.idx = idx;
  g.d = m->d;
  g.ff = m->ff;
  g.k = m->top_k;
  g.units = (m->top_k + 1) * m->ff;
  g.E = m->n_experts;
  g.mbuf = mbuf;
  int grid = (g.units + 3) / 4;
  if (grid > 2048) grid = 2048;
  hipLaunchKernelGGL(k_moe_gu<4>, dim3(grid), dim3(256), size_t(m->d) * 4, st, g);
  LPS_HIP(hipGetLastError());
  MoeDownP dn{};
  dn.w_e = static_cast<const uint16_t*>(m->w_d_e);
  dn.w_s = static_cast<const uint16_t*>(m->w_d_s);
  dn.idx = idx;
  dn.wts = wts;
  dn.mbuf = mbuf;
  dn.x = x;
  dn.d = m->d;
  dn.ff = m->ff;
  dn.k = m->top_k;
  dn.remote_from = m->remote_from;
  dn.E = m->n_experts;
  int gd = (m->d + 3) / 4;
  hipLaunchKernelGGL(k_moe_down, dim3(gd), dim3(256), size_t(m->top_k + 1) * m->ff * 4, st, dn);
  LPS_HIP(hipGetLastError());
  return LPS_OK;
}
