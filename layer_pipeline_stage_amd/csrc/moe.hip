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

#include <algorithm>
#include <cmath>

namespace lps {

constexpr int MOE_MAXK = 16;
constexpr int MOE_MAXE = 256;

// ---- A10: router logits, softmax, top-k ------------------------------------------
// Two launches.  k_route_logits: grid (ceil(E / 4), T), one expert per wave, every
// chunk load of the expert row in flight before the normed row is staged (the router
// weights are spread over many CUs: one workgroup cannot pull E * d * 2 bytes fast).
// k_route_topk: one wave per token selects the top k.  Stream order joins them, so
// no fence or counter is needed.
constexpr int ROUTE_EPB = 4;   // experts (waves) per logits workgroup
struct RouteP {
  const float* x;      // [T, d]
  const float* g;
  float eps;
  const uint16_t* wr;  // [E, d] bf16
  int d, E, k;
  float* logits;       // [T, E]
  int32_t* idx;        // [T, k]
  float* w;            // [T, k]
};

// lane l takes the 16-byte chunks l, l + 64, ... of the expert row in ascending
// order (the same per-lane split and order as the prefill router), then a wave sum
template <int CPL>
__global__ __launch_bounds__(ROUTE_EPB * WAVE) void k_route_logits(RouteP p) {
  extern __shared__ __attribute__((aligned(16))) float xs[];
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int e = blockIdx.x * ROUTE_EPB + wv;
  const int nck = p.d / 8;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.wr + (long long)(e < p.E ? e : 0) * p.d), (short)0,
      e < p.E ? p.d * 2 : 0, 0x00020000);
  // the row's loads and the gain's go out first: loads complete in issue order, so
  // the staging then waits one L2 round trip, not the expert rows
  f32x4 gpre[GPRE];
  stage_x_issue<true, ROUTE_EPB * WAVE>(p.x + (long long)t * p.d, p.g, p.d, xs, gpre);
  __builtin_amdgcn_sched_barrier(0);
  u32x4 v[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c)
    v[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (lane + WAVE * c) * 16, 0, 0));
  __builtin_amdgcn_sched_barrier(0);
  stage_x_finish<true, ROUTE_EPB * WAVE, CPL>(p.g, p.eps, p.d, xs, gpre);
  float a = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int ch = lane + WAVE * c;
    if (ch < nck) acc_chunk<LPS_BF16>(v[c], 0, xs + ch * 8, a);
  }
  a = wave_sum(a);
  if (lane == 0 && e < p.E) p.logits[(long long)t * p.E + e] = a;
}

__global__ __launch_bounds__(WAVE) void k_route_topk(RouteP p) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  // lane holds logits e = lane + 64 q
  float r[MOE_MAXE / 64];
#pragma unroll
  for (int q = 0; q < MOE_MAXE / 64; ++q) {
    const int e = lane + 64 * q;
    r[q] = e < p.E ? p.logits[(long long)t * p.E + e] : -INFINITY;
  }
  float m = -INFINITY;
#pragma unroll
  for (int q = 0; q < MOE_MAXE / 64; ++q) m = fmaxf(m, r[q]);
  m = wave_max(m);
  float z = 0.f;
#pragma unroll
  for (int q = 0; q < MOE_MAXE / 64; ++q) z += (lane + 64 * q < p.E) ? exp_native(r[q] - m) : 0.f;
  z = wave_sum(z);
  // k rounds of argmax over the logits (ties -> lower id); softmax is monotone
  __shared__ float sel_pi[MOE_MAXK];
  __shared__ int sel_id[MOE_MAXK];
  float ssum = 0.f;
  for (int j = 0; j < p.k; ++j) {
    // the largest logit (DPP max), then the lowest expert id holding it (DPP max of
    // -id over the candidates): exact selections, so ties go to the lower id
    float lv = -INFINITY;
    int li = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < MOE_MAXE / 64; ++q) {
      const int e = lane + 64 * q;
      if (e < p.E && (r[q] > lv || (r[q] == lv && e < li))) { lv = r[q]; li = e; }
    }
    const float bv = wave_max(lv);
    const float key = (lv == bv && li < p.E) ? -float(li) : -INFINITY;
    const float kb = wave_max(key);
    int bi = kb == -INFINITY ? 0x7fffffff : int(-kb);
    // non-finite router inputs leave nothing selectable: fall back to slot id j
    // with a NaN weight, so the step is poisoned loudly but every index stays valid
    const bool none = bi >= p.E;
    if (none) bi = j;
#pragma unroll
    for (int q = 0; q < MOE_MAXE / 64; ++q)
      if (lane + 64 * q == bi) r[q] = -INFINITY;
    const float pi = none ? __uint_as_float(0x7FC00000u) : exp_native(bv - m) / z;
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
  }
}

static int launch_route(const lps_moe_desc* m, const float* x, int T, float* logits, int32_t* idx,
                        float* w, hipStream_t st) {
  RouteP p{};
  p.x = x;
  p.g = m->g_ffn;
  p.eps = m->eps;
  p.wr = static_cast<const uint16_t*>(m->w_r);
  p.d = m->d;
  p.E = m->n_experts;
  p.k = m->top_k;
  p.logits = logits;
  p.idx = idx;
  p.w = w;
  const int cpl = (m->d / 8 + WAVE - 1) / WAVE;
  const size_t lds = size_t(m->d) * 4;
  const dim3 grid((m->n_experts + ROUTE_EPB - 1) / ROUTE_EPB, T);
  int rc;
#define LPS_ROUTE(C)                                                                  \
  do {                                                                                \
    if ((rc = ensure_lds((const void*)k_route_logits<C>, lds))) return rc;           \
    hipLaunchKernelGGL(k_route_logits<C>, grid, dim3(ROUTE_EPB * WAVE), lds, st, p);  \
  } while (0)
  if (cpl <= 1) LPS_ROUTE(1);
  else if (cpl <= 2) LPS_ROUTE(2);
  else if (cpl <= 4) LPS_ROUTE(4);
  else LPS_ROUTE(8);
#undef LPS_ROUTE
  LPS_HIP(hipGetLastError());
  hipLaunchKernelGGL(k_route_topk, dim3(T), dim3(WAVE), 0, st, p);
  LPS_HIP(hipGetLastError());
  return LPS_OK;
}

// ---- A11: gate/up + SwiGLU for the k selected experts and the shared one ----------
// launch_moe_gu (the weight-streaming GEMV with an expert-table row map).

// ---- A11 + A12: down projections of all slots and the fixed-order combine ----------
// launch_moe_down (the weight-streaming GEMV over every slot's down matrix, each
// slot's SwiGLU row staged side by side) writes z[j, r]; k_moe_combine then adds,
// per output row r, the k weighted terms in ascending expert id within each half:
// y = (shared + local) + f32(f16(remote)), x[r] += y.
struct MoeCombP {
  const int32_t* idx;    // [k]
  const float* wts;      // [k]
  const float* z;        // [(k+1), d]
  float* x;              // [d] residual, updated
  float* tee0;           // [d] or NULL: the updated row, also stored here and to tee1
  float* tee1;
  int d, k, remote_from, E;
};

__global__ __launch_bounds__(256) void k_moe_combine(MoeCombP p) {
  __shared__ int ids[MOE_MAXK];
  __shared__ float wts[MOE_MAXK];
  __shared__ int order[MOE_MAXK];   // slots sorted by ascending expert id
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
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= p.d) return;
  {
    // every term is rounded before it is added: no product is fused into a sum
#pragma clang fp contract(off)
    float local = 0.f, remote = 0.f;
    for (int n = 0; n < p.k; ++n) {
      const int j = order[n];
      const float term = wts[j] * p.z[(long long)j * p.d + r];
      if (ids[j] < p.remote_from) local += term;
      else remote += term;
    }
    const float r32 = static_cast<float>(static_cast<_Float16>(remote));
    const float y = (p.z[(long long)p.k * p.d + r] + local) + r32;
    const float v = p.x[r] + y;
    p.x[r] = v;
    if (p.tee0) {
      p.tee0[r] = v;
      p.tee1[r] = v;
    }
  }
}

// The down projections and the combine in one launch (rows of up to 256 chunks,
// ff <= 2048; longer rows take launch_moe_down and k_moe_combine).  A workgroup takes MOE_DC_R output rows for every slot: wave w walks the
// slots j = w, w + nw, ... and for each the MOE_DC_R rows of slot j's down matrix,
// each row's 16-byte chunks on the lanes as in the weight-streaming GEMV (lane l:
// chunks l, l + 64, ...; chunks past the row load as zeros and meet zero
// activations), so every z[j, r] is the GEMV's own value; the terms then meet in
// LDS and the first MOE_DC_R threads add them as k_moe_combine does.
#ifndef LPS_MOE_DC_R
#define LPS_MOE_DC_R 4
#endif
constexpr int MOE_DC_R = LPS_MOE_DC_R;   // output rows per workgroup
constexpr int MOE_DC_MAXW = 16;   // waves per workgroup at most
struct MoeDownCombP {
  const uint16_t* w_e;   // [E, d, ff] bf16
  const uint16_t* w_s;   // [d, ff] bf16
  const int32_t* idx;    // [k]
  const float* wts;      // [k]
  const float* m;        // [(k+1), ff] SwiGLU rows (slot k: the shared expert)
  float* x;              // [d] residual, updated
  float* tee0;           // [d] or NULL: the updated row, also stored here and to tee1
  float* tee1;
  int d, ff, k, remote_from, E;
};

template <int CPL>
__global__ __launch_bounds__(MOE_DC_MAXW * WAVE) void k_moe_down_combine(MoeDownCombP p) {
  __shared__ int ids[MOE_MAXK];
  __shared__ float wts[MOE_MAXK];
  __shared__ int order[MOE_MAXK];
  __shared__ float zs[MOE_MAXK + 1][MOE_DC_R];
  const int lane = threadIdx.x & (WAVE - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  const int nw = blockDim.x / WAVE;
  const int r0 = blockIdx.x * MOE_DC_R;
  const int nck = p.ff / 8;
  const int rowb = p.ff * 2;
  if (threadIdx.x < p.k) {
    ids[threadIdx.x] = min(max(p.idx[threadIdx.x], 0), p.E - 1);   // indices are device data
    wts[threadIdx.x] = p.wts[threadIdx.x];
  }
  for (int j = wv; j <= p.k; j += nw) {
    const int e = j < p.k ? min(max(p.idx[j], 0), p.E - 1) : 0;
    const uint16_t* base = j < p.k ? p.w_e + (long long)e * p.d * p.ff : p.w_s;
    u32x4 v[MOE_DC_R][CPL];
#pragma unroll
    for (int q = 0; q < MOE_DC_R; ++q) {
      const int r = r0 + q;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(base + (long long)(r < p.d ? r : 0) * p.ff), (short)0,
          r < p.d ? rowb : 0, 0x00020000);
#pragma unroll
      for (int c = 0; c < CPL; ++c)
        v[q][c] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (lane + WAVE * c) * 16, 0, 2));
    }
    f32x4 x0[CPL], x1[CPL];
    const float* mj = p.m + (long long)j * p.ff;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ch = lane + WAVE * c;
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      x0[c] = ch < nck ? *reinterpret_cast<const f32x4*>(mj + ch * 8) : zero;
      x1[c] = ch < nck ? *reinterpret_cast<const f32x4*>(mj + ch * 8 + 4) : zero;
    }
#pragma unroll
    for (int q = 0; q < MOE_DC_R; ++q) {
      // the products of acc_chunk<LPS_BF16>, in its order
      float a = 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const u32x4 w = v[q][c];
        a = fmaf(bf16_lo(w.x), x0[c].x, a);
        a = fmaf(bf16_hi(w.x), x0[c].y, a);
        a = fmaf(bf16_lo(w.y), x0[c].z, a);
        a = fmaf(bf16_hi(w.y), x0[c].w, a);
        a = fmaf(bf16_lo(w.z), x1[c].x, a);
        a = fmaf(bf16_hi(w.z), x1[c].y, a);
        a = fmaf(bf16_lo(w.w), x1[c].z, a);
        a = fmaf(bf16_hi(w.w), x1[c].w, a);
      }
      a = wave_sum(a);
      if (lane == 0) zs[j][q] = a;
    }
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
  if (threadIdx.x < MOE_DC_R && r0 + int(threadIdx.x) < p.d) {
#pragma clang fp contract(off)
    // as k_moe_combine: every term rounded before it is added
    const int q = threadIdx.x, r = r0 + q;
    float local = 0.f, remote = 0.f;
    for (int n = 0; n < p.k; ++n) {
      const int j = order[n];
      const float term = wts[j] * zs[j][q];
      if (ids[j] < p.remote_from) local += term;
      else remote += term;
    }
    const float r32 = static_cast<float>(static_cast<_Float16>(remote));
    const float y = (zs[p.k][q] + local) + r32;
    const float v = p.x[r] + y;
    p.x[r] = v;
    if (p.tee0) {
      p.tee0[r] = v;
      p.tee1[r] = v;
    }
  }
}

struct MoeScratch {
  size_t idx, w, logits, mbuf, z, total;
};
static MoeScratch moe_scratch(const lps_moe_desc* m) {
  MoeScratch s{};
  s.idx = 0;
  s.w = s.idx + align256(size_t(MOE_MAXK) * 4);
  s.logits = s.w + align256(size_t(m->top_k) * 4);
  s.mbuf = s.logits + align256(size_t(m->n_experts) * 4);
  s.z = s.mbuf + align256(size_t(m->top_k + 1) * m->ff * 4);
  s.total = s.z + align256(size_t(m->top_k + 1) * m->d * 4);
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
  LPS_REQUIRE(size_t(m->d) * 4 <= 160 * 1024 && (size_t(m->top_k + 1) * m->ff + 8) * 4 <= 160 * 1024,
              LPS_EUNSUP, "%s: activations exceed 160 KiB of LDS", who);
  LPS_REQUIRE(m->g_ffn && m->w_r && m->w_gu_e && m->w_d_e && m->w_gu_s && m->w_d_s, LPS_EINVAL,
              "%s: null weight pointer", who);
  return LPS_OK;
}


}  // namespace lps

using namespace lps;

extern "C" size_t lps_moe_route_scratch_bytes(const lps_moe_desc* m, int32_t T) {
  if (check_moe(m, "lps_moe_route_scratch_bytes") || T < 0) return 0;
  return align256(size_t(T) * m->n_experts * 4);
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
  LPS_REQUIRE(m->d <= 4096, LPS_EUNSUP, "lps_moe_route: d %d > 4096", m->d);
  return launch_route(m, x, T, static_cast<float*>(scratch), idx, w, as_stream(stream));
}

extern "C" size_t lps_moe_layer_scratch_bytes(const lps_moe_desc* m) {
  if (check_moe(m, "lps_moe_layer_scratch_bytes")) return 0;
  return moe_scratch(m).total;
}

namespace lps {
int check_moe_decode(const lps_moe_desc* m, const char* who) {
  int rc = check_moe(m, who);
  if (rc) return rc;
  LPS_REQUIRE(m->d <= 4096 && m->d % 8 == 0, LPS_EUNSUP, "%s: d %d (a multiple of 8, <= 4096)", who,
              m->d);
  return LPS_OK;
}
size_t moe_decode_scratch(const lps_moe_desc* m) { return moe_scratch(m).total; }

// One MoE FFN layer for one token (validated by the caller): route, the selected
// and the shared expert's gate/up + SwiGLU and down GEMVs, the ordered combine.
int moe_decode(const lps_moe_desc* m, float* x, void* scratch, hipStream_t st, float* tee0,
               float* tee1) {
  const MoeScratch s = moe_scratch(m);
  char* sc = static_cast<char*>(scratch);
  int32_t* idx = reinterpret_cast<int32_t*>(sc + s.idx);
  float* wts = reinterpret_cast<float*>(sc + s.w);
  float* mbuf = reinterpret_cast<float*>(sc + s.mbuf);
  int rc = launch_route(m, x, 1, reinterpret_cast<float*>(sc + s.logits), idx, wts, st);
  if (rc) return rc;
  rc = launch_moe_gu(m->w_gu_e, m->w_gu_s, idx, m->n_experts, m->top_k, m->ff, m->d, x, m->g_ffn,
                     m->eps, mbuf, st, timer_take(LPS_KIND_MOE_GU));
  if (rc) return rc;
  const int cpl = (m->ff / 8 + WAVE - 1) / WAVE;
  if (cpl <= 4) {   // rows of up to 256 chunks: down projections and combine in one launch
    MoeDownCombP dp{};
    dp.w_e = static_cast<const uint16_t*>(m->w_d_e);
    dp.w_s = static_cast<const uint16_t*>(m->w_d_s);
    dp.idx = idx;
    dp.wts = wts;
    dp.m = mbuf;
    dp.x = x;
    if (tee0 && tee1) {
      dp.tee0 = tee0;
      dp.tee1 = tee1;
    }
    dp.d = m->d;
    dp.ff = m->ff;
    dp.k = m->top_k;
    dp.remote_from = m->remote_from;
    dp.E = m->n_experts;
    const dim3 grid((m->d + MOE_DC_R - 1) / MOE_DC_R);
    const dim3 block(std::min(m->top_k + 1, MOE_DC_MAXW) * WAVE);
    const Stamp sp = timer_take(LPS_KIND_MOE_DOWN);
#define LPS_DC(C) LPS_LAUNCH(k_moe_down_combine<C>, grid, block, 0, st, sp.start, sp.stop, dp)
    if (cpl <= 1) LPS_DC(1);
    else if (cpl <= 2) LPS_DC(2);
    else LPS_DC(4);
#undef LPS_DC
    LPS_HIP(hipGetLastError());
    return LPS_OK;
  }
  float* z = reinterpret_cast<float*>(sc + s.z);
  rc = launch_moe_down(m->w_d_e, m->w_d_s, idx, m->n_experts, m->top_k, m->d, m->ff, mbuf, z, st,
                       timer_take(LPS_KIND_MOE_DOWN));
  if (rc) return rc;
  MoeCombP cp{};
  cp.idx = idx;
  cp.wts = wts;
  cp.z = z;
  cp.x = x;
  if (tee0 && tee1) {
    cp.tee0 = tee0;
    cp.tee1 = tee1;
  }
  cp.d = m->d;
  cp.k = m->top_k;
  cp.remote_from = m->remote_from;
  cp.E = m->n_experts;
  hipLaunchKernelGGL(k_moe_combine, dim3((m->d + 255) / 256), dim3(256), 0, st, cp);
  LPS_HIP(hipGetLastError());
  return LPS_OK;
}
}  // namespace lps

extern "C" int lps_moe_layer_decode(const lps_moe_desc* m, float* x, void* scratch,
                                    size_t scratch_bytes, void* stream) {
  int rc = check_moe_decode(m, "lps_moe_layer_decode");
  if (rc) return rc;
  LPS_REQUIRE(x && scratch, LPS_EINVAL, "lps_moe_layer_decode: null x or scratch");
  const MoeScratch s = moe_scratch(m);
  LPS_REQUIRE(scratch_bytes >= s.total, LPS_EINVAL, "lps_moe_layer_decode: scratch %zu < %zu",
              scratch_bytes, s.total);
  return moe_decode(m, x, scratch, as_stream(stream));
}
