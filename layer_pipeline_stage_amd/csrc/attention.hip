// GQA decode attention over a layer's KV cache (split over the context).
//
// q head h reads kv head h / G, G = nq / nkv (TP3 zero-padded dummy heads plan,
// Implementation status item 2 and Geometry: the GQA map is part of the
// weights).  One workgroup takes one (kv head, 64-row chunk) tile: the chunk's
// K and V rows are streamed once from HBM with 16-byte loads and reused by all
// G query heads of the group; scores are reduced across the lanes of a row by
// DPP row operations, the chunk softmax (max, sum) by wave reductions, and the
// V tile is staged in LDS so that each thread forms whole output columns.  Each tile
// writes (m, l, o) partials; a second small launch merges every q head's chunks
// in chunk order, so the result does not depend on the order the tiles ran in
// (and no tile waits on, or fences for, another).
#include "dev.h"
#include "internal.h"

#include <cmath>

namespace lps {

constexpr int ATT_THREADS = 256;
constexpr int ATT_NW = ATT_THREADS / WAVE;
constexpr int ATT_CH = 64;  // cache rows per tile

struct AttnP {
  const void* kc;
  const void* vc;
  const float* q;
  float* o;
  float* pm;   // [nkv, nch, G]
  float* pl;   // [nkv, nch, G]
  float* po;   // [nkv, nch, G, HD]
  int G, ctx_max, n, nch;
  float scale;
};

template <int HD, int KVT>
struct AttnCfg {
  static constexpr int ESZ = KVT == LPS_F32 ? 4 : 2;
  static constexpr int E16 = 16 / ESZ;        // elements per 16-byte load
  static constexpr int LPR = HD / E16;        // lanes per cache row
  static constexpr int RPP = ATT_THREADS / LPR;  // rows per pass of the workgroup
  static constexpr int RPW = WAVE / LPR;      // rows per wave per pass
  static_assert(LPR <= WAVE && ATT_CH % RPP == 0, "unsupported head dim / cache dtype");
};

template <int KVT>
__device__ __forceinline__ void widen16(const u32x4 v, float* out) {
  if constexpr (KVT == LPS_F32) {
    out[0] = __uint_as_float(v.x);
    out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z);
    out[3] = __uint_as_float(v.w);
  } else {
    out[0] = bf16_lo(v.x);
    out[1] = bf16_hi(v.x);
    out[2] = bf16_lo(v.y);
    out[3] = bf16_hi(v.y);
    out[4] = bf16_lo(v.z);
    out[5] = bf16_hi(v.z);
    out[6] = bf16_lo(v.w);
    out[7] = bf16_hi(v.w);
  }
}

// at head dim 256 the tile's K rows and the G query heads compete for registers:
// ask for at least 3 waves per SIMD
template <int HD, int KVT, int G>
__global__ __launch_bounds__(ATT_THREADS, HD >= 256 ? 3 : 1) void k_attn(AttnP p) {
  using C = AttnCfg<HD, KVT>;
  constexpr int E16 = C::E16, LPR = C::LPR, RPP = C::RPP;
  constexpr int NP = ATT_CH / RPP;          // rows per thread
  constexpr int ESZ = C::ESZ;
  constexpr int VROW = HD * ESZ + 16;       // LDS bytes per V row (padded against bank conflicts)
  __shared__ float qs[G][HD];
  __shared__ float sc[G][ATT_CH];
  __shared__ __attribute__((aligned(16))) char vs[ATT_CH * VROW];

  const int chunk = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wv = tid / WAVE;
  const int li = tid % LPR, rr = tid / LPR;
  const int row0 = chunk * ATT_CH;
  const long long head_base = (long long)g * p.ctx_max * HD;

  // every K and V load of the tile goes out first: one HBM round trip
  u32x4 kraw[NP], vraw[NP];
#pragma unroll
  for (int ps = 0; ps < NP; ++ps) {
    const int j = row0 + ps * RPP + rr;
    if (j < p.n) {
      const long long off = (head_base + (long long)j * HD + li * E16) * ESZ;
      kraw[ps] = ld16(static_cast<const char*>(p.kc) + off);
      vraw[ps] = ld16(static_cast<const char*>(p.vc) + off);
    } else {
      kraw[ps] = vraw[ps] = u32x4{0, 0, 0, 0};   // rows past n: zero V, -inf score
    }
  }
  for (int i = tid; i < G * HD; i += ATT_THREADS) qs[i / HD][i % HD] = p.q[(g * G) * HD + i];
  // the V tile is staged in LDS for the weighted sum (read there by output column)
#pragma unroll
  for (int ps = 0; ps < NP; ++ps)
    *reinterpret_cast<u32x4*>(vs + (ps * RPP + rr) * VROW + li * 16) = vraw[ps];
  __syncthreads();

  // ---- scores s[h][j] = q_h . k_j * scale: LPR lanes per row, DPP sums ----
#pragma unroll
  for (int ps = 0; ps < NP; ++ps) {
    const int jl = ps * RPP + rr;
    const int j = row0 + jl;
    float kv[E16];
    widen16<KVT>(kraw[ps], kv);
    float s[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s[h] = 0.f;
#pragma unroll
      for (int e = 0; e < E16; ++e) s[h] = fmaf(kv[e], qs[h][li * E16 + e], s[h]);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = group_sum<LPR>(s[h]);
    if (li == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) sc[h][jl] = (j < p.n) ? s[h] * p.scale : -INFINITY;
    }
  }
  __syncthreads();
  // ---- chunk softmax: one wave per head, one row per lane ----
  for (int h = wv; h < G; h += ATT_NW) {
    const float v = sc[h][lane];
    const float m = wave_max(v);
    const float e = (v == -INFINITY) ? 0.f : expf(v - m);
    const float l = wave_sum(e);
    sc[h][lane] = e;
    if (lane == 0) {
      const long long pi = ((long long)g * p.nch + chunk) * G + h;
      p.pm[pi] = m;
      p.pl[pi] = l;
    }
  }
  __syncthreads();
  // ---- o[h][e] = sum_j p[h][j] v_j[e]: one thread per (head, column pair) ----
  const long long ob = ((long long)g * p.nch + chunk) * G * HD;
  for (int idx = tid; idx < G * (HD / 2); idx += ATT_THREADS) {
    const int h = idx / (HD / 2), e2 = idx - h * (HD / 2);
    float a0 = 0.f, a1 = 0.f;
#pragma unroll 8
    for (int j = 0; j < ATT_CH; ++j) {
      const float w = sc[h][j];
      float v0, v1;
      if constexpr (KVT == LPS_F32) {
        const f32x2 v = *reinterpret_cast<const f32x2*>(vs + j * VROW + e2 * 8);
        v0 = v.x;
        v1 = v.y;
      } else {
        const uint32_t v = *reinterpret_cast<const uint32_t*>(vs + j * VROW + e2 * 4);
        v0 = bf16_lo(v);
        v1 = bf16_hi(v);
      }
      a0 = fmaf(w, v0, a0);
      a1 = fmaf(w, v1, a1);
    }
    *reinterpret_cast<f32x2*>(p.po + ob + h * HD + 2 * e2) = f32x2{a0, a1};
  }
}

// Merge of the chunk partials of one q head, in chunk order: M = max m_c,
// L = sum_c l_c e^(m_c - M), o = sum_c o_c e^(m_c - M) / L.  A separate launch:
// the partials of all tiles are complete when it starts (stream order), so no
// device-scope fence or counter is needed.  1024 threads per head: thread
// (part, e) sums the chunks c = part (mod P) for element e, with all of its
// loads in flight at once, and the P partial sums are added in part order.
constexpr int MERGE_THREADS = 1024;
constexpr int MERGE_CH = 1024;   // chunk weights staged in LDS per round

template <int HD>
__global__ __launch_bounds__(MERGE_THREADS) void k_attn_merge(AttnP p) {
  constexpr int P = MERGE_THREADS / HD;
  constexpr int NWM = MERGE_THREADS / WAVE;
  const int hq = blockIdx.x;               // q head
  const int g = hq / p.G, h = hq - g * p.G;
  const int t = threadIdx.x, e = t % HD, part = t / HD;
  __shared__ float wsh[MERGE_CH];
  __shared__ float red[NWM];
  __shared__ float opart[P][HD];
  const long long base = (long long)g * p.nch;
  // one read of every chunk's (m, l): the first MERGE_CH chunks stay in registers
  float mreg = -INFINITY, lreg = 0.f;
  if (t < p.nch) {
    mreg = p.pm[(base + t) * p.G + h];
    lreg = p.pl[(base + t) * p.G + h];
  }
  float M = mreg;
  for (int c = t + MERGE_THREADS; c < p.nch; c += MERGE_THREADS) M = fmaxf(M, p.pm[(base + c) * p.G + h]);
  M = wave_max(M);
  if ((t & (WAVE - 1)) == 0) red[t / WAVE] = M;
  __syncthreads();
  M = red[0];
#pragma unroll
  for (int i = 1; i < NWM; ++i) M = fmaxf(M, red[i]);
  float Lp = 0.f, O = 0.f;
  const long long step = (long long)p.G * HD;
  for (int c0 = 0; c0 < p.nch; c0 += MERGE_CH) {
    const int n = min(MERGE_CH, p.nch - c0);
    __syncthreads();
    for (int c = t; c < n; c += MERGE_THREADS) {
      const long long pi = (base + c0 + c) * p.G + h;
      const bool first = c0 == 0 && c == t;
      const float w = expf((first ? mreg : p.pm[pi]) - M);
      wsh[c] = w;
      Lp = fmaf(w, first ? lreg : p.pl[pi], Lp);
    }
    __syncthreads();
    const float* po = p.po + ((base + c0) * p.G + h) * HD + e;
    int c = part;
    for (; c + 7 * P < n; c += 8 * P) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = po[(c + k * P) * step];
#pragma unroll
      for (int k = 0; k < 8; ++k) O = fmaf(wsh[c + k * P], v[k], O);
    }
    for (; c < n; c += P) O = fmaf(wsh[c], po[c * step], O);
  }
  opart[part][e] = O;
  __syncthreads();
  Lp = wave_sum(Lp);
  if ((t & (WAVE - 1)) == 0) red[t / WAVE] = Lp;
  __syncthreads();
  if (t < HD) {
    float L = 0.f;
#pragma unroll
    for (int i = 0; i < NWM; ++i) L += red[i];
    float o = opart[0][e];
#pragma unroll
    for (int q = 1; q < P; ++q) o += opart[q][e];
    p.o[(long long)hq * HD + e] = o / L;
  }
}

static int nchunks(int rows) { return (rows + ATT_CH - 1) / ATT_CH; }

size_t attn_scratch(int nq, int nkv, int hd, int ctx_max) {
  const size_t nch = nchunks(ctx_max);
  const int G = nq / nkv;
  return 2 * align256(size_t(nkv) * nch * G * 4) + align256(size_t(nkv) * nch * G * hd * 4);
}

template <int HD, int KVT>
static int go(const AttnP& p, int nkv, hipStream_t st, Stamp sp) {
  const dim3 grid(p.nch, nkv), blk(ATT_THREADS);
  hipEvent_t a = sp.start;
  switch (p.G) {
    case 1: hipExtLaunchKernelGGL((k_attn<HD, KVT, 1>), grid, blk, 0, st, a, nullptr, 0, p); break;
    case 2: hipExtLaunchKernelGGL((k_attn<HD, KVT, 2>), grid, blk, 0, st, a, nullptr, 0, p); break;
    case 4: hipExtLaunchKernelGGL((k_attn<HD, KVT, 4>), grid, blk, 0, st, a, nullptr, 0, p); break;
    case 6: hipExtLaunchKernelGGL((k_attn<HD, KVT, 6>), grid, blk, 0, st, a, nullptr, 0, p); break;
    case 8: hipExtLaunchKernelGGL((k_attn<HD, KVT, 8>), grid, blk, 0, st, a, nullptr, 0, p); break;
    default: return fail(LPS_EUNSUP, "attention: %d q heads per kv head not built (1, 2, 4, 6, 8)", p.G);
  }
  hipExtLaunchKernelGGL((k_attn_merge<HD>), dim3(nkv * p.G), dim3(MERGE_THREADS), 0, st, nullptr,
                        sp.stop, 0, p);
  return LPS_OK;
}

int launch_attention(int nq, int nkv, int hd, int kvdtype, const void* kc, const void* vc,
                     int ctx_max, int n_rows, const float* q, float* o, void* scratch,
                     hipStream_t st, Stamp sp) {
  AttnP p{};
  p.kc = kc;
  p.vc = vc;
  p.q = q;
  p.o = o;
  p.G = nq / nkv;
  p.ctx_max = ctx_max;
  p.n = n_rows;
  p.nch = nchunks(n_rows);
  p.scale = 1.0f / sqrtf(float(hd));
  const size_t nch_max = nchunks(ctx_max);
  char* s = static_cast<char*>(scratch);
  p.pm = reinterpret_cast<float*>(s);
  s += align256(size_t(nkv) * nch_max * p.G * 4);
  p.pl = reinterpret_cast<float*>(s);
  s += align256(size_t(nkv) * nch_max * p.G * 4);
  p.po = reinterpret_cast<float*>(s);
  const bool f32 = kvdtype == LPS_F32;
  int rc;
  switch (hd) {
    case 64: rc = f32 ? go<64, LPS_F32>(p, nkv, st, sp) : go<64, LPS_BF16>(p, nkv, st, sp); break;
    case 128: rc = f32 ? go<128, LPS_F32>(p, nkv, st, sp) : go<128, LPS_BF16>(p, nkv, st, sp); break;
    case 256: rc = f32 ? go<256, LPS_F32>(p, nkv, st, sp) : go<256, LPS_BF16>(p, nkv, st, sp); break;
    default: return fail(LPS_EUNSUP, "attention: head dim %d not built (64, 128, 256)", hd);
  }
  if (rc) return rc;
  LPS_HIP(hipGetLastError());
  return LPS_OK;
}

}  // namespace lps
