// GQA decode attention over a layer's KV cache (split over the context).
//
// q head h reads kv head h / G, G = nq / nkv (TP3 zero-padded dummy heads plan,
// Implementation status item 2 and Geometry: the GQA map is part of the
// weights).  One workgroup takes one (kv head, 64-row chunk) tile: the chunk's
// K and V rows are streamed once from HBM with 16-byte loads and reused by all
// G query heads of the group; scores are reduced across the lanes of a row by
// wavefront shuffles, the chunk softmax (max, sum) by wave reductions, and the
// V-weighted sums across rows by shuffles and a small LDS tree.  Each tile
// writes (m, l, o) partials; a second small launch merges every q head's chunks
// in chunk order, so the result does not depend on the order the tiles ran in
// (and no tile waits on, or fences for, another).
#include "dev.h"
#include "internal.h"

#include <cmath>

namespace lps {

constexpr int ATT_THREADS = 256;
constexpr int ATT_NW = ATT_THREADS / WAVE;
constexpr int ATT_MAXG = 8;
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

template <int KVT, int E16>
__device__ __forceinline__ void load_row(const void* base, long long elem_off, float* out) {
  const u32x4 v = ld16(static_cast<const char*>(base) + elem_off * (KVT == LPS_F32 ? 4 : 2));
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

template <int HD, int KVT>
__global__ __launch_bounds__(ATT_THREADS) void k_attn(AttnP p) {
  using C = AttnCfg<HD, KVT>;
  constexpr int E16 = C::E16, LPR = C::LPR, RPP = C::RPP;
  __shared__ float qs[ATT_MAXG][HD];
  __shared__ float sc[ATT_MAXG][ATT_CH];
  __shared__ float red[ATT_NW][ATT_MAXG][HD];

  const int chunk = blockIdx.x, g = blockIdx.y;
  const int G = p.G;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wv = tid / WAVE;
  const int li = tid % LPR, rr = tid / LPR;
  const int row0 = chunk * ATT_CH;

  for (int i = tid; i < G * HD; i += ATT_THREADS) qs[i / HD][i % HD] = p.q[(g * G) * HD + i];
  __syncthreads();

  const long long head_base = (long long)g * p.ctx_max * HD;
  // ---- scores s[h][j] = q_h . k_j * scale ----
#pragma unroll
  for (int pass = 0; pass < ATT_CH / RPP; ++pass) {
    const int jl = pass * RPP + rr;
    const int j = row0 + jl;
    float kv[E16];
    if (j < p.n) {
      load_row<KVT, E16>(p.kc, head_base + (long long)j * HD + li * E16, kv);
    } else {
#pragma unroll
      for (int e = 0; e < E16; ++e) kv[e] = 0.f;
    }
#pragma unroll
    for (int h = 0; h < ATT_MAXG; ++h) {
      if (h < G) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < E16; ++e) s = fmaf(kv[e], qs[h][li * E16 + e], s);
        s = group_sum<LPR>(s);
        if (li == 0) sc[h][jl] = (j < p.n) ? s * p.scale : -INFINITY;
      }
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
  // ---- o[h] = sum_j p[h][j] v_j ----
  float acc[ATT_MAXG][E16];
#pragma unroll
  for (int h = 0; h < ATT_MAXG; ++h)
#pragma unroll
    for (int e = 0; e < E16; ++e) acc[h][e] = 0.f;
#pragma unroll
  for (int pass = 0; pass < ATT_CH / RPP; ++pass) {
    const int jl = pass * RPP + rr;
    const int j = row0 + jl;
    if (j < p.n) {
      float vv[E16];
      load_row<KVT, E16>(p.vc, head_base + (long long)j * HD + li * E16, vv);
#pragma unroll
      for (int h = 0; h < ATT_MAXG; ++h) {
        if (h < G) {
          const float w = sc[h][jl];
#pragma unroll
          for (int e = 0; e < E16; ++e) acc[h][e] = fmaf(w, vv[e], acc[h][e]);
        }
      }
    }
  }
  // rows of one wave: lanes li + LPR*r; sum over r by shuffles
#pragma unroll
  for (int h = 0; h < ATT_MAXG; ++h) {
    if (h < G) {
#pragma unroll
      for (int e = 0; e < E16; ++e) {
        float v = acc[h][e];
#pragma unroll
        for (int o = LPR; o < WAVE; o <<= 1) v += __shfl_xor(v, o, WAVE);
        acc[h][e] = v;
      }
    }
  }
  if (lane < LPR) {
#pragma unroll
    for (int h = 0; h < ATT_MAXG; ++h)
      if (h < G)
#pragma unroll
        for (int e = 0; e < E16; ++e) red[wv][h][li * E16 + e] = acc[h][e];
  }
  __syncthreads();
  const long long ob = ((long long)g * p.nch + chunk) * G * HD;
  for (int i = tid; i < G * HD; i += ATT_THREADS) {
    const int h = i / HD, e = i % HD;
    float v = red[0][h][e];
#pragma unroll
    for (int w = 1; w < ATT_NW; ++w) v += red[w][h][e];
    p.po[ob + i] = v;
  }
}

// Merge of the chunk partials of one q head, in chunk order: M = max m_c,
// L = sum_c l_c e^(m_c - M), o = sum_c o_c e^(m_c - M) / L.  A separate launch:
// the partials of all tiles are complete when it starts (stream order), so no
// device-scope fence or counter is needed.
template <int HD>
__global__ __launch_bounds__(HD) void k_attn_merge(AttnP p) {
  const int hq = blockIdx.x;               // q head
  const int g = hq / p.G, h = hq - g * p.G;
  const int e = threadIdx.x;
  __shared__ float wsh[1024];               // e^(m_c - M) per chunk, chunk-tiled
  float M = -INFINITY;
  for (int c = e; c < p.nch; c += HD) M = fmaxf(M, p.pm[((long long)g * p.nch + c) * p.G + h]);
  // block max over the per-thread maxima (HD threads)
  __shared__ float red[HD / WAVE];
  M = wave_max(M);
  if ((e & (WAVE - 1)) == 0) red[e / WAVE] = M;
  __syncthreads();
  M = red[0];
#pragma unroll
  for (int i = 1; i < HD / WAVE; ++i) M = fmaxf(M, red[i]);
  float L = 0.f, O = 0.f;
  for (int c0 = 0; c0 < p.nch; c0 += 1024) {
    const int n = min(1024, p.nch - c0);
    __syncthreads();
    for (int c = e; c < n; c += HD)
      wsh[c] = expf(p.pm[((long long)g * p.nch + c0 + c) * p.G + h] - M);
    __syncthreads();
    for (int c = 0; c < n; ++c) {
      const long long pi = ((long long)g * p.nch + c0 + c) * p.G + h;
      const float w = wsh[c];
      L = fmaf(w, p.pl[pi], L);
      O = fmaf(w, p.po[pi * HD + e], O);
    }
  }
  p.o[(long long)hq * HD + e] = O / L;
}

static int nchunks(int rows) { return (rows + ATT_CH - 1) / ATT_CH; }

size_t attn_scratch(int nq, int nkv, int hd, int ctx_max) {
  const size_t nch = nchunks(ctx_max);
  const int G = nq / nkv;
  return 2 * align256(size_t(nkv) * nch * G * 4) + align256(size_t(nkv) * nch * G * hd * 4);
}

template <int HD, int KVT>
static void go(const AttnP& p, int nkv, hipStream_t st) {
  hipLaunchKernelGGL((k_attn<HD, KVT>), dim3(p.nch, nkv), dim3(ATT_THREADS), 0, st, p);
  hipLaunchKernelGGL((k_attn_merge<HD>), dim3(nkv * p.G), dim3(HD), 0, st, p);
}

int launch_attention(int nq, int nkv, int hd, int kvdtype, const void* kc, const void* vc,
                     int ctx_max, int n_rows, const float* q, float* o, void* scratch,
                     hipStream_t st) {
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
  switch (hd) {
    case 64: f32 ? go<64, LPS_F32>(p, nkv, st) : go<64, LPS_BF16>(p, nkv, st); break;
    case 128: f32 ? go<128, LPS_F32>(p, nkv, st) : go<128, LPS_BF16>(p, nkv, st); break;
    case 256: f32 ? go<256, LPS_F32>(p, nkv, st) : go<256, LPS_BF16>(p, nkv, st); break;
    default: return fail(LPS_EUNSUP, "attention: head dim %d not built (64, 128, 256)", hd);
  }
  LPS_HIP(hipGetLastError());
  return LPS_OK;
}

}  // namespace lps
