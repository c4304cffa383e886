// Batch-1 weight-streaming GEMV for gfx950, with the decode path's fused
// prologues and epilogues.
//
// Decode at batch 1 reads every weight byte once per token and does ~1 flop per
// byte, so these kernels are HBM-bound (ninfer "Multi-GPU: layer pipeline
// stages", What it is and is not: decode is weight-bandwidth-bound).  Design:
//  - one wave (64 lanes) computes one "unit" of two rows; lane l takes the
//    16-byte chunks l, l+64, l+128, ... of both rows, so a wave issues fully
//    coalesced 1 KiB loads per instruction and keeps U of them in flight per
//    row; every chunk of a row always lands on the same lane in the same order
//    whatever the row length, so zero chunks appended at the end of K (the
//    padded dummy columns) leave each lane's partial sum, and the result,
//    bit for bit unchanged;
//  - the activation vector (f32, optionally RMS-normalised on the way in) sits
//    in LDS, read once per block from L2 and shared by the block's waves;
//  - the two rows of a unit are chosen so that the epilogue has what it needs:
//    rows (i, i + hd/2) of one head for RoPE, rows (i, ff + i) for SwiGLU;
//  - MXFP4 chunks are 16 bytes of codes = one 32-value e8m0 group, decoded by
//    the gfx950 scaled FP4 -> f32 conversion; the K loop is bounded per group,
//    so no K % 128 assumption exists (TP3 zero-padded dummy heads plan,
//    Implementation status, item 1).
#include "dev.h"
#include "gemv_core.h"
#include "internal.h"

#include <cmath>

namespace lps {

enum { EPI_STORE = LPS_EPI_STORE, EPI_ADD = LPS_EPI_ADD, EPI_SWIGLU = LPS_EPI_SWIGLU, EPI_QKV = 3,
       EPI_LOGITS = 4 };

struct GemvP {
  const uint8_t* w;
  const uint8_t* s;
  long long wrow;   // bytes per weight row
  long long srow;   // bytes per scale row (MXFP4)
  int N, K, units;
  const float* x;
  const float* g;
  float eps;
  float* y;
  // QKV epilogue
  int nq, nkv, hd, pos, ctx_max, kvdtype;
  void* kc;
  void* vc;
  // cos / sin of pos * base^(-2i/hd) for i < hd/2, formed on the host in double
  float rope[2 * 128];
  // LM-head epilogue: every wave's (max, lowest index of it) over its rows
  float* pval;
  int* pidx;
};

template <int EPI>
__device__ __forceinline__ void unit_rows(const GemvP& p, int u, int& r0, int& r1) {
  if constexpr (EPI == EPI_SWIGLU) {
    r0 = u;
    r1 = u + (p.N >> 1);
  } else if constexpr (EPI == EPI_QKV) {
    const int half = p.hd >> 1;
    const int hh = u / half, i = u - hh * half;
    r0 = hh * p.hd + i;
    r1 = r0 + half;
  } else {
    r0 = 2 * u;
    r1 = (2 * u + 1 < p.N) ? 2 * u + 1 : -1;
  }
}

__device__ __forceinline__ void store_kv(void* base, int kvdtype, long long off, float v) {
  if (kvdtype == LPS_F32)
    reinterpret_cast<float*>(base)[off] = v;
  else
    reinterpret_cast<uint16_t*>(base)[off] = f32_to_bf16(v);
}

template <int EPI>
__device__ __forceinline__ void epilogue(const GemvP& p, int u, int r0, int r1, float a0, float a1) {
  if constexpr (EPI == EPI_STORE || EPI == EPI_LOGITS) {
    p.y[r0] = a0;
    if (r1 >= 0) p.y[r1] = a1;
  } else if constexpr (EPI == EPI_ADD) {
    p.y[r0] += a0;
    if (r1 >= 0) p.y[r1] += a1;
  } else if constexpr (EPI == EPI_SWIGLU) {
    p.y[u] = silu(a0) * a1;
  } else {  // QKV: rotate q and k heads at pos, store q, append k and v to the caches
    const int half = p.hd >> 1;
    const int hh = u / half, i = u - hh * half;
    float o0 = a0, o1 = a1;
    if (hh < p.nq + p.nkv) {
      const float cs = p.rope[2 * i], sn = p.rope[2 * i + 1];
      o0 = a0 * cs - a1 * sn;
      o1 = a0 * sn + a1 * cs;
    }
    if (hh < p.nq) {
      p.y[r0] = o0;
      p.y[r1] = o1;
    } else {
      const bool is_k = hh < p.nq + p.nkv;
      const int gkv = is_k ? hh - p.nq : hh - p.nq - p.nkv;
      const long long off = ((long long)gkv * p.ctx_max + p.pos) * p.hd + i;
      void* base = is_k ? p.kc : p.vc;
      store_kv(base, p.kvdtype, off, o0);
      store_kv(base, p.kvdtype, off + half, o1);
    }
  }
}

// threads per GEMV workgroup and the grid cap (workgroups); a block stages the
// activation vector once for all of its waves
#ifndef LPS_GEMV_NT
#define LPS_GEMV_NT 256
#endif
#ifndef LPS_GEMV_MAXB
#define LPS_GEMV_MAXB 2048
#endif
constexpr int GEMV_NT = LPS_GEMV_NT;

// Loads of one batch (U chunks of both rows of a unit), then its FMAs.  Kept as
// macros over local arrays: the compiler then issues all 2U loads of a batch
// before the first wait.
#define GEMV_LOAD(J0)                                              \
  _Pragma("unroll") for (int i = 0; i < U; ++i) {                  \
    const int c = (J0) + WAVE * i;                                 \
    if (c < nck) {                                                 \
      v0[i] = ld_stream16(w0 + (long long)c * 16);                 \
      v1[i] = ld_stream16(w1 + (long long)c * 16);                 \
      if constexpr (WT == LPS_MXFP4) {                             \
        sc0[i] = s0[c];                                            \
        sc1[i] = s1[c];                                            \
      } else {                                                     \
        sc0[i] = sc1[i] = 0;                                       \
      }                                                            \
    } else {                                                       \
      v0[i] = v1[i] = u32x4{0, 0, 0, 0};                           \
      sc0[i] = sc1[i] = 127;                                       \
    }                                                              \
  }
#define GEMV_FMA(J0)                                               \
  _Pragma("unroll") for (int i = 0; i < U; ++i) {                  \
    const int c = (J0) + WAVE * i;                                 \
    if (c < nck) {                                                 \
      acc_chunk<WT>(v0[i], sc0[i], xs + c * CH, a0);               \
      acc_chunk<WT>(v1[i], sc1[i], xs + c * CH, a1);               \
    }                                                              \
  }
#define GEMV_ROWS(UU)                                              \
  int r0, r1;                                                      \
  unit_rows<EPI>(p, (UU), r0, r1);                                 \
  const int rr1 = r1 >= 0 ? r1 : r0;                               \
  const uint8_t* w0 = p.w + (long long)r0 * p.wrow;                \
  const uint8_t* w1 = p.w + (long long)rr1 * p.wrow;               \
  const uint8_t* s0 = nullptr;                                     \
  const uint8_t* s1 = nullptr;                                     \
  if constexpr (WT == LPS_MXFP4) {                                 \
    s0 = p.s + (long long)r0 * p.srow;                             \
    s1 = p.s + (long long)rr1 * p.srow;                            \
  }

template <int EPI>
__device__ __forceinline__ void finish(const GemvP& p, int u, int r0, int r1, float a0, float a1,
                                       int lane, float& best, int& bidx) {
  a0 = wave_sum(a0);
  a1 = wave_sum(a1);
  if (lane == 0) epilogue<EPI>(p, u, r0, r1, a0, a1);
  if constexpr (EPI == EPI_LOGITS) {
    if (a0 > best) { best = a0; bidx = r0; }
    if (r1 >= 0 && a1 > best) { best = a1; bidx = r1; }
  }
}

// PF: for launches where a wave's first unit fits one batch (K <= 64 U chunks),
// that batch is loaded before the activation vector is staged, so its HBM
// latency overlaps the staging and the norm; further units take the plain path.
template <int WT, int EPI, int U, bool NORM, bool PF>
__global__ __launch_bounds__(GEMV_NT) void k_gemv(GemvP p) {
  extern __shared__ float xs[];
  constexpr int CH = Fmt<WT>::CH;
  constexpr int NW = GEMV_NT / WAVE;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wv = threadIdx.x / WAVE;
  const int nck = p.K / CH;
  float best = -INFINITY;   // EPI_LOGITS: rows rise with u, so '>' keeps the first maximum
  int bidx = 0x7fffffff;
  int u = blockIdx.x * NW + wv;
  if constexpr (PF) {
    const int uu = u < p.units ? u : p.units - 1;   // waves without a unit load a valid row
    GEMV_ROWS(uu)
    u32x4 v0[U], v1[U];
    uint32_t sc0[U], sc1[U];
    GEMV_LOAD(lane)
    stage_x<NORM, GEMV_NT>(p.x, p.g, p.eps, p.K, xs);
    if (u < p.units) {
      float a0 = 0.f, a1 = 0.f;
      GEMV_FMA(lane)
      finish<EPI>(p, u, r0, r1, a0, a1, lane, best, bidx);
    }
    u += gridDim.x * NW;
  } else {
    stage_x<NORM, GEMV_NT>(p.x, p.g, p.eps, p.K, xs);
  }
  for (; u < p.units; u += gridDim.x * NW) {
    GEMV_ROWS(u)
    float a0 = 0.f, a1 = 0.f;
    for (int j0 = lane; j0 < nck; j0 += WAVE * U) {
      u32x4 v0[U], v1[U];
      uint32_t sc0[U], sc1[U];
      GEMV_LOAD(j0)
      GEMV_FMA(j0)
    }
    finish<EPI>(p, u, r0, r1, a0, a1, lane, best, bidx);
  }
  if constexpr (EPI == EPI_LOGITS) {
    if (lane == 0) {
      p.pval[blockIdx.x * NW + wv] = best;
      p.pidx[blockIdx.x * NW + wv] = bidx;
    }
  }
}
#undef GEMV_LOAD
#undef GEMV_FMA
#undef GEMV_ROWS

// A16 argmax over the LM head's per-wave partials (value, lowest index with
// that value), one workgroup: max with ties to the lower index is an exact
// selection, so any order gives the same answer.  Its own launch after the head
// GEMV: no fence or counter is needed.
__global__ __launch_bounds__(1024) void k_argmax(const float* pval, const int* pidx, int n, int* out) {
  float b = -INFINITY;
  int ix = 0x7fffffff;
  for (int i = threadIdx.x; i < n; i += 1024) {
    const float v = pval[i];
    const int j = pidx[i];
    if (v > b || (v == b && j < ix)) { b = v; ix = j; }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ob = __shfl_xor(b, o, WAVE);
    const int oi = __shfl_xor(ix, o, WAVE);
    if (ob > b || (ob == b && oi < ix)) { b = ob; ix = oi; }
  }
  __shared__ float bv[16];
  __shared__ int bi[16];
  const int wv = threadIdx.x / WAVE;
  if ((threadIdx.x & (WAVE - 1)) == 0) { bv[wv] = b; bi[wv] = ix; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < 16; ++i)
      if (bv[i] > b || (bv[i] == b && bi[i] < ix)) { b = bv[i]; ix = bi[i]; }
    // no maximum (all NaN): report 0 rather than an index outside the vocabulary
    *out = ix == 0x7fffffff ? 0 : ix;
  }
}

// ---- launch configuration ---------------------------------------------------
static int max_blocks() { return LPS_GEMV_MAXB; }



template <int WT, int EPI, bool NORM>
static int launch_t(const GemvP& p, hipStream_t st, Stamp sp) {
  const int NW = GEMV_NT / WAVE;
  int grid = (p.units + NW - 1) / NW;
  if (grid > max_blocks()) grid = max_blocks();
  if (grid < 1) grid = 1;
  const size_t lds = size_t(p.K) * sizeof(float);
  constexpr int CH = Fmt<WT>::CH;
  const int per_lane = (p.K / CH + WAVE - 1) / WAVE;
  // keep up to 8 (bf16 / f32) or 4 (MXFP4, whose decode needs more registers)
  // chunk loads per row in flight per lane; prefetch under the staging when a
  // wave has at most two units
  const bool pf = per_lane <= (per_lane <= 4 || WT == LPS_MXFP4 ? 4 : 8) && p.units <= 2 * grid * NW;
#define LPS_GO(UU, PFV)                                                                     \
  do {                                                                                      \
    int rc_ = ensure_lds((const void*)k_gemv<WT, EPI, UU, NORM, PFV>, lds);                 \
    if (rc_) return rc_;                                                                    \
    hipExtLaunchKernelGGL((k_gemv<WT, EPI, UU, NORM, PFV>), dim3(grid), dim3(GEMV_NT), lds, \
                          st, sp.start, sp.stop, 0, p);                                     \
  } while (0)
  if (per_lane <= 4 || WT == LPS_MXFP4) {
    if (pf) LPS_GO(4, true);
    else LPS_GO(4, false);
  } else {
    if (pf) LPS_GO(8, true);
    else LPS_GO(8, false);
  }
#undef LPS_GO
  LPS_HIP(hipGetLastError());
  return LPS_OK;
}

template <int EPI, bool NORM>
static int launch_wt(int wdtype, const GemvP& p, hipStream_t st, Stamp sp) {
  switch (wdtype) {
    case LPS_F32: return launch_t<LPS_F32, EPI, NORM>(p, st, sp);
    case LPS_BF16: return launch_t<LPS_BF16, EPI, NORM>(p, st, sp);
    case LPS_MXFP4: return launch_t<LPS_MXFP4, EPI, NORM>(p, st, sp);
  }
  return fail(LPS_EINVAL, "gemv: unknown wdtype %d", wdtype);
}

static void set_rows(GemvP& p, int wdtype, int K) {
  if (wdtype == LPS_F32) p.wrow = (long long)K * 4;
  else if (wdtype == LPS_BF16) p.wrow = (long long)K * 2;
  else { p.wrow = K / 2; p.srow = K / 32; }
}

int launch_gemv(int wdtype, const void* w, const uint8_t* s, int N, int K, const float* x,
                const float* g, float eps, float* y, int mode, hipStream_t st, Stamp sp) {
  GemvP p{};
  p.w = static_cast<const uint8_t*>(w);
  p.s = s;
  p.N = N;
  p.K = K;
  p.x = x;
  p.g = g;
  p.eps = eps;
  p.y = y;
  set_rows(p, wdtype, K);
  const bool norm = g != nullptr;
  if (mode == EPI_SWIGLU) {
    p.units = N / 2;
    return norm ? launch_wt<EPI_SWIGLU, true>(wdtype, p, st, sp) : launch_wt<EPI_SWIGLU, false>(wdtype, p, st, sp);
  }
  p.units = (N + 1) / 2;
  if (mode == EPI_ADD)
    return norm ? launch_wt<EPI_ADD, true>(wdtype, p, st, sp) : launch_wt<EPI_ADD, false>(wdtype, p, st, sp);
  return norm ? launch_wt<EPI_STORE, true>(wdtype, p, st, sp) : launch_wt<EPI_STORE, false>(wdtype, p, st, sp);
}

int launch_qkv(const QkvArgs& a, hipStream_t st, Stamp sp) {
  const lps_layer_desc* L = a.L;
  GemvP p{};
  p.w = static_cast<const uint8_t*>(L->w_qkv);
  p.s = L->s_qkv;
  p.N = (L->nq + 2 * L->nkv) * L->hd;
  p.K = L->d;
  p.x = a.x;
  p.g = L->g_attn;
  p.eps = L->eps;
  p.y = a.q;
  p.units = p.N / 2;
  p.nq = L->nq;
  p.nkv = L->nkv;
  p.hd = L->hd;
  p.pos = a.pos;
  p.ctx_max = L->ctx_max;
  p.kvdtype = L->kvdtype;
  // the rotation angle pos * theta_i reaches ~1e4 rad: form it and its cos / sin
  // in double, once per launch, and hand the f32 values to every block
  for (int i = 0; i < L->hd / 2; ++i) {
    const double theta = std::pow(double(L->rope_base), -2.0 * double(i) / double(L->hd));
    const double ang = double(a.pos) * theta;
    p.rope[2 * i] = float(std::cos(ang));
    p.rope[2 * i + 1] = float(std::sin(ang));
  }
  p.kc = L->k_cache;
  p.vc = L->v_cache;
  set_rows(p, L->wdtype, L->d);
  return launch_wt<EPI_QKV, true>(L->wdtype, p, st, sp);
}

size_t head_scratch(const lps_head_desc* h) {
  (void)h;
  return 2 * align256(size_t(LPS_GEMV_MAXB) * (GEMV_NT / WAVE) * 4);
}

int launch_head(const lps_head_desc* h, const float* x, float* logits, int32_t* tok, void* scratch,
                size_t bytes, hipStream_t st, Stamp sp) {
  (void)bytes;
  GemvP p{};
  p.w = static_cast<const uint8_t*>(h->w_lm);
  p.N = h->vocab;
  p.K = h->d;
  p.x = x;
  p.g = h->g_out;
  p.eps = h->eps;
  p.y = logits;
  p.units = (h->vocab + 1) / 2;
  set_rows(p, h->wdtype, h->d);
  char* sc = static_cast<char*>(scratch);
  p.pval = reinterpret_cast<float*>(sc);
  p.pidx = reinterpret_cast<int*>(sc + align256(size_t(LPS_GEMV_MAXB) * (GEMV_NT / WAVE) * 4));
  int rc = launch_wt<EPI_LOGITS, true>(h->wdtype, p, st, Stamp{sp.start, nullptr});
  if (rc) return rc;
  const int NW = GEMV_NT / WAVE;
  int grid = (p.units + NW - 1) / NW;
  if (grid > max_blocks()) grid = max_blocks();
  hipExtLaunchKernelGGL(k_argmax, dim3(1), dim3(1024), 0, st, nullptr, sp.stop, 0, p.pval, p.pidx,
                        grid * NW, tok);
  LPS_HIP(hipGetLastError());
  return LPS_OK;
}

}  // namespace lps
