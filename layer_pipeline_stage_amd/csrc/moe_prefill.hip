// MoE FFN layer over a prefill chunk of T tokens on gfx950.
//
// strata PR #3648 (Problem and result; Approach): every MoE layer of a prompt
// chunk routes its tokens, groups them per expert, runs the experts, and
// combines per-token sums where one half of the experts returns FP16 sums in
// pieces, converted exactly and added in a fixed order.  Here all experts run
// on one GPU: the expert matmuls are grouped GEMMs on the bf16 matrix cores.
//
// Steps (each its own launch, in stream order, so no kernel waits on another):
//  0. norm: RMSNorm rows (f32) rounded to their bf16 copy for the expert GEMMs,
//     one wave per row (rows wider than 2304: per 8-token tile).  The activation half of the piece transfer starts here: on the
//     second stream the bf16 rows go to the remote half's own copy in P row
//     pieces while the main stream routes and groups (strata PR #3648, Approach:
//     the activations leave before the router; both halves read the same values,
//     so the pieces change timing, not results).
//  1. route: the same RMSNorm recomputed per tile (bit for bit), router logits
//     from the f32 rows on the f32 matrix cores for 16 tokens x 64 experts per
//     workgroup (rows wider than 2300: on the vector ALUs, with the decode
//     router's lane / chunk split), softmax, top-k by logit with ties to the
//     lower id, weights renormalised over the k.
//  2. group: per expert, the tokens that selected it, in token order (a stable
//     counting sort: each expert's list is a compaction of the token sequence).
//  3. tiles: per-expert offsets and two lists of 256-row tiles: the local
//     experts in ascending id then the shared expert over all tokens (main
//     stream), and the remote experts (second stream, reading the remote copy of
//     the rows once every piece has landed and the lists exist).
//  4. GEMM1: [rows x d] x [d x 2ff] on MFMA 32x32x16 bf16 -> f32; the gate and
//     up columns of one output sit in the same lanes, so SwiGLU is applied in
//     registers; the product is rounded to bf16 for GEMM2.
//  5. GEMM2: [rows x ff] x [ff x d] -> f32, scaled by the token's gate weight
//     and written to the token's slot (the shared expert to its own buffer).
//  6. halves: per token, the selected experts' terms in ascending expert id:
//     local (f32) and remote, the latter rounded to f16.
//  7. combine (lps_moe_combine): the f16 sums widened piece by piece on the
//     second stream, then x += (shared + local) + remote.
#include "dev.h"
#include "gemv_core.h"
#include "internal.h"
#include "mm_core.h"

#include <cmath>

namespace lps {


constexpr int PF_TOK = 8;      // tokens per routing tile
constexpr int PF_MAXE = 64;    // experts the tile router is built for
constexpr int PF_RCPL = 10;    // router row chunks per lane (d <= 5120, the LDS bound below)
constexpr int PF_MAXK = 16;
// grouped GEMM tile: GM token rows x GBN weight rows; K a multiple of 2 GBK
constexpr int GM = 256, GBN = 256, GBK = 64;

struct PfP {
  const float* x;        // [T, d] residual
  const float* g;
  float eps;
  const uint16_t* wr;    // [E, d]
  const uint16_t* w_gu_e;
  const uint16_t* w_d_e;
  const uint16_t* w_gu_s;
  const uint16_t* w_d_s;
  int T, d, E, k, ff, remote_from;
  uint16_t* xb;          // [T, d] bf16 normed rows
  int32_t* idx;          // [T, k]
  float* w;              // [T, k]
  int32_t* cnt;          // [E + 1]
  int32_t* off;          // [E + 1]
  int32_t* lst;          // [E, T] tokens per expert
  int32_t* lslot;        // [E, T] slot of the expert in the token's top-k
  float* lw;             // [E, T] gate weight
  int32_t* tiles;        // [max_tiles] packed (expert << 20) | m0: this launch's list
  int32_t* n_tiles;      // [1]
  int32_t* tiles_r;      // the remote experts' list (built with the local one)
  int32_t* n_tiles_r;
  uint16_t* act;         // [T*k + T, ff] bf16 SwiGLU outputs, rows by (off[e] + i)
  float* z;              // [T, k, d] weighted expert outputs by slot
  float* shared;         // [T, d]
  float* local;          // [T, d]
  uint16_t* remote16;    // [T, d]
};

__device__ __forceinline__ uint16_t bf16_rne(float f) { return f32_to_bf16(f); }

// Token t's top k of its E router logits lgr (one wave, lane = expert id):
// softmax over all E, the k largest (ties to the lower id), weights renormalised.
__device__ __forceinline__ void pf_select(const PfP& p, const float* lgr, int t, int lane) {
  float v = lane < p.E ? lgr[lane] : -INFINITY;
  const float m = wave_max(v);
  const float z = wave_sum(lane < p.E ? exp_native(v - m) : 0.f);
  float ssum = 0.f;
  float pis = 0.f;   // this lane's selected pi, if selected
  int slot = -1;
  for (int j = 0; j < p.k; ++j) {
    const float mx = wave_max(v);
    const unsigned long long msk = __ballot(v == mx && lane < p.E);
    const int sel = msk ? __ffsll((long long)msk) - 1 : j;     // no finite logit: slot id
    const float pi = msk ? exp_native(mx - m) / z : __uint_as_float(0x7FC00000u);
    if (lane == sel) {
      v = -INFINITY;
      pis = pi;
      slot = j;
    }
    ssum += pi;
    if (lane == 0) p.idx[(long long)t * p.k + j] = sel;
  }
  if (slot >= 0) p.w[(long long)t * p.k + slot] = pis / ssum;
}

// ---- 1. route ------------------------------------------------------------------
// ROUTE = false: only the normed rows' bf16 copy (step 0); ROUTE = true: the router
// on the same f32 rows, recomputed by the same code (step 1)
template <bool ROUTE>
__global__ __launch_bounds__(256) void k_pf_route(PfP p) {
  extern __shared__ float hs[];            // [PF_TOK][d] normed rows (f32)
  __shared__ float lg[PF_TOK][PF_MAXE];
  const int t0 = blockIdx.x * PF_TOK;
  const int lane = threadIdx.x & 63, wv = threadIdx.x / 64;
  const int d = p.d;
  // each wave normalises two rows
  for (int q = 0; q < 2; ++q) {
    const int r = wv * 2 + q, t = t0 + r;
    float* h = hs + r * d;
    if (t < p.T) {
      const float* xr = p.x + (long long)t * d;
      float ss = 0.f;
      for (int c = lane * 4; c < d; c += 256) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(xr + c);
        *reinterpret_cast<f32x4*>(h + c) = v;
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      }
      ss = wave_sum(ss);
      const float rinv = 1.0f / sqrtf(ss / float(d) + p.eps);
      for (int c = lane * 4; c < d; c += 256) {
        f32x4 v = *reinterpret_cast<f32x4*>(h + c);
        const f32x4 gg = *reinterpret_cast<const f32x4*>(p.g + c);
        v.x = v.x * rinv * gg.x;
        v.y = v.y * rinv * gg.y;
        v.z = v.z * rinv * gg.z;
        v.w = v.w * rinv * gg.w;
        *reinterpret_cast<f32x4*>(h + c) = v;
        if constexpr (!ROUTE) {
          const uint32_t lo = uint32_t(bf16_rne(v.x)) | (uint32_t(bf16_rne(v.y)) << 16);
          const uint32_t hi = uint32_t(bf16_rne(v.z)) | (uint32_t(bf16_rne(v.w)) << 16);
          *reinterpret_cast<uint2*>(p.xb + (long long)t * d + c) = make_uint2(lo, hi);
        }
      }
    } else {
      for (int c = lane * 4; c < d; c += 256) *reinterpret_cast<f32x4*>(h + c) = f32x4{0, 0, 0, 0};
    }
  }
  if constexpr (!ROUTE) return;
  __syncthreads();
  // router logits: wave wv takes experts wv, wv + 4, ...; the lane / chunk split of
  // a row is the decode router's (chunk c of 8 values on lane c % 64, ascending).
  // All of an expert row's chunks are loaded at once, and the next expert's row is
  // in flight while the current one is multiplied (two register sets), so a wave
  // waits for about one L2 round trip instead of one per chunk.
  const int nck = d / 8;
  u32x4 va[PF_RCPL], vb[PF_RCPL];
#define PF_RLOAD(V, EX)                                                                   \
  _Pragma("unroll") for (int i = 0; i < PF_RCPL; ++i) {                                  \
    const int c = lane + 64 * i;                                                         \
    V[i] = ((EX) < p.E && c < nck) ? ld16(p.wr + (long long)(EX) * d + (long long)c * 8)   \
                                  : u32x4{0u, 0u, 0u, 0u};                               \
  }
#define PF_RDOT(V, EX)                                                                    \
  {                                                                                      \
    float a[PF_TOK];                                                                     \
    _Pragma("unroll") for (int r = 0; r < PF_TOK; ++r) a[r] = 0.f;                       \
    _Pragma("unroll") for (int i = 0; i < PF_RCPL; ++i) {                                \
      const int c = lane + 64 * i;                                                       \
      if (c < nck) {                                                                     \
        _Pragma("unroll") for (int r = 0; r < PF_TOK; ++r)                               \
          acc_chunk<LPS_BF16>(V[i], 0, hs + r * d + c * 8, a[r]);                        \
      }                                                                                  \
    }                                                                                    \
    _Pragma("unroll") for (int r = 0; r < PF_TOK; ++r) {                                 \
      const float s_ = wave_sum(a[r]);                                                   \
      if (lane == 0) lg[r][EX] = s_;                                                      \
    }                                                                                    \
  }
  PF_RLOAD(va, wv)
  for (int e = wv; e < p.E; e += 8) {
    PF_RLOAD(vb, e + 4)
    PF_RDOT(va, e)
    if (e + 4 >= p.E) break;
    PF_RLOAD(va, e + 8)
    PF_RDOT(vb, e + 4)
  }
#undef PF_RLOAD
#undef PF_RDOT
  __syncthreads();
  // top-k: wave wv selects for tokens 2wv, 2wv + 1; lane = expert id
  for (int q = 0; q < 2; ++q) {
    const int r = wv * 2 + q, t = t0 + r;
    if (t < p.T) pf_select(p, lg[r], t, lane);
  }
}


// The router on the matrix cores: 16 tokens per workgroup, their normed f32 rows
// held in registers (each wave four rows) and staged in LDS one half of the columns
// at a time (row pitch half + 4 floats, so the 16 rows of an operand read fall on
// distinct banks; 66 KiB at d = 2048, so two workgroups share a CU),
// logits[t, e] = sum_k h[t, k] Wr[e, k] on the matrix cores with the f32 rows split
// exactly into bf16 parts (the router reads the unrounded rows; bf16 weights widen
// exactly).  Wave wv takes experts 16 wv .. 16 wv + 15 (as 16 columns); lane
// (n, g) supplies token n's and expert 16 wv + n's values at k = 32 s + 8 g .. + 7
// for step s, the steps in ascending order across both halves.  The selection is
// the tile router's.  d % 32 == 0, E <= 64, d <= 256 PF_MROW; wider rows take the
// tile router.
constexpr int PF_MTOK = 16;
constexpr int PF_MUNR = 8;   // router k steps per lane and batch (two batches in flight)
constexpr int PF_MROW = 9;   // float4s per lane of a normed row (d <= 2304)

// floats of LDS the router stages per token row (the wider half plus the pad)
inline int pf_mx_pitch(int d) { const int ns = d / 32; return 32 * (ns - ns / 2) + 4; }

__global__ __launch_bounds__(256) void k_pf_route_mx(PfP p) {
  extern __shared__ float hs[];            // [PF_MTOK][pitch]: one half of the normed rows
  __shared__ float lg[PF_MTOK][PF_MAXE];
  const int t0 = blockIdx.x * PF_MTOK;
  const int lane = threadIdx.x & 63, wv = threadIdx.x / 64;
  const int d = p.d;
  const int ns = d / 32, hb = ns / 2;      // k steps; the first half's
  const int dp = 32 * (ns - hb) + 4;
  // each wave normalises four rows; the four rows' float4s all go out at once (rows
  // past T are zero)
  f32x4 vq[4][PF_MROW];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int t = t0 + wv * 4 + q;
#pragma unroll
    for (int i = 0; i < PF_MROW; ++i) {
      const int c = lane * 4 + 256 * i;
      vq[q][i] = (t < p.T && c < d) ? *reinterpret_cast<const f32x4*>(p.x + (long long)t * d + c)
                                    : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  // the sum of squares visits the row in the order the tile router does
  float rinv[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4* v = vq[q];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < PF_MROW; ++i) ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
    ss = wave_sum(ss);
    rinv[q] = 1.0f / sqrtf(ss / float(d) + p.eps);
  }
  // logits[t, e] = sum_k h[t, k] Wr[e, k] on v_mfma_f32_16x16x32_bf16: wave wv takes
  // experts 16 wv .. 16 wv + 15 as columns, the 16 tokens as rows; lane (n, g) supplies
  // token n's and expert 16 wv + n's values at k = 32 s + 8 g .. + 7 for step s.  The
  // f32 row values enter as three bf16 parts (hi = the top 8 significant bits, mid the
  // next 8, lo the rest: hi + mid + lo is the value exactly, each part's product with a
  // bf16 weight is exact in f32), so the sum is an f32 dot product in another order.
  const int n = lane & 15, g = lane >> 4;
  const int e = 16 * wv + n;
  const float* ha = hs + n * dp + 8 * g;    // A: token n
  // one descriptor for the whole router matrix (wave-uniform); expert rows past E
  // lie past its end and read as zeros
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.wr), (short)0, p.E * d * 2, 0x00020000);
  const int boff = (e * d + 8 * g) * 2;     // this lane's row and k offset, in bytes
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  u32x4 bq0[PF_MUNR], bq1[PF_MUNR];
#define PF_RLOAD_B(BQ, S0)                                                                     \
  _Pragma("unroll") for (int u = 0; u < PF_MUNR; ++u)                                          \
    BQ[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(                   \
                                          rs, boff + min((S0) + u, ns - 1) * 64, 0, 0));
#define PF_RMMA_B(BQ, S0)                                                                      \
  _Pragma("unroll") for (int u = 0; u < PF_MUNR; ++u) {                                        \
    const int st = (S0) + u;                                                                   \
    if (st < se) {                                                                             \
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(ha + 32 * (st - sb));                   \
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(ha + 32 * (st - sb) + 4);               \
      const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};                    \
      bf16x8 hi, mid, lo;                                                                      \
      _Pragma("unroll") for (int j = 0; j < 8; ++j) {                                          \
        const float xh = __uint_as_float(__float_as_uint(av[j]) & 0xFFFF0000u);                \
        const float r1 = av[j] - xh;                                                           \
        const float xm = __uint_as_float(__float_as_uint(r1) & 0xFFFF0000u);                   \
        const float r2 = r1 - xm;                                                              \
        hi[j] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(xh) >> 16));             \
        mid[j] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(xm) >> 16));            \
        lo[j] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(r2) >> 16));             \
      }                                                                                        \
      const bf16x8 b = __builtin_bit_cast(bf16x8, BQ[u]);                                      \
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, b, acc, 0, 0, 0);                      \
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mid, b, acc, 0, 0, 0);                     \
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, b, acc, 0, 0, 0);                      \
    }                                                                                          \
  }
  // the columns c_lo .. c_hi - 1 of the wave's four rows (v), scaled, into LDS
  auto stage = [&](const f32x4 (&v)[4][PF_MROW], int c_lo, int c_hi) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = wv * 4 + q, t = t0 + r;
      float* h = hs + r * dp - c_lo;
#pragma unroll
      for (int i = 0; i < PF_MROW; ++i) {
        const int c = lane * 4 + 256 * i;
        if (c >= c_lo && c < c_hi) {
          f32x4 y = v[q][i];
          if (t < p.T) {
            const f32x4 gg = *reinterpret_cast<const f32x4*>(p.g + c);
            y.x = y.x * rinv[q] * gg.x;
            y.y = y.y * rinv[q] * gg.y;
            y.z = y.z * rinv[q] * gg.z;
            y.w = y.w * rinv[q] * gg.w;
          }
          *reinterpret_cast<f32x4*>(h + c) = y;
        }
      }
    }
  };
  // the k steps sb .. se - 1 over the staged columns; the router rows stream from L2
  // in batches of PF_MUNR steps, double-buffered
  auto mma = [&](int sb, int se) {
    PF_RLOAD_B(bq0, sb)
    for (int s0 = sb; s0 < se; s0 += 2 * PF_MUNR) {
      PF_RLOAD_B(bq1, s0 + PF_MUNR)
      PF_RMMA_B(bq0, s0)
      PF_RLOAD_B(bq0, s0 + 2 * PF_MUNR)
      PF_RMMA_B(bq1, s0 + PF_MUNR)
    }
  };
  stage(vq, 0, 32 * hb);
  __syncthreads();
  mma(0, hb);
  __syncthreads();   // every wave is done with the first half's rows
  {
    // the second half's columns again (from L2), so the rows need not stay in
    // registers through the first half's products
    f32x4 v2[4][PF_MROW];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int t = t0 + wv * 4 + q;
#pragma unroll
      for (int i = 0; i < PF_MROW; ++i) {
        const int c = lane * 4 + 256 * i;
        v2[q][i] = (t < p.T && c >= 32 * hb && c < d)
                       ? *reinterpret_cast<const f32x4*>(p.x + (long long)t * d + c)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    stage(v2, 32 * hb, d);
  }
  __syncthreads();
  mma(hb, ns);
#undef PF_RLOAD_B
#undef PF_RMMA_B
  // acc[i] = logits[token 4 g + i][expert 16 wv + n]
  if (e < p.E) {
#pragma unroll
    for (int i = 0; i < 4; ++i) lg[4 * g + i][e] = acc[i];
  }
  __syncthreads();
  for (int q = 0; q < 4; ++q) {            // wave wv selects for its four tokens
    const int r = wv * 4 + q, t = t0 + r;
    if (t < p.T) pf_select(p, lg[r], t, lane);
  }
}

// Step 0 for rows up to 256 PF_MROW wide: one wave per row, the row's float4s all in
// flight, then the tile router's norm (same per-lane order and arithmetic, so the
// same bits) rounded to the bf16 rows.  No LDS.
__global__ __launch_bounds__(256) void k_pf_norm_rows(PfP p) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + threadIdx.x / 64;
  if (t >= p.T) return;
  const int d = p.d;
  f32x4 v[PF_MROW];
#pragma unroll
  for (int i = 0; i < PF_MROW; ++i) {
    const int c = lane * 4 + 256 * i;
    v[i] = c < d ? *reinterpret_cast<const f32x4*>(p.x + (long long)t * d + c) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < PF_MROW; ++i) ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
  ss = wave_sum(ss);
  const float rinv = 1.0f / sqrtf(ss / float(d) + p.eps);
#pragma unroll
  for (int i = 0; i < PF_MROW; ++i) {
    const int c = lane * 4 + 256 * i;
    if (c < d) {
      const f32x4 gg = *reinterpret_cast<const f32x4*>(p.g + c);
      const float y0 = v[i].x * rinv * gg.x, y1 = v[i].y * rinv * gg.y;
      const float y2 = v[i].z * rinv * gg.z, y3 = v[i].w * rinv * gg.w;
      const uint32_t lo = uint32_t(bf16_rne(y0)) | (uint32_t(bf16_rne(y1)) << 16);
      const uint32_t hi = uint32_t(bf16_rne(y2)) | (uint32_t(bf16_rne(y3)) << 16);
      *reinterpret_cast<uint2*>(p.xb + (long long)t * d + c) = make_uint2(lo, hi);
    }
  }
}

// ---- 2. group: stable per-expert token lists ------------------------------------------
// Each thread takes one token of every 256: its KW 16-byte words of indices and of
// weights for B such steps are loaded at once (one round trip per 256 B tokens), then
// the B steps take their ballots and prefix sums from registers.  The per-step totals
// alternate between two LDS rows, so one barrier per step keeps them apart.
template <int KW, int B>
__global__ __launch_bounds__(256) void k_pf_group(PfP p) {
  const int e = blockIdx.x;
  const int lane = threadIdx.x & 63, wv = threadIdx.x / 64;
  __shared__ int wtot[2][4];
  const int bytes = p.T * p.k * 4;
  const __amdgpu_buffer_rsrc_t ri = __builtin_amdgcn_make_buffer_rsrc(p.idx, (short)0, bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(p.w, (short)0, bytes, 0x00020000);
  int base = 0;
  for (int t0 = 0; t0 < p.T; t0 += 256 * B) {
    u32x4 vi[B][KW], vw[B][KW];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int off = (t0 + 256 * b + threadIdx.x) * p.k * 4;   // past T: zeros, masked below
#pragma unroll
      for (int q = 0; q < KW; ++q) {
        vi[b][q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ri, off + 16 * q, 0, 0));
        vw[b][q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, off + 16 * q, 0, 0));
      }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int t = t0 + 256 * b + threadIdx.x;
      int slot = -1;
      uint32_t wbits = 0;
      if (t < p.T) {
#pragma unroll
        for (int j = 0; j < 4 * KW; ++j) {
          const uint32_t id = vi[b][j / 4][j % 4];
          if (j < p.k && slot < 0 && int(id) == e) {
            slot = j;
            wbits = vw[b][j / 4][j % 4];
          }
        }
      }
      const unsigned long long msk = __ballot(slot >= 0);
      const int before = __popcll(msk & ((1ull << lane) - 1ull));
      if (lane == 0) wtot[b & 1][wv] = __popcll(msk);
      __syncthreads();
      int wbase = 0;
      for (int i = 0; i < wv; ++i) wbase += wtot[b & 1][i];
      if (slot >= 0) {
        const long long pos = (long long)e * p.T + base + wbase + before;
        p.lst[pos] = t;
        p.lslot[pos] = slot;
        p.lw[pos] = __uint_as_float(wbits);
      }
      base += wtot[b & 1][0] + wtot[b & 1][1] + wtot[b & 1][2] + wtot[b & 1][3];
    }
  }
  if (threadIdx.x == 0) p.cnt[e] = base;
}

// ---- 3. tiles ----------------------------------------------------------------------
// One wave: lane e < E takes routed expert e.  Exclusive prefix sums over the lanes
// give each expert's first row in the grouped buffers (off) and its first entry in
// the local or the remote tile list; the shared expert (every token) follows the
// routed ones, its tiles last in the local list.  Lists hold (expert << 20) | m0.
// exclusive prefix sum of v over the wave's lanes; *tot = the sum over all lanes
__device__ __forceinline__ int wave_excl_scan(int v, int lane, int* tot) {
  int x = v;
#pragma unroll
  for (int o = 1; o < WAVE; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  *tot = __shfl(x, WAVE - 1);
  return x - v;
}
__global__ __launch_bounds__(WAVE) void k_pf_tiles(PfP p) {
  const int e = threadIdx.x;
  const int c = e < p.E ? p.cnt[e] : 0;
  const int nt = (c + GM - 1) / GM;
  const bool remote = e >= p.remote_from && e < p.E;
  int tot, nl, nr;
  const int off = wave_excl_scan(c, e, &tot);
  const int sl = wave_excl_scan(remote ? 0 : nt, e, &nl);
  const int sr = wave_excl_scan(remote ? nt : 0, e, &nr);
  if (e < p.E) {
    p.off[e] = off;
    int32_t* lst = remote ? p.tiles_r + sr : p.tiles + sl;
    for (int i = 0; i < nt; ++i) lst[i] = (e << 20) | (i * GM);
  }
  const int ns = (p.T + GM - 1) / GM;
  for (int i = e; i < ns; i += WAVE) p.tiles[nl + i] = (p.E << 20) | (i * GM);
  if (e == 0) {
    p.off[p.E] = tot;
    p.cnt[p.E] = p.T;
    *p.n_tiles = nl + ns;
    *p.n_tiles_r = nr;
  }
}

// ---- 4/5. grouped GEMM on MFMA -----------------------------------------------------------
// C[m, n] = sum_k A[m, k] B[n, k]: A rows are gathered activation rows (bf16), B
// rows weight rows (bf16, K contiguous).  A 256 x 256 tile per workgroup, the main
// loop of mm_core.h (four waves of 128 x 128, LDS DMA staging); this kernel maps the
// tile's rows (the expert's token list, its rows of the SwiGLU buffer, its weight
// rows) and applies the epilogue.
static_assert(GM == MM_TILE && GBN == MM_TILE, "the grouped GEMM tile is the core's");

template <bool FIRST>
__global__ __launch_bounds__(MM_THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_pf_gemm(PfP p) {
  const int tile = blockIdx.y;
  if (tile >= *p.n_tiles) return;
  const int packed = p.tiles[tile];
  const int e = packed >> 20, m0 = packed & 0xFFFFF;
  const bool shared_e = e == p.E;
  const int cnt = p.cnt[e];
  const int K = FIRST ? p.d : p.ff;
  const int n0 = FIRST ? blockIdx.x * (GBN / 2) : blockIdx.x * GBN;
  extern __shared__ __attribute__((aligned(16))) uint16_t gsm[];
  char* lds = reinterpret_cast<char*>(gsm);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid / 64);
  const int wm = wv >> 1, wn = wv & 1;
  const uint16_t* abase = FIRST ? p.xb : p.act;
  const uint16_t* bbase = FIRST ? (shared_e ? p.w_gu_s : p.w_gu_e + (long long)e * 2 * p.ff * p.d)
                                : (shared_e ? p.w_d_s : p.w_d_e + (long long)e * p.d * p.ff);
  const long long abytes = FIRST ? (long long)p.T * p.d * 2 : ((long long)p.T * p.k + p.T) * p.ff * 2;
  const long long bbytes = FIRST ? 2LL * p.ff * p.d * 2 : (long long)p.d * p.ff * 2;
  const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(abase), (short)0, (int)(abytes < 0x7FFFFFFF ? abytes : 0x7FFFFFFF), 0x00020000);
  const __amdgpu_buffer_rsrc_t bres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(bbase), (short)0, (int)(bbytes < 0x7FFFFFFF ? bbytes : 0x7FFFFFFF), 0x00020000);
  // GEMM2: this thread's tile row's output offset and gate weight, loaded first
  // (the first operand wait covers them), put in LDS for the epilogue
  long long eo = 0;
  float ewt = 0.f;
  if (!FIRST) {
    const int m = m0 + tid;
    if (m < cnt) {
      if (shared_e) {
        eo = (long long)m * p.d;
        ewt = 1.f;
      } else {
        const long long li = (long long)e * p.T + m;
        eo = ((long long)p.lst[li] * p.k + p.lslot[li]) * p.d;
        ewt = p.lw[li];
      }
    }
  }
  int aoff[MM_NI], boff[MM_NI];
#pragma unroll
  for (int j = 0; j < MM_NI; ++j) {
    const int sr = mm_stage_row(wv, lane, j);
    const int gch = mm_stage_chunk(sr, lane);
    const int r = m0 + sr;
    const int rr = r < cnt ? r : m0;          // rows past the list repeat a valid row
    if (FIRST) {
      const int tok = shared_e ? rr : p.lst[(long long)e * p.T + rr];
      aoff[j] = (tok * p.d + 8 * gch) * 2;
    } else {
      aoff[j] = ((p.off[e] + rr) * p.ff + 8 * gch) * 2;
    }
    int wrow;
    if (FIRST) {
      // staged B rows of wave column wc = sr / 128: blocks of 32 gate rows and 32 up
      // rows of the same outputs, alternating, so gate and up of an output share lanes
      const int wc = sr >> 7, jb = (sr >> 5) & 3, cc = sr & 31;
      wrow = ((jb & 1) ? p.ff : 0) + n0 + 64 * wc + 32 * (jb >> 1) + cc;
    } else {
      wrow = n0 + sr;
    }
    boff[j] = (wrow * K + 8 * gch) * 2;
  }

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  // A rows (reused by the other column tiles) cached, weight rows streamed
  mm_tile<0, 2>(ares, bres, aoff, boff, K / MM_BK, lds, acc);

  // epilogue: acc[i][j][r] is C[128 wm + 32 i + 8 (r / 4) + 4 (lane / 32) + r % 4][128 wn + 32 j + lane % 32]
  if constexpr (FIRST) {
    // blocks j = 0, 2 hold gate and 1, 3 up of outputs 64 wn + 32 (j / 2) + lane % 32;
    // the SwiGLU tile [GM][GBN / 2] (bf16) is assembled in LDS, then leaves as whole
    // 16-byte pieces of its rows
    constexpr int OP = GBN / 2 + 8;           // row pitch (bf16): rows 4 apart on other banks
    uint16_t* ot = gsm;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 128 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          ot[row * OP + 64 * wn + 32 * h + (lane & 31)] =
              bf16_rne(silu_fast(acc[i][2 * h][r]) * acc[i][2 * h + 1][r]);
        }
      }
    }
    __syncthreads();
    const long long obase = (long long)(p.off[e] + m0) * p.ff + n0;
    constexpr int CPR = GBN / 2 / 8;          // 16-byte pieces per row
#pragma unroll
    for (int q = 0; q < GM * CPR / MM_THREADS; ++q) {
      const int c = tid + q * MM_THREADS;
      const int row = c / CPR, c8 = (c % CPR) * 8;
      if (m0 + row < cnt)
        *reinterpret_cast<u32x4*>(p.act + obase + (long long)row * p.ff + c8) =
            *reinterpret_cast<const u32x4*>(ot + row * OP + c8);
    }
  } else {
    long long* eoff = reinterpret_cast<long long*>(lds);
    float* ew = reinterpret_cast<float*>(eoff + GM);
    eoff[tid] = eo;
    ew[tid] = ewt;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 128 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m0 + row < cnt) {
          const float wgt = ew[row];
          float* dst = (shared_e ? p.shared : p.z) + eoff[row];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int col = n0 + 128 * wn + 32 * j + (lane & 31);
            __builtin_nontemporal_store(shared_e ? acc[i][j][r] : wgt * acc[i][j][r], dst + col);
          }
        }
        __builtin_amdgcn_sched_barrier(0);   // one row at a time: keeps the epilogue's live range short
      }
    }
  }
}

// ---- 6. per-token halves in ascending expert id -------------------------------------------
__global__ __launch_bounds__(256) void k_pf_halves(PfP p) {
  const int t = blockIdx.x;
  __shared__ int ids[PF_MAXK];
  __shared__ int order[PF_MAXK];
  if (threadIdx.x < p.k) ids[threadIdx.x] = p.idx[(long long)t * p.k + threadIdx.x];
  __syncthreads();
  if (threadIdx.x < p.k) {
    int rank = 0;
    for (int j = 0; j < p.k; ++j)
      rank += ids[j] < ids[threadIdx.x] || (ids[j] == ids[threadIdx.x] && j < int(threadIdx.x));
    order[rank] = threadIdx.x;
  }
  __syncthreads();
  for (int c = threadIdx.x * 4; c < p.d; c += 256 * 4) {
    f32x4 lo = {0, 0, 0, 0}, re = {0, 0, 0, 0};
    for (int n = 0; n < p.k; ++n) {
      const int j = order[n];
      // read once: nontemporal, so the stream does not evict what the combine reads next
      const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p.z + ((long long)t * p.k + j) * p.d + c));
      if (ids[j] < p.remote_from) {
        lo.x += v.x; lo.y += v.y; lo.z += v.z; lo.w += v.w;
      } else {
        re.x += v.x; re.y += v.y; re.z += v.z; re.w += v.w;
      }
    }
    *reinterpret_cast<f32x4*>(p.local + (long long)t * p.d + c) = lo;
    const _Float16 h0 = static_cast<_Float16>(re.x), h1 = static_cast<_Float16>(re.y);
    const _Float16 h2 = static_cast<_Float16>(re.z), h3 = static_cast<_Float16>(re.w);
    const uint32_t a = uint32_t(__builtin_bit_cast(uint16_t, h0)) | (uint32_t(__builtin_bit_cast(uint16_t, h1)) << 16);
    const uint32_t b = uint32_t(__builtin_bit_cast(uint16_t, h2)) | (uint32_t(__builtin_bit_cast(uint16_t, h3)) << 16);
    *reinterpret_cast<uint2*>(p.remote16 + (long long)t * p.d + c) = make_uint2(a, b);
  }
}

// ---- scratch -----------------------------------------------------------------------------
struct PfScratch {
  size_t xb, xr, idx, w, cnt, off, lst, lslot, lw, tiles, ntiles, tiles_r, ntiles_r, act, z,
      shared, local, remote16, bo, total;
  int max_tiles;
};
static PfScratch pf_scratch(const lps_moe_desc* m, int T) {
  PfScratch s{};
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o += align256(bytes); return r; };
  const size_t Tk = size_t(T) * m->top_k;
  s.max_tiles = int((Tk + GM - 1) / GM + m->n_experts + (size_t(T) + GM - 1) / GM + 1);
  s.xb = take(size_t(T) * m->d * 2);
  s.xr = take(size_t(T) * m->d * 2);          // the remote half's copy of the bf16 rows
  s.idx = take(Tk * 4);
  s.w = take(Tk * 4);
  s.cnt = take(size_t(m->n_experts + 1) * 4);
  s.off = take(size_t(m->n_experts + 1) * 4);
  s.lst = take(size_t(m->n_experts) * T * 4);
  s.lslot = take(size_t(m->n_experts) * T * 4);
  s.lw = take(size_t(m->n_experts) * T * 4);
  s.tiles = take(size_t(s.max_tiles) * 4);
  s.ntiles = take(4);
  s.tiles_r = take(size_t(s.max_tiles) * 4);
  s.ntiles_r = take(4);
  s.act = take((Tk + T) * m->ff * 2);
  s.z = take(Tk * m->d * 4);
  s.shared = take(size_t(T) * m->d * 4);
  s.local = take(size_t(T) * m->d * 4);
  s.remote16 = take(size_t(T) * m->d * 2);
  s.bo = take(size_t(T) * m->d * 4);
  s.total = o;
  return s;
}

}  // namespace lps

using namespace lps;

extern "C" size_t lps_moe_prefill_scratch_bytes(const lps_moe_desc* m, int32_t T) {
  if (!m || T <= 0) return 0;
  return pf_scratch(m, T).total;
}

extern "C" int lps_moe_prefill(const lps_moe_desc* m, float* x, int32_t T, int32_t n_pieces,
                               void* scratch, size_t scratch_bytes, void* s_main, void* s_remote) {
  LPS_REQUIRE(m, LPS_EINVAL, "lps_moe_prefill: null MoE descriptor");
  LPS_REQUIRE(T >= 1 && T <= (1 << 20) - 1, LPS_EINVAL, "lps_moe_prefill: T %d outside [1, 2^20)", T);
  LPS_REQUIRE(m->n_experts >= 1 && m->n_experts <= PF_MAXE, LPS_EUNSUP,
              "lps_moe_prefill: n_experts %d outside [1, %d]", m->n_experts, PF_MAXE);
  LPS_REQUIRE(m->top_k >= 1 && m->top_k <= PF_MAXK && m->top_k <= m->n_experts, LPS_EUNSUP,
              "lps_moe_prefill: top_k %d", m->top_k);
  LPS_REQUIRE(m->d % GBN == 0 && m->ff % (GBN / 2) == 0 && m->d % (2 * GBK) == 0 &&
                  m->ff % (2 * GBK) == 0, LPS_EUNSUP,
              "lps_moe_prefill: d %d must be a multiple of %d and ff %d of %d", m->d, GBN, m->ff,
              GBN / 2);
  LPS_REQUIRE(size_t(PF_TOK) * m->d * 4 <= 160 * 1024, LPS_EUNSUP, "lps_moe_prefill: d %d too wide", m->d);
  LPS_REQUIRE(m->remote_from >= 0 && m->remote_from <= m->n_experts, LPS_EINVAL,
              "lps_moe_prefill: remote_from %d", m->remote_from);
  LPS_REQUIRE(m->g_ffn && m->w_r && m->w_gu_e && m->w_d_e && m->w_gu_s && m->w_d_s && x && scratch,
              LPS_EINVAL, "lps_moe_prefill: null pointer");
  {
    // every kernel addresses its operands with 32-bit byte offsets (buffer
    // resources, int row offsets): each operand stays below 2 GiB, else the chunk
    // is refused before anything is enqueued (e.g. T >= 32768 at d 2048, top 8:
    // the per-slot expert outputs [T, k, d] f32)
    const long long Tk = (long long)T * m->top_k;
    const long long big = std::max({(long long)T * m->d * 4, Tk * m->d * 4, (Tk + T) * m->ff * 2,
                                    4LL * m->ff * m->d, (long long)m->n_experts * T * 4});
    LPS_REQUIRE(big < (1LL << 31), LPS_EUNSUP,
                "lps_moe_prefill: a %lld-byte operand at T %d (the kernels address below 2 GiB "
                "with 32-bit offsets; split the chunk)", big, T);
  }
  const PfScratch s = pf_scratch(m, T);
  LPS_REQUIRE(scratch_bytes >= s.total, LPS_EINVAL, "lps_moe_prefill: scratch %zu < %zu",
              scratch_bytes, s.total);
  char* sc = static_cast<char*>(scratch);
  PfP p{};
  p.x = x;
  p.g = m->g_ffn;
  p.eps = m->eps;
  p.wr = static_cast<const uint16_t*>(m->w_r);
  p.w_gu_e = static_cast<const uint16_t*>(m->w_gu_e);
  p.w_d_e = static_cast<const uint16_t*>(m->w_d_e);
  p.w_gu_s = static_cast<const uint16_t*>(m->w_gu_s);
  p.w_d_s = static_cast<const uint16_t*>(m->w_d_s);
  p.T = T;
  p.d = m->d;
  p.E = m->n_experts;
  p.k = m->top_k;
  p.ff = m->ff;
  p.remote_from = m->remote_from;
  p.xb = reinterpret_cast<uint16_t*>(sc + s.xb);
  p.idx = reinterpret_cast<int32_t*>(sc + s.idx);
  p.w = reinterpret_cast<float*>(sc + s.w);
  p.cnt = reinterpret_cast<int32_t*>(sc + s.cnt);
  p.off = reinterpret_cast<int32_t*>(sc + s.off);
  p.lst = reinterpret_cast<int32_t*>(sc + s.lst);
  p.lslot = reinterpret_cast<int32_t*>(sc + s.lslot);
  p.lw = reinterpret_cast<float*>(sc + s.lw);
  p.tiles = reinterpret_cast<int32_t*>(sc + s.tiles);
  p.n_tiles = reinterpret_cast<int32_t*>(sc + s.ntiles);
  p.tiles_r = reinterpret_cast<int32_t*>(sc + s.tiles_r);
  p.n_tiles_r = reinterpret_cast<int32_t*>(sc + s.ntiles_r);
  p.act = reinterpret_cast<uint16_t*>(sc + s.act);
  p.z = reinterpret_cast<float*>(sc + s.z);
  p.shared = reinterpret_cast<float*>(sc + s.shared);
  p.local = reinterpret_cast<float*>(sc + s.local);
  p.remote16 = reinterpret_cast<uint16_t*>(sc + s.remote16);
  float* bo = reinterpret_cast<float*>(sc + s.bo);
  LPS_REQUIRE(n_pieces >= 1 && n_pieces <= 64, LPS_EINVAL,
              "lps_moe_prefill: n_pieces %d outside [1, 64]", n_pieces);
  hipStream_t st = as_stream(s_main), sr = as_stream(s_remote);
  uint16_t* xr = reinterpret_cast<uint16_t*>(sc + s.xr);
  const size_t rlds = size_t(PF_TOK) * m->d * 4;
  // the matrix-core router where its rows fit its registers (d <= 2304), else the tile router
  const size_t mlds = size_t(PF_MTOK) * pf_mx_pitch(m->d) * 4;
  const bool route_mx = m->d % 32 == 0 && m->d <= 256 * PF_MROW;
  int rc = ensure_lds((const void*)k_pf_route<false>, rlds);
  if (!rc) rc = route_mx ? ensure_lds((const void*)k_pf_route_mx, mlds)
                         : ensure_lds((const void*)k_pf_route<true>, rlds);
  if (rc) return rc;
  const size_t glds = MM_LDS, glds2 = MM_LDS;
  rc = ensure_lds((const void*)k_pf_gemm<true>, glds);
  if (!rc) rc = ensure_lds((const void*)k_pf_gemm<false>, glds2);
  if (rc) return rc;
  hipEvent_t ev[3];   // rows normed (main), tile lists built (main), remote experts done
  for (int i = 0; i < 3; ++i) {
    if (hipEventCreateWithFlags(&ev[i], hipEventDisableTiming | hipEventDisableSystemFence) != hipSuccess) {
      for (int j = 0; j < i; ++j) (void)hipEventDestroy(ev[j]);
      return fail(LPS_EHIP, "lps_moe_prefill: hipEventCreate failed");
    }
  }
  if (m->d <= 256 * PF_MROW) {
    hipLaunchKernelGGL(k_pf_norm_rows, dim3((T + 3) / 4), dim3(256), 0, st, p);
  } else {
    hipLaunchKernelGGL(k_pf_route<false>, dim3((T + PF_TOK - 1) / PF_TOK), dim3(256), rlds, st, p);
  }
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = hipEventRecord(ev[0], st);
  // activation half: the remote copy of the bf16 rows, in P row pieces, on the
  // second stream while the main stream routes and groups
  if (e == hipSuccess) e = hipStreamWaitEvent(sr, ev[0], 0);
  int pieces = 0;
  for (int pc = 0; e == hipSuccess && pc < n_pieces; ++pc) {
    const long long lo = (long long)pc * T / n_pieces, hi = (long long)(pc + 1) * T / n_pieces;
    if (hi == lo) continue;
    // bf16 rows as 32-bit words (d is even): lo * d / 2 .. hi * d / 2
    rc = launch_copy_f32(reinterpret_cast<const float*>(p.xb) + lo * m->d / 2,
                         reinterpret_cast<float*>(xr) + lo * m->d / 2, (hi - lo) * m->d / 2, sr);
    if (rc) break;
    ++pieces;
  }
  if (e == hipSuccess && !rc) {
    if (route_mx)
      hipLaunchKernelGGL(k_pf_route_mx, dim3((T + PF_MTOK - 1) / PF_MTOK), dim3(256), mlds, st, p);
    else
      hipLaunchKernelGGL(k_pf_route<true>, dim3((T + PF_TOK - 1) / PF_TOK), dim3(256), rlds, st, p);
    if (m->top_k <= 8) hipLaunchKernelGGL((k_pf_group<2, 4>), dim3(m->n_experts), dim3(256), 0, st, p);
    else hipLaunchKernelGGL((k_pf_group<4, 2>), dim3(m->n_experts), dim3(256), 0, st, p);
    hipLaunchKernelGGL(k_pf_tiles, dim3(1), dim3(64), 0, st, p);
    e = hipGetLastError();
  }
  if (e == hipSuccess && !rc) e = hipEventRecord(ev[1], st);
  // remote experts: their tile list, rows from the remote copy, on the second stream
  if (e == hipSuccess && !rc) e = hipStreamWaitEvent(sr, ev[1], 0);
  if (e == hipSuccess && !rc) {
    PfP pr = p;
    pr.xb = xr;
    pr.tiles = p.tiles_r;
    pr.n_tiles = p.n_tiles_r;
    Stamp t1 = timer_take(LPS_KIND_MOE_GEMM1), t2 = timer_take(LPS_KIND_MOE_GEMM2);
    LPS_LAUNCH(k_pf_gemm<true>, dim3(m->ff / (GBN / 2), s.max_tiles), dim3(MM_THREADS), glds, sr,
               t1.start, t1.stop, pr);
    LPS_LAUNCH(k_pf_gemm<false>, dim3(m->d / GBN, s.max_tiles), dim3(MM_THREADS), glds2, sr,
               t2.start, t2.stop, pr);
    e = hipGetLastError();
  }
  if (e == hipSuccess && !rc) e = hipEventRecord(ev[2], sr);
  // local experts and the shared one on the main stream
  if (e == hipSuccess && !rc) {
    Stamp t1 = timer_take(LPS_KIND_MOE_GEMM1), t2 = timer_take(LPS_KIND_MOE_GEMM2);
    LPS_LAUNCH(k_pf_gemm<true>, dim3(m->ff / (GBN / 2), s.max_tiles), dim3(MM_THREADS), glds, st,
               t1.start, t1.stop, p);
    LPS_LAUNCH(k_pf_gemm<false>, dim3(m->d / GBN, s.max_tiles), dim3(MM_THREADS), glds2, st,
               t2.start, t2.stop, p);
    e = hipGetLastError();
  }
  if (e == hipSuccess && !rc) e = hipStreamWaitEvent(st, ev[2], 0);
  if (e == hipSuccess && !rc) {
    hipLaunchKernelGGL(k_pf_halves, dim3(T), dim3(256), 0, st, p);
    e = hipGetLastError();
  }
  for (int i = 0; i < 3; ++i) (void)hipEventDestroy(ev[i]);   // released once fired
  if (rc) return rc;
  if (e != hipSuccess) return fail(LPS_EHIP, "lps_moe_prefill: %s", hipGetErrorString(e));
  count_act_pieces(pieces);
  return lps_moe_combine(x, x, p.shared, p.local, p.remote16, bo, T, m->d, n_pieces, s_remote, s_main);
}
