// Chunked dense prefill through a stage's layers on gfx950.
//
// memra pp module docs (functions on the prime split) and ninfer pipeline
// stages (What is not covered yet): a prompt chunk runs through the stages in
// turn, each stage walking its own layers over all T rows of the chunk.  Per
// layer, each step its own launch, in stream order:
//  1. rows: RMSNorm of every row, rounded to bf16 (the matrix-core operand);
//  2. QKV GEMM [T, d] x [d, (nq + 2 nkv) hd] -> f32;
//  3. RoPE of the q and k heads at positions p0 + t (cos / sin from the layer's
//     table) and the chunk's K and V rows appended to the caches;
//  4. causal attention of every row over cache rows 0 .. p0 + t on the matrix
//     cores, the output rounded to bf16;
//  5. O GEMM, residual add into x;
//  6. rows: RMSNorm again, bf16;
//  7. gate/up GEMM with SwiGLU in registers, rounded to bf16;
//  8. down GEMM, residual add into x.
// bf16 weights and bf16 caches (16-row tiles) only: the shapes of the dense
// model whose prompts run through the stages.
#include "dev.h"
#include "internal.h"
#include "mm_core.h"

#include <cmath>
#include <type_traits>

namespace lps {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// ---- 1/6. per-row RMSNorm -> bf16 -------------------------------------------------------
__global__ __launch_bounds__(256) void k_pf_rows_norm(const float* x, const float* g, float eps,
                                                      int d, uint16_t* xb) {
  constexpr int NPT = 16;                    // rows up to 4096 wide stay in registers
  const long long t = blockIdx.x;
  const float* xr = x + t * d;
  __shared__ float red[4];
  float ss = 0.f;
  if (d <= NPT * 256) {
    // every element of the thread's share in flight at once; the same elements and
    // summation order as the loop below (zeros past d add nothing)
    float v[NPT];
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      const int i = threadIdx.x + 256 * k;
      v[k] = i < d ? xr[i] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < NPT; ++k) ss += v[k] * v[k];
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x / 64] = ss;
    __syncthreads();
    const float r = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / float(d) + eps);
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      const int i = threadIdx.x + 256 * k;
      if (i < d) xb[t * d + i] = f32_to_bf16(v[k] * r * g[i]);
    }
    return;
  }
  for (int i = threadIdx.x; i < d; i += 256) ss += xr[i] * xr[i];
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x / 64] = ss;
  __syncthreads();
  const float r = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / float(d) + eps);
  for (int i = threadIdx.x; i < d; i += 256) xb[t * d + i] = f32_to_bf16(xr[i] * r * g[i]);
}

// ---- 2/5/7/8. dense GEMM on the matrix cores -----------------------------------------------
// C[m, n] = sum_k A[m, k] B[n, k]; A [T, K] bf16 rows, B [N, K] bf16 weight rows.  A
// 256 x 256 tile per workgroup, the main loop of mm_core.h (four waves of 128 x 128,
// LDS DMA staging, K % 128 == 0).  Rows past T repeat row T - 1 (valid memory, never
// stored).  Epilogues:
//   GE_STORE   out[m, n] = C            (f32)
//   GE_ADD     out[m, n] += C           (f32, the residual)
//   GE_SWIGLU  out[m, j] = bf16(silu(C[m, j]) * C[m, ff + j]): a workgroup takes
//              128 outputs; per wave column its staged B rows alternate blocks of 32
//              gate rows and the 32 matching up rows, so both land in the same lanes.
enum { GE_STORE = 0, GE_ADD = 1, GE_SWIGLU = 2 };
constexpr int DM = MM_TILE, DN = MM_TILE;

struct DgP {
  const uint16_t* a;
  const uint16_t* b;
  void* out;
  int T, N, K;    // N: output columns (GE_SWIGLU: ff)
};

template <int EPI>
__global__ __launch_bounds__(MM_THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_dense_gemm(DgP p) {
  const int m0 = blockIdx.y * DM;
  const int n0 = EPI == GE_SWIGLU ? blockIdx.x * (DN / 2) : blockIdx.x * DN;
  const int K = p.K;
  extern __shared__ __attribute__((aligned(16))) uint16_t dsm[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid / 64);
  const int wm = wv >> 1, wn = wv & 1;
  const long long abytes = (long long)p.T * K * 2;
  const long long bbytes = (long long)(EPI == GE_SWIGLU ? 2 * p.N : p.N) * K * 2;
  const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.a), (short)0, (int)abytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t bres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.b), (short)0, (int)bbytes, 0x00020000);
  int aoff[MM_NI], boff[MM_NI];
#pragma unroll
  for (int j = 0; j < MM_NI; ++j) {
    const int sr = mm_stage_row(wv, lane, j);
    const int gch = mm_stage_chunk(sr, lane);
    const int r = min(m0 + sr, p.T - 1);
    aoff[j] = (r * K + 8 * gch) * 2;
    int wrow;
    if constexpr (EPI == GE_SWIGLU) {
      const int wc = sr >> 7, jb = (sr >> 5) & 3, cc = sr & 31;
      wrow = ((jb & 1) ? p.N : 0) + n0 + 64 * wc + 32 * (jb >> 1) + cc;
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
  // chunk rows (reused by the other column tiles) cached, weight rows streamed
  mm_tile<0, 2>(ares, bres, aoff, boff, K / MM_BK, reinterpret_cast<char*>(dsm), acc);

  // acc[i][j][r] is C[128 wm + 32 i + 8 (r / 4) + 4 (lane / 32) + r % 4][128 wn + 32 j + lane % 32]
  if constexpr (EPI == GE_SWIGLU) {
    // blocks j = 0, 2 hold gate and 1, 3 up of outputs 64 wn + 32 (j / 2) + lane % 32;
    // the bf16 tile [DM][DN / 2] is assembled in LDS (free once the main loop
    // returns) and leaves as whole 16-byte pieces of its rows (2-byte stores from
    // the accumulator layout covered half a cache line per half-wave)
    constexpr int OP = DN / 2 + 8;            // row pitch (bf16): rows 4 apart on other banks
    uint16_t* ot = dsm;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 128 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          ot[row * OP + 64 * wn + 32 * h + (lane & 31)] =
              f32_to_bf16(silu_fast(acc[i][2 * h][r]) * acc[i][2 * h + 1][r]);
        }
      }
    }
    __syncthreads();
    constexpr int CPR = DN / 2 / 8;           // 16-byte pieces per row
#pragma unroll
    for (int q = 0; q < DM * CPR / MM_THREADS; ++q) {
      const int c = tid + q * MM_THREADS;
      const int row = c / CPR, c8 = (c % CPR) * 8;
      if (m0 + row < p.T)
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.out) + (long long)(m0 + row) * p.N + n0 + c8) =
            *reinterpret_cast<const u32x4*>(ot + row * OP + c8);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // GE_ADD: the 16 rows' residual values of this block all in flight at once,
      // then the sums (one round trip per block instead of one per row)
      float old[16][4];
      if constexpr (EPI == GE_ADD) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + 128 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int col = n0 + 128 * wn + 32 * j + (lane & 31);
            old[r][j] = m < p.T ? static_cast<const float*>(p.out)[(long long)m * p.N + col] : 0.f;
          }
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + 128 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < p.T) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int col = n0 + 128 * wn + 32 * j + (lane & 31);
            float* o = static_cast<float*>(p.out) + (long long)m * p.N + col;
            if constexpr (EPI == GE_ADD) *o = old[r][j] + acc[i][j][r];
            else *o = acc[i][j][r];
          }
        }
        __builtin_amdgcn_sched_barrier(0);   // one row at a time: short live ranges
      }
    }
  }
}

// ---- 3. RoPE + K/V append for the chunk ------------------------------------------------------
// qkv [T, (nq + 2 nkv) hd] f32 from the GEMM: q heads are rotated in place; k heads
// rotated and v heads copied into cache rows p0 .. p0 + T - 1 (bf16, 16-row tiles).

// q heads: rotated in place, one thread per (row, head, 4 dims of the first half) and
// their partners i + hd/2 (16-byte accesses)
__global__ void k_pf_rope_q(float* qkv, int T, int nq, int nkv, int hd, int p0, const float* rope_cs) {
  const int half = hd >> 1, h4 = half >> 2;
  const int heads = nq + 2 * nkv;
  const long long n = (long long)T * nq * h4;
  for (long long u = blockIdx.x * (long long)blockDim.x + threadIdx.x; u < n;
       u += (long long)gridDim.x * blockDim.x) {
    const int t = int(u / (nq * h4));
    const int rem = int(u - (long long)t * nq * h4);
    const int hh = rem / h4, i0 = 4 * (rem - hh * h4);
    const int pos = p0 + t;
    float* row = qkv + (long long)t * heads * hd + (long long)hh * hd;
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(row + i0);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(row + half + i0);
    const float* cs = rope_cs + 2 * ((long long)pos * half + i0);
    const f32x4 c01 = *reinterpret_cast<const f32x4*>(cs), c23 = *reinterpret_cast<const f32x4*>(cs + 4);
    const float c[4] = {c01.x, c01.z, c23.x, c23.z}, sn[4] = {c01.y, c01.w, c23.y, c23.w};
    const float x0[4] = {a0.x, a0.y, a0.z, a0.w}, x1[4] = {a1.x, a1.y, a1.z, a1.w};
    float o0[4], o1[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o0[e] = x0[e] * c[e] - x1[e] * sn[e];
      o1[e] = x0[e] * sn[e] + x1[e] * c[e];
    }
    *reinterpret_cast<f32x4*>(row + i0) = f32x4{o0[0], o0[1], o0[2], o0[3]};
    *reinterpret_cast<f32x4*>(row + half + i0) = f32x4{o1[0], o1[1], o1[2], o1[3]};
  }
}

// k and v heads into the cache tiles with whole 16-byte pieces.  Units [0, nk): one
// thread per (row, kv head, group of 8 dims of the first half): the 8 dims and their
// rotation partners i + hd/2, each group's 8 bf16 of one row contiguous in the K tile.
// Units [nk, nk + nv): one thread per (kv head, dim, 16-row tile the chunk touches):
// that dim's 16 rows of the V^T tile (32 bytes) when the chunk covers the whole tile,
// else only its own rows.
__global__ void k_pf_kv_append(const float* qkv, int T, int nq, int nkv, int hd, int p0,
                               const float* rope_cs, int ctx_max, uint16_t* kc, uint16_t* vc) {
  const int half = hd >> 1, hg = half >> 3;
  const int heads = nq + 2 * nkv;
  const int tb = p0 >> 4, ntl = ((p0 + T - 1) >> 4) - tb + 1;
  const long long nk = (long long)T * nkv * hg, nv = (long long)nkv * hd * ntl;
  for (long long u = blockIdx.x * (long long)blockDim.x + threadIdx.x; u < nk + nv;
       u += (long long)gridDim.x * blockDim.x) {
    if (u < nk) {
      const int t = int(u / (nkv * hg));
      const int rem = int(u - (long long)t * nkv * hg);
      const int g = rem / hg, j = rem - g * hg, i0 = 8 * j;
      const int pos = p0 + t;
      const float* row = qkv + (long long)t * heads * hd + (long long)(nq + g) * hd;
      const float* cs = rope_cs + 2 * ((long long)pos * half + i0);
      uint32_t w0[4], w1[4];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(row + i0 + 4 * q);
        const f32x4 a1 = *reinterpret_cast<const f32x4*>(row + half + i0 + 4 * q);
        const f32x4 c01 = *reinterpret_cast<const f32x4*>(cs + 8 * q);       // cos, sin of i0 + 4q, + 1
        const f32x4 c23 = *reinterpret_cast<const f32x4*>(cs + 8 * q + 4);   // of i0 + 4q + 2, + 3
        const float c[4] = {c01.x, c01.z, c23.x, c23.z}, sn[4] = {c01.y, c01.w, c23.y, c23.w};
        const float x0[4] = {a0.x, a0.y, a0.z, a0.w}, x1[4] = {a1.x, a1.y, a1.z, a1.w};
        uint16_t o0[4], o1[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o0[e] = f32_to_bf16(x0[e] * c[e] - x1[e] * sn[e]);
          o1[e] = f32_to_bf16(x0[e] * sn[e] + x1[e] * c[e]);
        }
        w0[2 * q] = o0[0] | (uint32_t)o0[1] << 16;
        w0[2 * q + 1] = o0[2] | (uint32_t)o0[3] << 16;
        w1[2 * q] = o1[0] | (uint32_t)o1[1] << 16;
        w1[2 * q + 1] = o1[2] | (uint32_t)o1[3] << 16;
      }
      const long long tile = (long long)g * (ctx_max >> 4) + (pos >> 4);
      const long long off = (tile * (hd >> 3) + j) * 128 + (pos & 15) * 8;
      *reinterpret_cast<u32x4*>(kc + off) = u32x4{w0[0], w0[1], w0[2], w0[3]};
      *reinterpret_cast<u32x4*>(kc + off + (long long)hg * 128) = u32x4{w1[0], w1[1], w1[2], w1[3]};
    } else {
      const long long v = u - nk;
      const int i = int(v % hd);
      const long long r2 = v / hd;
      const int k = int(r2 % ntl), g = int(r2 / ntl);
      const int tp0 = (tb + k) << 4;                       // the tile's first row
      const int lo = max(tp0, p0), hi = min(tp0 + 16, p0 + T);
      const float* col = qkv + (long long)(nq + nkv + g) * hd + i;   // v dim i, row stride heads hd
      const long long base = (((long long)g * (ctx_max >> 4) + (tb + k)) * hd + i) * 16;
      if (lo == tp0 && hi == tp0 + 16) {
        uint32_t wv[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const long long t0 = (long long)(tp0 + 2 * r - p0) * heads * hd;
          wv[r] = f32_to_bf16(col[t0]) | (uint32_t)f32_to_bf16(col[t0 + (long long)heads * hd]) << 16;
        }
        *reinterpret_cast<u32x4*>(vc + base) = u32x4{wv[0], wv[1], wv[2], wv[3]};
        *reinterpret_cast<u32x4*>(vc + base + 8) = u32x4{wv[4], wv[5], wv[6], wv[7]};
      } else {
        for (int pos = lo; pos < hi; ++pos)
          vc[base + (pos & 15)] = f32_to_bf16(col[(long long)(pos - p0) * heads * hd]);
      }
    }
  }
}

// ---- 4. causal attention of the chunk on the matrix cores -----------------------------------
// The decode tile kernel's products with CB blocks of 16 query columns per wave
// (CB = 2, 1 for head dim 256): a workgroup takes kv head g and PA_WAVES CB R
// query rows (R = 16 / G); block b of wave w has the rows t0 + (w CB + b) R ..
// + R - 1, its column c = r G + j being q head g G + j of the block's row r.  Each
// K and V operand read from LDS feeds the products of all CB blocks.  The workgroup walks the key tiles (16 cache rows each) from
// row 0 to its last row's position; each tile of K and V is loaded from HBM / L2
// once per workgroup into LDS (double-buffered through registers: step j + 1 is
// fetched while step j is multiplied, one barrier per step) and every wave forms,
// with an online softmax per column (in base 2: the scale carries log2 e),
//   S^T[16 keys, 16 cols] = K_tile . Q^T          (16x16x32 bf16, q as bf16)
//   O^T[hd, 16 cols]     += V_pair^T . P_pair^T   (16x16x32 bf16, p as bf16)
// where lane (col, grp) holds the scores of keys 4 grp .. 4 grp + 3 of a tile
// for column col.  A pair of tiles (u0, u1) makes one 32-deep PV product: its
// k index 8 grp + e stands for key 4 grp + e of tile u0 (e < 4) or key
// 4 grp + e - 4 of tile u1, which is where lane (col, grp) already holds those
// keys' weights (B operand) and where it reads V^T (A operand), so the weights
// never leave the lane.  K and V are the bf16 cache rows; q and the unnormalised
// weights enter as single bf16 operands (relative error up to 2^-9 each, a
// deviation from the plain softmax(S) V that the decode kernel does not take: it
// splits both into bf16 hi + lo); accumulation is f32 and the softmax sum l adds
// the f32 weights.  Keys past a column's position are masked, and V rows past the
// workgroup's last position (stale cache rows, possibly never written) are
// zeroed as they are staged, so whatever they hold cannot reach the output
// through a zero weight.  The output o / l is rounded to bf16 for the O projection.
struct PaP {
  const float* q;          // [T, nq, hd] rotated (the q part of qkv: row stride qs)
  const uint16_t* kc;      // tiled bf16 caches of the layer
  const uint16_t* vc;
  uint16_t* ob;            // [T, nq hd] bf16
  int T, nq, nkv, p0, ctx_max, qs;
  float scale;
};

constexpr int PA_WAVES = 8;
#ifndef LPS_PA_ORDER
#define LPS_PA_ORDER 1
#endif
constexpr int PA_THREADS = PA_WAVES * WAVE;
#ifndef LPS_PA_KT
#define LPS_PA_KT 4
#endif
// 16-row key tiles per step (one softmax update, one barrier); head dim 256 takes
// half as many so that a step's operands stay in registers
constexpr int pa_nt(int hd) { return hd >= 256 ? LPS_PA_KT / 2 : LPS_PA_KT; }
static_assert(LPS_PA_KT % 4 == 0, "PV takes the key tiles in pairs");
typedef short i16x8 __attribute__((ext_vector_type(8)));

// column blocks (16 columns each) per wave: two share every K and V operand read
constexpr int pa_cb(int hd) { return hd >= 256 ? 1 : 2; }

template <int HD, int G>
__global__ __launch_bounds__(PA_THREADS) __attribute__((amdgpu_waves_per_eu(1, 2)))
void k_pf_attn(PaP p) {
  constexpr int KK = HD / 32, DT = HD / 16, R = 16 / G;
  constexpr int CB = pa_cb(HD);                 // column blocks per wave
  constexpr int TILE = 16 * HD;                 // elements of one K (or V) 16-row tile
  constexpr int VP = 20;                        // LDS row of a V^T tile: 16 keys + 4 pad
  constexpr int VTILE = HD * VP;                // LDS elements of one V tile
  constexpr int NT = pa_nt(HD);                 // tiles per step
  constexpr int BUF = NT * (TILE + VTILE);      // LDS elements of one step buffer
  constexpr int CK = NT * TILE / 8;             // 16-byte chunks of a step's K (and of its V) tiles
  static_assert(CK % PA_THREADS == 0, "whole chunks of K and of V per thread");
  constexpr int LPT = CK / PA_THREADS;          // K (and V) chunks per thread per step
  // [2][NT K tiles | NT V tiles]: K tiles as in the cache; V^T rows padded to 40 bytes
  // so the 16 lanes of a PV operand read (rows 32 bytes apart otherwise) hit
  // distinct banks
  extern __shared__ __attribute__((aligned(16))) uint16_t kv_lds[];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int col = lane & 15, grp = lane >> 4;
  // One linear grid over (row block, kv head): workgroup b takes kv head b % nkv,
  // so consecutive workgroups, which the dispatcher deals to the 8 XCDs in turn,
  // keep each head on the same XCDs (its K/V tiles stay in those L2s), and row
  // block nrb - 1 - b / nkv, so the longest causal walks start first.
#if LPS_PA_ORDER
  const int nrb = (p.T + PA_WAVES * CB * R - 1) / (PA_WAVES * CB * R);
  const int g = blockIdx.x % p.nkv;
  const int rb = nrb - 1 - (int)blockIdx.x / p.nkv;
#else
  const int g = blockIdx.y;
  const int rb = blockIdx.x;
#endif
  const int tb = rb * PA_WAVES * CB * R;   // the workgroup's first row
  const int r = col / G, hh = col - r * G;
  int tr[CB], pos[CB];
#pragma unroll
  for (int b = 0; b < CB; ++b) {
    tr[b] = tb + (w * CB + b) * R + r;
    pos[b] = p.p0 + min(tr[b], p.T - 1);        // rows past T: a valid row's copy, never stored
  }
  const int last = p.p0 + min(tb + PA_WAVES * CB * R, p.T) - 1;   // the workgroup's last position
  const int nsteps = (last >> 4) / NT + 1;
  // steps whose keys every row of the workgroup sees (no mask): keys < p0 + tb + 1
  const int nfree = min((p.p0 + tb + 1) / (16 * NT), nsteps);
  // scores in base 2: e^(s / sqrt(hd) - m) = 2^(s log2(e) / sqrt(hd) - m'), one v_exp_f32 each
  const float scale2 = p.scale * 1.44269504088896341f;

  // B operands of S^T: q of column col of each block, dims 32 kk + 8 grp .. + 7, as bf16
  bf16x8 qb[CB][KK];
#pragma unroll
  for (int b = 0; b < CB; ++b) {
    const float* qrow = p.q + (long long)(pos[b] - p.p0) * p.qs + (long long)(g * G + hh) * HD + 8 * grp;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const f32x4 q0 = *reinterpret_cast<const f32x4*>(qrow + 32 * kk);
      const f32x4 q1 = *reinterpret_cast<const f32x4*>(qrow + 32 * kk + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) qb[b][kk][e] = static_cast<__bf16>(e < 4 ? q0[e] : q1[e - 4]);
    }
  }
  const long long head = (long long)g * p.ctx_max * HD;     // elements before kv head g
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.kc + head), (short)0, p.ctx_max * HD * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.vc + head), (short)0, p.ctx_max * HD * 2, 0x00020000);
  // Thread tid stages chunks tid, tid + PA_THREADS, ... of the step's K tiles and the
  // same chunks of its V tiles.  A step's NT tiles are contiguous in the caches, so
  // chunk c of step S sits at byte S * NT * TILE * 2 + 16 c; tiles past the cache
  // read as zeros through the resource bound (their keys are masked).  The LDS
  // places are the same every step: K chunks packed, V chunks (half a V^T row of
  // one tile) at their padded row.
  int vdst[LPT];
#pragma unroll
  for (int c = 0; c < LPT; ++c) {
    const int e = (tid + c * PA_THREADS) * 8;   // element in the NT V tiles
    vdst[c] = NT * TILE + (e / TILE) * VTILE + ((e % TILE) >> 4) * VP + (e & 15);
  }
  u32x4 stk[LPT], stv[LPT];
#define PA_FETCH(S)                                                                           \
  _Pragma("unroll") for (int c = 0; c < LPT; ++c) {                                           \
    const int off = (S) * (NT * TILE * 2) + (tid + c * PA_THREADS) * 16;                      \
    stk[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0)); \
    stv[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0)); \
  }
  // V elements of keys past `last` in the staged step S: the chunk's 8 elements are
  // 8 consecutive keys of one V^T row, two per 32-bit word (the lower key in the low half)
  auto zero_stale_v = [&](int S) {
#pragma unroll
    for (int c = 0; c < LPT; ++c) {
      const int e = (tid + c * PA_THREADS) * 8;
      const int key0 = 16 * (S * NT + e / TILE) + (e & 15);
      uint32_t wv[4] = {stv[c].x, stv[c].y, stv[c].z, stv[c].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (key0 + 2 * j > last) wv[j] = 0u;
        else if (key0 + 2 * j + 1 > last) wv[j] &= 0xFFFFu;
      }
      stv[c] = u32x4{wv[0], wv[1], wv[2], wv[3]};
    }
  };
#define PA_PUT(BUFI)                                                                          \
  _Pragma("unroll") for (int c = 0; c < LPT; ++c) {                                           \
    *reinterpret_cast<u32x4*>(kv_lds + (BUFI) * BUF + (tid + c * PA_THREADS) * 8) = stk[c];    \
    uint16_t* dst = kv_lds + (BUFI) * BUF + vdst[c];                                          \
    *reinterpret_cast<u32x2*>(dst) = u32x2{stv[c].x, stv[c].y};                               \
    *reinterpret_cast<u32x2*>(dst + 4) = u32x2{stv[c].z, stv[c].w};                           \
  }

  f32x4 o[CB][DT];
  float m2[CB], l[CB];   // running max of the base-2 scores, sum of weights
#pragma unroll
  for (int b = 0; b < CB; ++b) {
    m2[b] = -INFINITY;
    l[b] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[b][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One step: NT key tiles.  The first step holds key 0, which every row sees, so
  // the running max is finite from then on and a masked score (-inf) gives a zero
  // weight through exp2 without any select.
  auto step = [&](int sj, auto masked) {
    constexpr bool MASK = decltype(masked)::value;
    const int bi = sj & 1;
    if (sj + 1 < nsteps) { PA_FETCH(sj + 1) }
    const uint16_t* kt = kv_lds + bi * BUF;
    const uint16_t* vt = kt + NT * TILE;
    f32x4 s[CB][NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) {
#pragma unroll
      for (int b = 0; b < CB; ++b) s[b][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + u * TILE + (4 * kk + grp) * 128 + col * 8);
#pragma unroll
        for (int b = 0; b < CB; ++b)
          s[b][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[b][kk], s[b][u], 0, 0, 0);
      }
    }
    bf16x8 pp[CB][NT / 2];   // B operands of the tile pairs
    bool moved = false;
    float alpha[CB];
#pragma unroll
    for (int b = 0; b < CB; ++b) {
      float mt = -INFINITY;
#pragma unroll
      for (int u = 0; u < NT; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (MASK) {
            const int key = 16 * (sj * NT + u) + 4 * grp + i;
            s[b][u][i] = key <= pos[b] ? s[b][u][i] : -INFINITY;
          }
          mt = fmaxf(mt, s[b][u][i]);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 16, WAVE));
      mt = fmaxf(mt, __shfl_xor(mt, 32, WAVE));
      const float mn2 = fmaxf(m2[b], mt * scale2);
      alpha[b] = __builtin_amdgcn_exp2f(m2[b] - mn2);
      moved |= alpha[b] != 1.f;
      float ls = 0.f;
      i16x4 pb[NT];
#pragma unroll
      for (int u = 0; u < NT; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(s[b][u][i], scale2, -mn2));
          ls += pv;
          pb[u][i] = __builtin_bit_cast(short, static_cast<__bf16>(pv));
        }
      ls += __shfl_xor(ls, 16, WAVE);
      ls += __shfl_xor(ls, 32, WAVE);
      l[b] = fmaf(l[b], alpha[b], ls);
      m2[b] = mn2;
#pragma unroll
      for (int v = 0; v < NT / 2; ++v)
        pp[b][v] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(pb[2 * v], pb[2 * v + 1], 0, 1, 2, 3,
                                                                       4, 5, 6, 7));
    }
    if (__any(moved)) {   // a column's maximum moved: rescale the sums
#pragma unroll
      for (int b = 0; b < CB; ++b)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[b][dt] *= alpha[b];
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int v = 0; v < NT / 2; ++v) {
        const uint16_t* vp = vt + (16 * dt + col) * VP + 4 * grp;
        const i16x4 a0 = *reinterpret_cast<const i16x4*>(vp + (2 * v) * VTILE);
        const i16x4 a1 = *reinterpret_cast<const i16x4*>(vp + (2 * v + 1) * VTILE);
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int b = 0; b < CB; ++b)
          o[b][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pp[b][v], o[b][dt], 0, 0, 0);
      }
    if (sj + 1 < nsteps) {
      if (sj + 2 == nsteps) zero_stale_v(sj + 1);
      PA_PUT(bi ^ 1)
    }
    __syncthreads();
  };

  PA_FETCH(0)
  if (nsteps == 1) zero_stale_v(0);
  PA_PUT(0)
  __syncthreads();
  int sj = 0;
  for (; sj < nfree; ++sj) step(sj, std::false_type{});
  for (; sj < nsteps; ++sj) step(sj, std::true_type{});
#undef PA_FETCH
#undef PA_PUT
#pragma unroll
  for (int b = 0; b < CB; ++b) {
    if (tr[b] < p.T) {
      const float inv = 1.0f / l[b];
      uint16_t* dst = p.ob + (long long)tr[b] * p.nq * HD + (long long)(g * G + hh) * HD + 4 * grp;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint32_t lo = f32_to_bf16(o[b][dt][0] * inv) | (uint32_t)f32_to_bf16(o[b][dt][1] * inv) << 16;
        const uint32_t hi = f32_to_bf16(o[b][dt][2] * inv) | (uint32_t)f32_to_bf16(o[b][dt][3] * inv) << 16;
        *reinterpret_cast<u32x2*>(dst + 16 * dt) = u32x2{lo, hi};
      }
    }
  }
}

// ---- host side ---------------------------------------------------------------------------
static dim3 rows_grid(long long n) {
  long long b = (n + 255) / 256;
  return dim3((unsigned)(b < 8192 ? (b < 1 ? 1 : b) : 8192));
}

template <int EPI>
static int gemm(const uint16_t* a, const uint16_t* b, void* out, int T, int N, int K, hipStream_t st) {
  const size_t lds = MM_LDS;
  int rc = ensure_lds((const void*)k_dense_gemm<EPI>, lds);
  if (rc) return rc;
  DgP p{a, b, out, T, N, K};
  const int nt = EPI == GE_SWIGLU ? N / (DN / 2) : N / DN;
  hipLaunchKernelGGL((k_dense_gemm<EPI>), dim3(nt, (T + DM - 1) / DM), dim3(MM_THREADS), lds, st, p);
  LPS_HIP(hipGetLastError());
  return LPS_OK;
}

template <int HD, int G>
static int attn_go(const PaP& p, hipStream_t st) {
  const int rows = PA_WAVES * pa_cb(HD) * (16 / G);   // rows per workgroup
#if LPS_PA_ORDER
  const dim3 grid(((p.T + rows - 1) / rows) * p.nkv);
#else
  const dim3 grid((p.T + rows - 1) / rows, p.nkv);
#endif
  const size_t lds = size_t(2) * pa_nt(HD) * (16 * HD + 20 * HD) * 2;
  int rc = ensure_lds((const void*)k_pf_attn<HD, G>, lds);
  if (rc) return rc;
  hipLaunchKernelGGL((k_pf_attn<HD, G>), grid, dim3(PA_THREADS), lds, st, p);
  LPS_HIP(hipGetLastError());
  return LPS_OK;
}

template <int HD>
static int attn_hd(const PaP& p, int G, hipStream_t st) {
  switch (G) {
    case 1: return attn_go<HD, 1>(p, st);
    case 2: return attn_go<HD, 2>(p, st);
    case 4: return attn_go<HD, 4>(p, st);
    case 8: return attn_go<HD, 8>(p, st);
    default: return fail(LPS_EUNSUP, "prefill attention: %d q heads per kv head (1, 2, 4, 8)", G);
  }
}

PrefillScratch prefill_scratch(const lps_layer_desc* L, int T) {
  PrefillScratch s{};
  const int nqkv = (L->nq + 2 * L->nkv) * L->hd;
  const int w = std::max(L->d, L->nq * L->hd);
  s.xb = 0;                                            // [T, max(d, nq hd)] bf16 (normed rows, o)
  s.qkv = align256(size_t(T) * w * 2);                 // [T, nqkv] f32
  s.mb = s.qkv + align256(size_t(T) * nqkv * 4);       // [T, ff] bf16
  s.total = s.mb + align256(size_t(T) * L->ff * 2);
  return s;
}

int check_prefill_layer(const lps_layer_desc* L, int T, int p0, const char* who) {
  LPS_REQUIRE(L->nq > 0 && L->ffn_kind == LPS_FFN_DENSE, LPS_EUNSUP,
              "%s: the chunked prefill walks attention layers with a dense FFN (MoE FFN layers "
              "take lps_moe_prefill)", who);
  LPS_REQUIRE(L->wdtype == LPS_BF16 && L->kvdtype == LPS_BF16, LPS_EUNSUP,
              "%s: prefill runs bf16 weights with bf16 caches (got %d / %d)", who, L->wdtype,
              L->kvdtype);
  const int G = L->nq / L->nkv;
  LPS_REQUIRE(G == 1 || G == 2 || G == 4 || G == 8, LPS_EUNSUP,
              "%s: prefill attention needs 1, 2, 4 or 8 q heads per kv head (got %d)", who, G);
  LPS_REQUIRE(L->hd == 64 || L->hd == 128 || L->hd == 256, LPS_EUNSUP, "%s: head dim %d", who, L->hd);
  const int nqkv = (L->nq + 2 * L->nkv) * L->hd;
  LPS_REQUIRE(L->d % 256 == 0 && nqkv % 256 == 0 && (L->nq * L->hd) % 128 == 0 &&
                  L->ff % 128 == 0,
              LPS_EUNSUP,
              "%s: prefill GEMM tiles need d %% 256, (nq + 2 nkv) hd %% 256, nq hd %% 128 and "
              "ff %% 128 == 0 (d %d, qkv %d, nq hd %d, ff %d)",
              who, L->d, nqkv, L->nq * L->hd, L->ff);
  LPS_REQUIRE(L->rope_cs, LPS_EINVAL, "%s: prefill needs the layer's rope_cs table", who);
  LPS_REQUIRE(T >= 1 && p0 >= 0 && (long long)p0 + T <= L->ctx_max, LPS_ERANGE,
              "%s: rows %d .. %d outside the cache [0, %d)", who, p0, p0 + T - 1, L->ctx_max);
  // the GEMMs address their operands through buffer resources with 32-bit byte
  // offsets: every operand (bf16 rows, f32 QKV and residual rows, weights) stays
  // below 2 GiB, else the chunk is refused before anything is enqueued
  const long long big = std::max({(long long)T * std::max({L->d, L->nq * L->hd, L->ff}) * 2,
                                  (long long)T * nqkv * 4, (long long)T * L->d * 4,
                                  (long long)2 * L->ff * L->d * 2, (long long)nqkv * L->d * 2});
  LPS_REQUIRE(big < (1LL << 31), LPS_EUNSUP,
              "%s: a %lld-byte operand at T %d (the kernels address below 2 GiB with 32-bit "
              "offsets; split the chunk)", who, big, T);
  return LPS_OK;
}

int prefill_layer(const lps_layer_desc* L, float* x, int T, int p0, void* scratch, hipStream_t st) {
  const PrefillScratch s = prefill_scratch(L, T);
  char* sc = static_cast<char*>(scratch);
  uint16_t* xb = reinterpret_cast<uint16_t*>(sc + s.xb);
  float* qkv = reinterpret_cast<float*>(sc + s.qkv);
  uint16_t* mb = reinterpret_cast<uint16_t*>(sc + s.mb);
  const int d = L->d, nqh = L->nq * L->hd, nqkv = (L->nq + 2 * L->nkv) * L->hd;
  auto w = [](const void* v) { return static_cast<const uint16_t*>(v); };
  hipLaunchKernelGGL(k_pf_rows_norm, dim3(T), dim3(256), 0, st, x, L->g_attn, L->eps, d, xb);
  int rc = gemm<GE_STORE>(xb, w(L->w_qkv), qkv, T, nqkv, d, st);
  if (rc) return rc;
  {
    const int hd = L->hd, nkv = L->nkv;
    const long long nq_units = (long long)T * L->nq * (hd / 8);
    const long long nkv_units = (long long)T * nkv * (hd / 16) +
                                (long long)nkv * hd * (((p0 + T - 1) >> 4) - (p0 >> 4) + 1);
    hipLaunchKernelGGL(k_pf_rope_q, rows_grid(nq_units), dim3(256), 0, st, qkv, T, L->nq, nkv, hd, p0,
                       L->rope_cs);
    hipLaunchKernelGGL(k_pf_kv_append, rows_grid(nkv_units), dim3(256), 0, st, qkv, T, L->nq, nkv, hd,
                       p0, L->rope_cs, L->ctx_max, static_cast<uint16_t*>(L->k_cache),
                       static_cast<uint16_t*>(L->v_cache));
  }
  PaP pa{qkv, static_cast<const uint16_t*>(L->k_cache), static_cast<const uint16_t*>(L->v_cache),
         xb, T, L->nq, L->nkv, p0, L->ctx_max, nqkv, 1.0f / sqrtf(float(L->hd))};
  const int G = L->nq / L->nkv;
  switch (L->hd) {
    case 64: rc = attn_hd<64>(pa, G, st); break;
    case 128: rc = attn_hd<128>(pa, G, st); break;
    default: rc = attn_hd<256>(pa, G, st); break;
  }
  if (rc) return rc;
  rc = gemm<GE_ADD>(xb, w(L->w_o), x, T, d, nqh, st);
  if (rc) return rc;
  hipLaunchKernelGGL(k_pf_rows_norm, dim3(T), dim3(256), 0, st, x, L->g_ffn, L->eps, d, xb);
  rc = gemm<GE_SWIGLU>(xb, w(L->w_gu), mb, T, L->ff, d, st);
  if (rc) return rc;
  rc = gemm<GE_ADD>(mb, w(L->w_d), x, T, d, L->ff, st);
  if (rc) return rc;
  LPS_HIP(hipGetLastError());
  return LPS_OK;
}

// x rows = E[tok[t]] widened to f32 (tokens read on the device; outside [0, vocab): NaN)
template <int WT>
__global__ void k_embed_rows(const void* table, int vocab, int d, const int32_t* tok, float* x) {
  const int t = blockIdx.y;
  const int id = tok[t];
  const bool ok = id >= 0 && id < vocab;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < d; i += gridDim.x * blockDim.x) {
    float v;
    if (!ok) v = __uint_as_float(0x7FC00000u);
    else if (WT == LPS_F32) v = static_cast<const float*>(table)[(long long)id * d + i];
    else v = bf16_to_f32(static_cast<const uint16_t*>(table)[(long long)id * d + i]);
    x[(long long)t * d + i] = v;
  }
}

int launch_embed_rows(const void* table, int wdtype, int vocab, int d, const int32_t* tok, int T,
                      float* x, hipStream_t st) {
  const dim3 grid((d + 255) / 256, T);
  if (wdtype == LPS_F32)
    hipLaunchKernelGGL(k_embed_rows<LPS_F32>, grid, dim3(256), 0, st, table, vocab, d, tok, x);
  else
    hipLaunchKernelGGL(k_embed_rows<LPS_BF16>, grid, dim3(256), 0, st, table, vocab, d, tok, x);
  LPS_HIP(hipGetLastError());
  return LPS_OK;
}

}  // namespace lps
