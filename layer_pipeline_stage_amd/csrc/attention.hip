// GQA decode attention over a layer's KV cache (split over the context).
//
// q head h reads kv head h / G, G = nq / nkv (TP3 zero-padded dummy heads plan,
// Implementation status item 2 and Geometry: the GQA map is part of the
// weights).  One workgroup takes one (kv head, ATT_CH-row chunk) tile: the
// chunk's K and V rows are streamed once from HBM and reused by all G query
// heads of the group.  bf16 caches (16-row operand-order tiles) run on the
// matrix cores (k_attn_mfma); f32 caches on the VALU (k_attn: scores reduced
// across the lanes of a row by DPP row operations, the weighted V sum formed in
// registers and summed over row slots in LDS).  Each tile writes (m, l, o)
// partials; a second small launch merges every q head's chunks in chunk order,
// so the result does not depend on the order the tiles ran in (and no tile
// waits on, or fences for, another).
#include "dev.h"
#include "internal.h"

#include <cmath>

namespace lps {

#ifndef LPS_ATT_THREADS
#define LPS_ATT_THREADS 256
#endif
#ifndef LPS_ATT_CH
#define LPS_ATT_CH 128
#endif
constexpr int ATT_THREADS = LPS_ATT_THREADS;
constexpr int ATT_NW = ATT_THREADS / WAVE;
constexpr int ATT_CH = LPS_ATT_CH;  // cache rows per tile
constexpr int ATT_RPL = ATT_CH / WAVE;   // rows per lane in the tile softmax

struct AttnP {
  const void* kc;
  const void* vc;
  const float* q;
  float* o;
  float* pm;   // [nkv, nch, G]
  float* pl;   // [nkv, nch, G]
  float* po;   // [nkv, nch, G, HD]
  int G, ctx_max, n, nch;   // rows and chunks (with pos_dev: read on the device)
  int nstride;              // chunks per kv head in the partial arrays
  const int32_t* pos_dev;   // device position: rows 0 .. *pos_dev
  float scale;
};

// rows n and chunks nch of this launch
__device__ __forceinline__ void attn_rows(const AttnP& p, int& n, int& nch) {
  n = p.pos_dev ? min(max(*p.pos_dev, 0), p.ctx_max - 1) + 1 : p.n;   // clamped like the QKV store
  nch = p.pos_dev ? (n + ATT_CH - 1) / ATT_CH : p.nch;
}

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

// Thread (li, rr) of a tile owns elements li*E16 .. li*E16 + E16 - 1 of the rows
// rr, rr + RPP, rr + 2 RPP, ...: its K and V loads are 16 bytes each and all
// of them go out first (one HBM round trip per tile).  The G query heads'
// matching elements stay in registers.  Scores are summed over the LPR lanes of
// a row with DPP steps; the chunk softmax (max, sum) is one wave per head over
// the ATT_CH rows; the weighted V sum is formed in registers from the thread's own
// V rows and summed over the RPP row slots through LDS, in slot order.
template <int HD, int KVT, int G>
__global__ __launch_bounds__(ATT_THREADS) void k_attn(AttnP p) {
  using C = AttnCfg<HD, KVT>;
  constexpr int E16 = C::E16, LPR = C::LPR, RPP = C::RPP;
  constexpr int NP = ATT_CH / RPP;          // rows per thread
  constexpr int ESZ = C::ESZ;
  __shared__ float sc[G][ATT_CH];
  extern __shared__ float red[];            // [RPP][G][HD]

  const int chunk = blockIdx.x, g = blockIdx.y;
  int n_rows, nch;
  attn_rows(p, n_rows, nch);
  if (chunk >= nch) return;   // a device-position launch covers ctx_max rows
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wv = tid / WAVE;
  const int li = tid % LPR, rr = tid / LPR;
  const int row0 = chunk * ATT_CH;
  const long long head_base = (long long)g * p.ctx_max * HD;

  u32x4 kraw[NP], vraw[NP];
#pragma unroll
  for (int ps = 0; ps < NP; ++ps) {
    const int j = row0 + ps * RPP + rr;
    if (j < n_rows) {
      const long long off = (head_base + (long long)j * HD + li * E16) * ESZ;
      kraw[ps] = ld16(static_cast<const char*>(p.kc) + off);
      vraw[ps] = ld16(static_cast<const char*>(p.vc) + off);
    } else {
      kraw[ps] = vraw[ps] = u32x4{0, 0, 0, 0};   // rows past n: zero V, -inf score
    }
  }
  float qv[G][E16];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float* qh = p.q + (long long)(g * G + h) * HD + li * E16;
#pragma unroll
    for (int e = 0; e < E16; e += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(qh + e);
      qv[h][e] = v.x;
      qv[h][e + 1] = v.y;
      qv[h][e + 2] = v.z;
      qv[h][e + 3] = v.w;
    }
  }

  // ---- scores s[h][j] = q_h . k_j * scale ----
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
      for (int e = 0; e < E16; ++e) s[h] = fmaf(kv[e], qv[h][e], s[h]);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = group_sum<LPR>(s[h]);
    if (li == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) sc[h][jl] = (j < n_rows) ? s[h] * p.scale : -INFINITY;
    }
  }
  __syncthreads();
  // ---- chunk softmax: one wave per head, ATT_RPL rows per lane ----
  for (int h = wv; h < G; h += ATT_NW) {
    float v[ATT_RPL];
    float m = -INFINITY;
#pragma unroll
    for (int r = 0; r < ATT_RPL; ++r) {
      v[r] = sc[h][lane + WAVE * r];
      m = fmaxf(m, v[r]);
    }
    m = wave_max(m);
    float l = 0.f;
#pragma unroll
    for (int r = 0; r < ATT_RPL; ++r) {
      const float e = (v[r] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(v[r] - m);
      sc[h][lane + WAVE * r] = e;
      l += e;
    }
    l = wave_sum(l);
    if (lane == 0) {
      const long long pi = ((long long)g * p.nstride + chunk) * G + h;
      p.pm[pi] = m;
      p.pl[pi] = l;
    }
  }
  __syncthreads();
  // ---- o[h][e] = sum_j p[h][j] v_j[e]: per thread over its rows, then over slots ----
  float acc[G][E16];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < E16; ++e) acc[h][e] = 0.f;
#pragma unroll
  for (int ps = 0; ps < NP; ++ps) {
    const int jl = ps * RPP + rr;
    float vv[E16];
    widen16<KVT>(vraw[ps], vv);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float w = sc[h][jl];
#pragma unroll
      for (int e = 0; e < E16; ++e) acc[h][e] = fmaf(w, vv[e], acc[h][e]);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < E16; e += 4)
      *reinterpret_cast<f32x4*>(red + (rr * G + h) * HD + li * E16 + e) =
          f32x4{acc[h][e], acc[h][e + 1], acc[h][e + 2], acc[h][e + 3]};
  __syncthreads();
  const long long ob = ((long long)g * p.nstride + chunk) * G * HD;
  for (int idx = tid; idx < G * (HD / 2); idx += ATT_THREADS) {
    const int h = idx / (HD / 2), e2 = idx - h * (HD / 2);
    f32x2 o = *reinterpret_cast<const f32x2*>(red + h * HD + 2 * e2);
#pragma unroll
    for (int r = 1; r < RPP; ++r) {
      const f32x2 v = *reinterpret_cast<const f32x2*>(red + (r * G + h) * HD + 2 * e2);
      o.x += v.x;
      o.y += v.y;
    }
    *reinterpret_cast<f32x2*>(p.po + ob + h * HD + 2 * e2) = o;
  }
}

// ---- bf16 caches: both products on the matrix cores ---------------------------------
// Both caches are stored in 16-row tiles laid out as the MFMA operands are read:
//   K: [nkv, ctx_max/16, hd/8, 16, 8]  (8-dim groups of the tile's 16 rows)
//   V: [nkv, ctx_max/16, hd, 16]       (the tile transposed: rows contiguous)
// so one wave's 16 rows of K and of V are each one contiguous 4 KiB block
// (hd = 128) and every load instruction reads whole 128-byte lines, and the PV
// product reduces over rows that lie contiguously, as its operands want.  (A
// plain [hd, ctx] transpose of V spreads a wave's rows over hd DRAM pages and
// reads at half the rate.)
// One workgroup of AM_WAVES waves takes one (kv head, ATT_CH-row chunk) tile;
// wave w owns its 16 rows and keeps everything for them in registers:
//   S^T[16 rows, 16 cols] = K[16 rows, hd] . Q^T[hd, 16 cols]   (16x16x32 bf16)
// with the G query heads of the group in columns 0..G-1 (the rest zero) and q
// split into bf16 hi + lo parts (q - hi - lo is below 2^-16 |q|), so the scores
// keep nearly f32 accuracy.  Lane (col, grp) then holds the scores of rows
// 4 grp .. 4 grp + 3 for head col, which is exactly the B operand layout of
//   O^T[hd, 16 cols] += V^T[hd, 16 rows] . P^T[16 rows, 16 cols]   (16x16x16 bf16)
// so the softmax weights (again hi + lo) feed PV without leaving the lane.  The
// wave's softmax max and sum take two cross-lane steps; the AM_WAVES wave
// partials are merged through LDS into the tile's (m, l, o) partial, the same
// format the merge launch reads.
constexpr int AM_WAVES = ATT_CH / 16;
constexpr int AM_THREADS = AM_WAVES * WAVE;
static_assert(AM_THREADS <= 1024, "attention tile too large for one workgroup");
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t att_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// hi = bf16(v) (nearest even), lo = bf16(v - hi)
__device__ __forceinline__ void split_bf16(float v, __bf16& hi, __bf16& lo) {
  hi = static_cast<__bf16>(v);
  lo = static_cast<__bf16>(v - static_cast<float>(hi));
}

template <int HD, int G>
__global__ __launch_bounds__(AM_THREADS) __attribute__((amdgpu_waves_per_eu(1, 2)))
void k_attn_mfma(AttnP p) {
  constexpr int KK = HD / 32;        // QK steps over the head dim
  constexpr int DT = HD / 16;        // PV tiles of the head dim
  constexpr int HDP = HD + 4;        // padded LDS row (spreads the heads over the banks)
  extern __shared__ float red[];     // [AM_WAVES][G][HDP]
  __shared__ float mw[AM_WAVES][G], lw[AM_WAVES][G];

  const int chunk = blockIdx.x, g = blockIdx.y;
  int n_rows, nch;
  attn_rows(p, n_rows, nch);
  if (chunk >= nch) return;   // a device-position launch covers ctx_max rows
  const int lane = threadIdx.x & (WAVE - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  const int col = lane & 15, grp = lane >> 4;
  const int row0 = chunk * ATT_CH + 16 * w;          // the wave's first row
  const bool live = row0 < n_rows;                   // wave-uniform

  // the group's G q heads, staged once per workgroup (one 16-byte load per thread;
  // threads past the G * HD / 4 loads read a valid address and drop it)
  static_assert(G * HD / 4 <= AM_THREADS, "q staging takes one load per thread");
  __shared__ f32x4 qs[G * HD / 4];
  const int qi = min((int)threadIdx.x, G * HD / 4 - 1);
  const f32x4 qv = reinterpret_cast<const f32x4*>(p.q + (long long)g * G * HD)[qi];
  // K tile of rows row0 .. row0 + 15: lane (col, grp) takes row col, dims 32 kk + 8 grp .. + 7
  const char* kbase = static_cast<const char*>(p.kc) + (long long)g * p.ctx_max * HD * 2;
  const auto krs = att_rsrc(kbase, live ? p.ctx_max * HD * 2 : 0);
  u32x4 kr[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    kr[kk] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           krs, (row0 * HD + (4 * kk + grp) * 128 + col * 8) * 2, 0, 2));
  // V tile of rows row0 .. row0 + 15: dims 16 dt + col, rows 4 grp .. 4 grp + 3
  const char* vbase = static_cast<const char*>(p.vc) + (long long)g * HD * p.ctx_max * 2;
  const auto vrs = att_rsrc(vbase, live ? HD * p.ctx_max * 2 : 0);
  const int vt = (row0 >> 4) * HD * 16;              // the tile's first element
  u32x2 vr[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    vr[dt] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                           vrs, (vt + (16 * dt + col) * 16 + 4 * grp) * 2, 0, 2));
  // every load is in flight before any arithmetic: one HBM round trip per wave.  The
  // barrier waits for LDS traffic only, so the scores start once K has landed while
  // V is still on its way.
  __builtin_amdgcn_sched_barrier(0);
  if (threadIdx.x < G * HD / 4) qs[threadIdx.x] = qv;
  lds_barrier();

  // ---- scores ----
  // B operand: q of head col (zero for the padding columns), dims 32 kk + 8 grp .. + 7
  const bool hv = col < G;
  const f32x4* qh = qs + (hv ? col : 0) * (HD / 4) + 2 * grp;
  bf16x8 qhi[KK], qlo[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const f32x4 q0 = qh[8 * kk], q1 = qh[8 * kk + 1];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      __bf16 h, l;
      split_bf16(hv ? (e < 4 ? q0[e] : q1[e - 4]) : 0.f, h, l);
      qhi[kk][e] = h;
      qlo[kk][e] = l;
    }
  }
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, kr[kk]);
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qhi[kk], s, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qlo[kk], s, 0, 0, 0);
  }
  // ---- the wave's softmax over its 16 rows, per head (lanes col, col+16, col+32, col+48) ----
  const int rbase = row0 + 4 * grp;
  float sv[4];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sv[i] = (rbase + i < n_rows) ? s[i] * p.scale : -INFINITY;
    m = fmaxf(m, sv[i]);
  }
  m = fmaxf(m, __shfl_xor(m, 16, WAVE));
  m = fmaxf(m, __shfl_xor(m, 32, WAVE));
  float pv[4], l = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pv[i] = sv[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[i] - m);
    l += pv[i];
  }
  l += __shfl_xor(l, 16, WAVE);
  l += __shfl_xor(l, 32, WAVE);
  i16x4 phi, plo;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __bf16 h, lo;
    split_bf16(pv[i], h, lo);
    phi[i] = __builtin_bit_cast(short, h);
    plo[i] = __builtin_bit_cast(short, lo);
  }
  // ---- PV; V^T values of rows at or past n_rows are zeroed bit-wise first ----
  const int valid = min(max(n_rows - rbase, 0), 4);
  const unsigned long long vmask = valid >= 4 ? ~0ull : ((1ull << (16 * valid)) - 1ull);
  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const unsigned long long bits =
        ((unsigned long long)vr[dt].y << 32 | vr[dt].x) & vmask;
    const i16x4 a = __builtin_bit_cast(i16x4, bits);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, phi, acc, 0, 0, 0);
    o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, plo, acc, 0, 0, 0);
  }
  // ---- merge the waves' partials through LDS ----
  if (hv) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4*>(red + (w * G + col) * HDP + 16 * dt + 4 * grp) = o[dt];
    if (grp == 0) {
      mw[w][col] = m;
      lw[w][col] = l;
    }
  }
  __syncthreads();
  const long long pb = (long long)g * p.nstride + chunk;
  for (int idx = threadIdx.x; idx < G * (HD / 2); idx += AM_THREADS) {
    const int h = idx / (HD / 2), e2 = idx - h * (HD / 2);
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < AM_WAVES; ++v) M = fmaxf(M, mw[v][h]);
    float L = 0.f;
    f32x2 acc = {0.f, 0.f};
#pragma unroll
    for (int v = 0; v < AM_WAVES; ++v) {
      const float sc = mw[v][h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[v][h] - M);
      L = fmaf(sc, lw[v][h], L);
      const f32x2 x = *reinterpret_cast<const f32x2*>(red + (v * G + h) * HDP + 2 * e2);
      acc.x = fmaf(sc, x.x, acc.x);
      acc.y = fmaf(sc, x.y, acc.y);
    }
    if (e2 == 0) {
      p.pm[pb * G + h] = M;
      p.pl[pb * G + h] = L;
    }
    *reinterpret_cast<f32x2*>(p.po + (pb * G + h) * HD + 2 * e2) = acc;
  }
}

// Merge of the chunk partials of one q head: M = max m_c, L = sum_c l_c
// 2^(m_c - M), o = sum_c o_c 2^(m_c - M) / L (the maxima in base-2 units).  A
// separate launch: the partials of all tiles are complete when it starts (stream
// order), so no device-scope fence or counter is needed.  One workgroup per q head;
// thread (part, e2) owns output columns 2 e2, 2 e2 + 1 and the chunks c = part
// (mod P).  It loads the (m, l, o) of up to MERGE_B of its chunks at once, so a
// typical context costs one L2 round trip, and keeps a running maximum with
// rescaling.  The P part results are combined in part order: the result does not
// depend on timing.  512 threads (P = 8 parts at head dim 128, 4 at 256): half the
// parts of 1024 to combine at the end (C3 attention 13.45 -> 13.13 us; at head dim
// 256 an 8192-row context then takes three batches of loads instead of two, and the
// padded decode still gains: 19.28 -> 19.25 us); 256 threads were slower there.
constexpr int MERGE_THREADS = 512;
constexpr int MERGE_B = 8;   // chunks per thread in flight

template <int HD>
__global__ __launch_bounds__(MERGE_THREADS) void k_attn_merge(AttnP p) {
  constexpr int TPH = HD / 2;                  // threads per part
  constexpr int P = MERGE_THREADS / TPH;
  const int hq = blockIdx.x;               // q head
  const int g = hq / p.G, h = hq - g * p.G;
  const int t = threadIdx.x, e2 = t % TPH, part = t / TPH;
  __shared__ float sM[P], sL[P];
  __shared__ f32x2 sO[P][TPH];
  int n_rows, nch;
  attn_rows(p, n_rows, nch);
  const long long base = (long long)g * p.nstride;
  const long long step = (long long)p.G * HD;
  const float* po = p.po + (base * p.G + h) * HD + 2 * e2;
  float M = -INFINITY, L = 0.f;
  f32x2 O = {0.f, 0.f};
  for (int c0 = part; c0 < nch; c0 += MERGE_B * P) {
    float mv[MERGE_B], lv[MERGE_B];
    f32x2 ov[MERGE_B];
#pragma unroll
    for (int k = 0; k < MERGE_B; ++k) {
      const int c = c0 + k * P;
      if (c < nch) {
        const long long pi = (base + c) * p.G + h;
        mv[k] = p.pm[pi];
        lv[k] = p.pl[pi];
        ov[k] = *reinterpret_cast<const f32x2*>(po + c * step);
      } else {
        mv[k] = -INFINITY;
        lv[k] = 0.f;
        ov[k] = f32x2{0.f, 0.f};
      }
    }
    float Mn = M;
#pragma unroll
    for (int k = 0; k < MERGE_B; ++k) Mn = fmaxf(Mn, mv[k]);
    if (Mn != -INFINITY) {
      const float r = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
      L *= r;
      O.x *= r;
      O.y *= r;
#pragma unroll
      for (int k = 0; k < MERGE_B; ++k) {
        const float w = mv[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mv[k] - Mn);
        L = fmaf(w, lv[k], L);
        O.x = fmaf(w, ov[k].x, O.x);
        O.y = fmaf(w, ov[k].y, O.y);
      }
      M = Mn;
    }
  }
  sO[part][e2] = O;
  if (e2 == 0) {
    sM[part] = M;
    sL[part] = L;
  }
  __syncthreads();
  if (t < TPH) {
    float Mt = -INFINITY;
#pragma unroll
    for (int q = 0; q < P; ++q) Mt = fmaxf(Mt, sM[q]);
    float Lt = 0.f;
    f32x2 o = {0.f, 0.f};
#pragma unroll
    for (int q = 0; q < P; ++q) {
      const float w = sM[q] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sM[q] - Mt);
      Lt = fmaf(w, sL[q], Lt);
      o.x = fmaf(w, sO[q][t].x, o.x);
      o.y = fmaf(w, sO[q][t].y, o.y);
    }
    *reinterpret_cast<f32x2*>(p.o + (long long)hq * HD + 2 * t) = f32x2{o.x / Lt, o.y / Lt};
  }
}

static int nchunks(int rows) { return (rows + ATT_CH - 1) / ATT_CH; }

size_t attn_scratch(int nq, int nkv, int hd, int ctx_max) {
  const size_t nch = nchunks(ctx_max);
  const int G = nq / nkv;
  return 2 * align256(size_t(nkv) * nch * G * 4) + align256(size_t(nkv) * nch * G * hd * 4);
}

template <int HD, int KVT, int G>
static int go_g(const AttnP& p, int nkv, hipStream_t st, hipEvent_t start) {
  if constexpr (KVT == LPS_BF16) {
    const size_t lds = size_t(AM_WAVES) * G * (HD + 4) * sizeof(float);
    int rc = ensure_lds((const void*)k_attn_mfma<HD, G>, lds);
    if (rc) return rc;
    LPS_LAUNCH((k_attn_mfma<HD, G>), dim3(p.nch, nkv), dim3(AM_THREADS), lds, st, start, nullptr, p);
    return LPS_OK;
  } else {
    const size_t lds = size_t(AttnCfg<HD, KVT>::RPP) * G * HD * sizeof(float);
    int rc = ensure_lds((const void*)k_attn<HD, KVT, G>, lds);
    if (rc) return rc;
    LPS_LAUNCH((k_attn<HD, KVT, G>), dim3(p.nch, nkv), dim3(ATT_THREADS), lds, st, start, nullptr, p);
    return LPS_OK;
  }
}

template <int HD, int KVT>
static int go(const AttnP& p, int nkv, hipStream_t st, Stamp sp) {
  int rc;
  switch (p.G) {
    case 1: rc = go_g<HD, KVT, 1>(p, nkv, st, sp.start); break;
    case 2: rc = go_g<HD, KVT, 2>(p, nkv, st, sp.start); break;
    case 4: rc = go_g<HD, KVT, 4>(p, nkv, st, sp.start); break;
    case 6: rc = go_g<HD, KVT, 6>(p, nkv, st, sp.start); break;
    case 8: rc = go_g<HD, KVT, 8>(p, nkv, st, sp.start); break;
    default: return fail(LPS_EUNSUP, "attention: %d q heads per kv head not built (1, 2, 4, 6, 8)", p.G);
  }
  if (rc) return rc;
  LPS_LAUNCH((k_attn_merge<HD>), dim3(nkv * p.G), dim3(MERGE_THREADS), 0, st, nullptr, sp.stop, p);
  return LPS_OK;
}

int launch_attention(int nq, int nkv, int hd, int kvdtype, const void* kc, const void* vc,
                     int ctx_max, int n_rows, const float* q, float* o, void* scratch,
                     hipStream_t st, Stamp sp, const int32_t* pos_dev) {
  AttnP p{};
  p.kc = kc;
  p.vc = vc;
  p.q = q;
  p.o = o;
  p.G = nq / nkv;
  p.ctx_max = ctx_max;
  p.pos_dev = pos_dev;
  p.n = pos_dev ? ctx_max : n_rows;
  p.nch = nchunks(p.n);            // the grid; blocks past the device row count exit
  p.nstride = pos_dev ? nchunks(ctx_max) : p.nch;
  // scores in base 2: e^(q.k / sqrt(hd) - m) = 2^(q.k log2(e) / sqrt(hd) - m'), so every
  // softmax and merge weight is one v_exp_f32 (the partials' maxima are in these units)
  p.scale = float(1.4426950408889634 / std::sqrt(double(hd)));
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
