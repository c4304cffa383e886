// Batch-1 weight-streaming GEMV for gfx950, with the decode path's fused
// prologues and epilogues.
//
// Decode at batch 1 reads every weight byte once per token and does ~1 flop per
// byte, so these kernels are HBM-bound (ninfer "Multi-GPU: layer pipeline
// stages", What it is and is not: decode is weight-bandwidth-bound).  Design:
//  - one wave (64 lanes) computes one "unit" of two rows; lane l takes the
//    16-byte chunks l, l+64, l+128, ... of both rows, so every load instruction
//    of a wave moves 1 KiB of one row, fully coalesced; every chunk of a row
//    always lands on the same lane in the same order whatever the row length,
//    so zero chunks appended at the end of K (the padded dummy columns) leave
//    each lane's partial sum, and the result, bit for bit unchanged;
//  - a wave walks its units in batches of U chunks per lane and row, and issues
//    the loads of the next batch before the FMAs of the current one (double
//    buffering in registers), through buffer resources sized to the row, so a
//    ragged last batch needs no per-lane branch;
//  - the activation vector (f32, optionally RMS-normalised on the way in) sits
//    in LDS, copied there by the LDS DMA path, read once per block from L2 and
//    shared by the block's waves;
//  - the two rows of a unit are chosen so that the epilogue has what it needs:
//    rows (i, i + hd/2) of one head for RoPE, rows (i, ff + i) for SwiGLU;
//  - MXFP4 chunks are 16 bytes of codes = one 32-value e8m0 group, decoded by
//    the gfx950 scaled FP4 -> f32 conversion; the K loop is bounded per group,
//    so no K % 128 assumption exists (TP3 zero-padded dummy heads plan,
//    Implementation status, item 1).
#include "dev.h"
#include "gemv_core.h"
#include "internal.h"

#include <algorithm>
#include <cmath>
#include <type_traits>

namespace lps {

enum { EPI_STORE = LPS_EPI_STORE, EPI_ADD = LPS_EPI_ADD, EPI_SWIGLU = LPS_EPI_SWIGLU, EPI_QKV = 3,
       EPI_LOGITS = 4, EPI_MOEGU = 5, EPI_MOEDN = 6 };

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
  // residual add: when tee0 is set, every updated row also goes to tee0 and tee1
  float* tee0;
  float* tee1;
  // QKV epilogue
  int nq, nkv, hd, pos, ctx_max, kvdtype;
  void* kc;
  void* vc;
  // cos / sin of pos * base^(-2i/hd) for i < hd/2, formed on the host in double
  float rope[2 * 128];
  // device position: pos read from pos_dev, cos / sin from the table rope_cs[pos]
  const int32_t* pos_dev;
  const float* rope_cs;
  // LM-head epilogue: every wave's (max, lowest index of it) over its rows
  float* pval;
  int* pidx;
  // MoE gate/up: unit u = (slot j, i) of slot j's fused [2ff, d] matrix; slots
  // j < kslots are expert eidx[j] (w + eidx[j] * estride), slot kslots the shared w_s
  const uint8_t* w_s;
  const int32_t* eidx;
  long long estride;
  int kslots, ff, E;
  // MoE down: unit u = (slot j, row pair i) of slot j's [rps, K] matrix, dotted with
  // activation row j of x ([kslots + 1, K], all staged); out y[j * rps + row]
  int rps;
};

template <int EPI>
__device__ __forceinline__ void unit_rows(const GemvP& p, int u, int& r0, int& r1) {
  if constexpr (EPI == EPI_MOEGU) {
    const int j = u / p.ff;
    r0 = u - j * p.ff;
    r1 = r0 + p.ff;
  } else if constexpr (EPI == EPI_MOEDN) {
    const int half = p.rps >> 1;
    const int j = u / half;
    r0 = 2 * (u - j * half);
    r1 = r0 + 1;
  } else if constexpr (EPI == EPI_SWIGLU) {
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

// first weight row of the matrix unit u belongs to
template <int EPI>
__device__ __forceinline__ const uint8_t* unit_base(const GemvP& p, int u) {
  if constexpr (EPI == EPI_MOEGU || EPI == EPI_MOEDN) {
    const int j = EPI == EPI_MOEGU ? u / p.ff : u / (p.rps >> 1);
    if (j >= p.kslots) return p.w_s;
    const int e = min(max(p.eidx[j], 0), p.E - 1);   // indices are device data
    return p.w + (long long)e * p.estride;
  } else {
    return p.w;
  }
}

__device__ __forceinline__ void store_kv(void* base, int kvdtype, long long off, float v) {
  if (kvdtype == LPS_F32)
    reinterpret_cast<float*>(base)[off] = v;
  else
    reinterpret_cast<uint16_t*>(base)[off] = f32_to_bf16(v);
}

template <int EPI>
__device__ __forceinline__ void epilogue(const GemvP& p, int u, int r0, int r1, float a0, float a1,
                                         float y0, float y1) {
  if constexpr (EPI == EPI_STORE || EPI == EPI_LOGITS) {
    p.y[r0] = a0;
    if (r1 >= 0) p.y[r1] = a1;
  } else if constexpr (EPI == EPI_ADD) {   // y0, y1: the rows' residual values, loaded early
    const float v0 = y0 + a0, v1 = y1 + a1;
    p.y[r0] = v0;
    if (r1 >= 0) p.y[r1] = v1;
    if (p.tee0) {
      p.tee0[r0] = v0;
      p.tee1[r0] = v0;
      if (r1 >= 0) {
        p.tee0[r1] = v1;
        p.tee1[r1] = v1;
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU || EPI == EPI_MOEGU) {
    p.y[u] = silu(a0) * a1;
  } else if constexpr (EPI == EPI_MOEDN) {
    const int j = u / (p.rps >> 1);
    p.y[(long long)j * p.rps + r0] = a0;
    if (r1 < p.rps) p.y[(long long)j * p.rps + r1] = a1;
  } else {  // QKV: rotate q and k heads at pos, store q, append k and v to the caches
    const int half = p.hd >> 1;
    const int hh = u / half, i = u - hh * half;
    // a device position is clamped into the cache, so a stale one cannot write outside it
    const int pos = p.pos_dev ? min(max(*p.pos_dev, 0), p.ctx_max - 1) : p.pos;
    float o0 = a0, o1 = a1;
    if (hh < p.nq + p.nkv) {
      float cs, sn;
      if (p.pos_dev) {
        const f32x2 t = *reinterpret_cast<const f32x2*>(p.rope_cs + 2 * ((long long)pos * half + i));
        cs = t.x;
        sn = t.y;
      } else {
        cs = p.rope[2 * i];
        sn = p.rope[2 * i + 1];
      }
      o0 = a0 * cs - a1 * sn;
      o1 = a0 * sn + a1 * cs;
    }
    if (hh < p.nq) {
      p.y[r0] = o0;
      p.y[r1] = o1;
    } else {
      const bool is_k = hh < p.nq + p.nkv;
      const int gkv = is_k ? hh - p.nq : hh - p.nq - p.nkv;
      const long long tile = (long long)gkv * (p.ctx_max >> 4) + (pos >> 4);
      if (p.kvdtype == LPS_F32) {            // row pos of [nkv, ctx_max, hd]
        const long long off = ((long long)gkv * p.ctx_max + pos) * p.hd + i;
        void* base = is_k ? p.kc : p.vc;
        store_kv(base, p.kvdtype, off, o0);
        store_kv(base, p.kvdtype, off + half, o1);
      } else if (is_k) {                     // bf16 K: [nkv, ctx_max/16, hd/8, 16, 8]
        const long long off = (tile * (p.hd >> 3) + (i >> 3)) * 128 + (pos & 15) * 8 + (i & 7);
        store_kv(p.kc, p.kvdtype, off, o0);
        store_kv(p.kc, p.kvdtype, off + (long long)(half >> 3) * 128, o1);
      } else {                               // bf16 V: [nkv, ctx_max/16, hd, 16]
        const long long off = (tile * p.hd + i) * 16 + (pos & 15);
        store_kv(p.vc, p.kvdtype, off, o0);
        store_kv(p.vc, p.kvdtype, off + (long long)half * 16, o1);
      }
    }
  }
}

// Launch shapes: threads per workgroup, workgroup cap and U (chunks per lane
// and row in one batch).  Every workgroup stages the activation vector once, so
// staging costs grid * 4K bytes of L2 reads next to the N * K weight bytes.
//  - f32 / bf16 rows: 256 threads (512 for gate/up, O and down), up to 2048
//    groups, U = 4; the LM head 512 threads, up to 1000 groups;
//  - MXFP4 rows (0.53 bytes per weight, so the f32 vector is large next to a
//    row): U is the row's chunks per lane rounded up to 3, 5 or 9, so one batch
//    holds a whole row; 512-thread groups for short rows (many units per wave,
//    double-buffered), 640-thread groups, one per CU, for long rows (about one
//    unit per wave, all of it in flight at once).
#ifndef LPS_BF_NT
#define LPS_BF_NT 256
#endif
#ifndef LPS_BF_MAXB
#define LPS_BF_MAXB 2048
#endif
#ifndef LPS_BF_U
#define LPS_BF_U 4
#endif
// the LM head: 512-thread groups, at most 1000 of them (at a 32000-row vocabulary
// every wave walks two row pairs: 46.4 -> 45.1 us against 256-thread groups capped at
// 2048, which leave some waves one pair and most two)
#ifndef LPS_HEAD_NT
#define LPS_HEAD_NT 512
#endif
#ifndef LPS_HEAD_MAXB
#define LPS_HEAD_MAXB 1000
#endif
#ifndef LPS_MX_NT
#define LPS_MX_NT 512
#endif
#ifndef LPS_MX_MAXB
#define LPS_MX_MAXB 512
#endif
#ifndef LPS_MX_NTL
#define LPS_MX_NTL 640
#endif
#ifndef LPS_MX_MAXBL
#define LPS_MX_MAXBL 256
#endif

template <int EPI, typename A>
__device__ __forceinline__ void finish(const GemvP& p, int u, int r0, int r1, A acc0, A acc1,
                                       float xback, float y0, float y1, int lane, float& best,
                                       int& bidx) {
  float a0 = wave_sum(acc_value(acc0)) * xback;
  float a1 = wave_sum(acc_value(acc1)) * xback;
  if (lane == 0) epilogue<EPI>(p, u, r0, r1, a0, a1, y0, y1);
  if constexpr (EPI == EPI_LOGITS) {   // a NaN logit sticks: the step has no argmax
    if (a0 > best || a0 != a0) { best = a0; bidx = r0; }
    if (r1 >= 0 && (a1 > best || a1 != a1)) { best = a1; bidx = r1; }
  }
}

// A wave walks a flat sequence of
// batches (unit u, chunk base b0 = 0, 64U, 128U, ...; both the same on every
// lane) and issues the loads of the next batch, possibly of its next unit,
// before the FMAs of the current one, so one batch's HBM latency hides behind
// the previous batch's arithmetic.  Each row is read through a buffer resource
// whose size is the row length: a chunk past the row end (the ragged last
// batch) loads as zeros without a memory access, and the batch after the last
// one gets a zero-size resource, so the loop has no per-lane branches and the
// waits on the current batch never cover the next one.  Such lanes multiply the
// zeros by a zero chunk of the staged vector (placed after its K values), which
// adds exactly +0.  The per-lane chunk set and order are those of k_gemv.
typedef int i32x4 __attribute__((ext_vector_type(4)));
constexpr int BUF_DW3 = 0x00020000;   // gfx9 buffer descriptor word 3 (32-bit data format)
constexpr int BUF_NT = 2;             // non-temporal load

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, bytes, BUF_DW3);
}

#define BUF_LOAD(V0, V1, S0, S1, Y0, Y1, UU, B0, LIVE)                                  \
  {                                                                                     \
    const int uu_ = (LIVE) ? (UU) : 0;                                                  \
    int r0_, r1_;                                                                       \
    unit_rows<EPI>(p, uu_, r0_, r1_);                                                   \
    const int rr1_ = r1_ >= 0 ? r1_ : r0_;                                              \
    if constexpr (EPI == EPI_ADD) {                                                     \
      Y0 = p.y[r0_];                                                                    \
      Y1 = p.y[rr1_];                                                                   \
    }                                                                                   \
    const int wb_ = (LIVE) ? (int)p.wrow : 0;                                           \
    const uint8_t* ub_ = unit_base<EPI>(p, uu_);                                        \
    const auto w0_ = row_rsrc(ub_ + (long long)r0_ * p.wrow, wb_);                      \
    const auto w1_ = row_rsrc(ub_ + (long long)rr1_ * p.wrow, wb_);                     \
    /* MXFP4: the batch's scale bytes go out before its codes: loads complete in issue \
       order, and the products read every scale of the batch first, so scales issued  \
       last would hold the first product until the whole batch had landed */           \
    if constexpr (WT == LPS_MXFP4) {                                                    \
      const int sb_ = (LIVE) ? (int)p.srow : 0;                                         \
      const auto s0_ = row_rsrc(p.s + (long long)r0_ * p.srow, sb_);                    \
      const auto s1_ = row_rsrc(p.s + (long long)rr1_ * p.srow, sb_);                   \
      _Pragma("unroll") for (int i = 0; i < U; ++i) {                                   \
        const int c = (B0) + lane + WAVE * i;                                           \
        S0[i] = __builtin_amdgcn_raw_buffer_load_b8(s0_, c, 0, 0);                      \
        S1[i] = __builtin_amdgcn_raw_buffer_load_b8(s1_, c, 0, 0);                      \
      }                                                                                 \
    } else {                                                                            \
      _Pragma("unroll") for (int i = 0; i < U; ++i) S0[i] = S1[i] = 0;                  \
    }                                                                                   \
    _Pragma("unroll") for (int i = 0; i < U; ++i) {                                     \
      const int off = ((B0) + lane + WAVE * i) * 16;                                    \
      V0[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(w0_, off, 0, BUF_NT)); \
      V1[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(w1_, off, 0, BUF_NT)); \
      /* the chunks go out in the order the products read them (chunk i of both    \
         rows, then chunk i + 1), so each product waits only for its own */         \
      __builtin_amdgcn_sched_barrier(0);                                                \
    }                                                                                   \
  }
#define BUF_FMA(V0, V1, S0, S1, B0, XO)                            \
  _Pragma("unroll") for (int i = 0; i < U; ++i) {                  \
    const int c = (B0) + lane + WAVE * i;                          \
    const int xi = c < nck ? (XO) + c * XS : zoff;                 \
    if constexpr (WT == LPS_MXFP4) {                               \
      acc_chunk_mx16(V0[i], S0[i], xh + xi, a0);                   \
      acc_chunk_mx16(V1[i], S1[i], xh + xi, a1);                   \
    } else {                                                       \
      acc_chunk<WT>(V0[i], S0[i], xs + xi, a0);                    \
      acc_chunk<WT>(V1[i], S1[i], xs + xi, a1);                    \
    }                                                              \
  }
// One step of the double-buffered walk: issue the loads of the batch after the
// current one (into buffer N), then consume the current batch (buffer C).  A
// unit is finished when the next batch belongs to another unit.
#define BUF_STEP(CV0, CV1, CS0, CS1, CY0, CY1, NV0, NV1, NS0, NS1, NY0, NY1) \
  {                                                                \
    int nu = u, nb = b0 + WAVE * U;                                \
    if (nb >= nck) { nu = u + stride; nb = 0; }                    \
    const bool more = nu < p.units;                                \
    BUF_LOAD(NV0, NV1, NS0, NS1, NY0, NY1, nu, nb, more)           \
    BUF_FMA(CV0, CV1, CS0, CS1, b0, 0)            \
    if (nu != u) {                                                 \
      int r0, r1;                                                  \
      unit_rows<EPI>(p, u, r0, r1);                                \
      finish<EPI>(p, u, r0, r1, a0, a1, xback, CY0, CY1, lane, best, bidx); \
      a0 = a1 = AccT{};                                            \
    }                                                              \
    if (!more) break;                                              \
    u = nu;                                                        \
    b0 = nb;                                                       \
  }

template <int WT, int EPI, int U, bool NORM, int NT, bool DB>
__global__ __launch_bounds__(NT) void k_gemv_buf(GemvP p) {
  extern __shared__ __attribute__((aligned(16))) float xs[];
  constexpr int CH = Fmt<WT>::CH;
  constexpr int XS = WT == LPS_MXFP4 ? MX16_XS : CH;   // staged floats (MXFP4: halves) per chunk
  _Float16* const xh = reinterpret_cast<_Float16*>(xs);   // the MXFP4 staging (f16)
  constexpr int NW = NT / WAVE;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  const int nck = p.K / CH;
  const int stride = gridDim.x * NW;
  float best = -INFINITY;
  int bidx = 0x7fffffff;
  int u = blockIdx.x * NW + wv;
  int b0 = 0;
  u32x4 va0[U], va1[U], vb0[U], vb1[U];
  uint32_t sa0[U], sa1[U], sb0[U], sb1[U];
  float ya0 = 0.f, ya1 = 0.f, yb0 = 0.f, yb1 = 0.f;   // residual rows (EPI_ADD)
  // the vector's loads (and the norm gain's) go out before the first weight batch,
  // so the staging waits one L2 round trip rather than that batch (loads complete
  // in issue order)
  constexpr int MXR = WT == LPS_MXFP4 ? mx16_maxr(U, NT) : 1;
  Mx16Vec<NORM, MXR> xv;
  f32x4 gpre[GPRE];
  if constexpr (WT == LPS_MXFP4) {
    stage_x_mx16_load<NORM, NT, MXR>(p.x, p.g, p.K, xv);
  } else {
    // MoE down: a workgroup's units all belong to one slot (the launch gives every
    // wave one unit and a slot's unit count is a multiple of the waves per group),
    // so it stages only that slot's activations
    const float* xsrc = p.x;
    if constexpr (EPI == EPI_MOEDN)
      xsrc += (long long)((blockIdx.x * NW) / (p.rps >> 1)) * p.K;
    stage_x_issue<NORM, NT>(xsrc, p.g, p.K, xs, gpre);
  }
  __builtin_amdgcn_sched_barrier(0);
  BUF_LOAD(va0, va1, sa0, sa1, ya0, ya1, u, 0, u < p.units)
  __builtin_amdgcn_sched_barrier(0);
  // a chunk past the row end (zero weights) reads the zero chunk after the staged vector
  const int zoff = WT == LPS_MXFP4 ? nck * XS : p.K;
  float xback = 1.f;   // MXFP4: the power of two the staged vector was scaled down by
  if constexpr (WT == LPS_MXFP4) {
    xback = stage_x_mx16_store<NORM, NT, MXR>(xv, p.x, p.eps, p.K, xh);
  } else {
    if (threadIdx.x < CH) xs[zoff + threadIdx.x] = 0.f;   // zero chunk
    // the weight batch above is 2 U loads (2 U + 2 with the residual rows) after the copy
    stage_x_finish<NORM, NT, 2 * U>(p.g, p.eps, p.K, xs, gpre);
  }
  if (u < p.units) {
    // MXFP4: matrix-core accumulators (acc_chunk_mx16), one per row
    using AccT = std::conditional_t<WT == LPS_MXFP4, f32x4m, float>;
    AccT a0{}, a1{};
    if constexpr (DB) {
      for (;;) {
        BUF_STEP(va0, va1, sa0, sa1, ya0, ya1, vb0, vb1, sb0, sb1, yb0, yb1)
        BUF_STEP(vb0, vb1, sb0, sb1, yb0, yb1, va0, va1, sa0, sa1, ya0, ya1)
      }
    } else {
      // one batch in flight per wave, for launches where a wave meets one batch
      for (;;) {
        BUF_FMA(va0, va1, sa0, sa1, b0, 0)
        int nu = u, nb = b0 + WAVE * U;
        if (nb >= nck) { nu = u + stride; nb = 0; }
        if (nu != u) {
          int r0, r1;
          unit_rows<EPI>(p, u, r0, r1);
          finish<EPI>(p, u, r0, r1, a0, a1, xback, ya0, ya1, lane, best, bidx);
          a0 = a1 = AccT{};
        }
        if (nu >= p.units) break;
        u = nu;
        b0 = nb;
        BUF_LOAD(va0, va1, sa0, sa1, ya0, ya1, u, b0, true)
      }
    }
  }
  if constexpr (EPI == EPI_LOGITS) {
    if (lane == 0) {
      p.pval[blockIdx.x * NW + wv] = best;
      p.pidx[blockIdx.x * NW + wv] = bidx;
    }
  }
}
#undef BUF_LOAD
#undef BUF_FMA
#undef BUF_STEP

// A16 argmax over the LM head's per-wave partials (value, lowest index with
// that value), one workgroup: max with ties to the lower index is an exact
// selection, so any order gives the same answer.  Its own launch after the head
// GEMV: no fence or counter is needed.  A NaN partial (some logit of the step is
// NaN) beats every number, and then, as when no partial holds a maximum at all,
// the id written is `vocab`, outside the table: the next embedding gather turns
// it into a NaN row, so a poisoned step stays poisoned instead of feeding id 0.
__device__ __forceinline__ bool argmax_better(float v, int j, float b, int ix) {
  if (b != b) return false;            // a NaN holds its place
  return v != v || v > b || (v == b && j < ix);
}
// the lowest-index argmax over the head's per-wave partials (vocab when no finite
// maximum), valid on thread 0 (the caller's block is 1024 threads; all of them call)
__device__ __forceinline__ int argmax_partials(const float* pval, const int* pidx, int n, int vocab) {
  float b = -INFINITY;
  int ix = 0x7fffffff;
  // up to AB of a thread's partials loaded at once (one round trip, not one per
  // partial); the selection is exact, so the order of the candidates does not matter
  constexpr int AB = 8;
  for (int i0 = threadIdx.x; i0 < n; i0 += 1024 * AB) {
    float v[AB];
    int j[AB];
#pragma unroll
    for (int u = 0; u < AB; ++u) {
      const int i = i0 + 1024 * u;
      v[u] = i < n ? pval[i] : -INFINITY;
      j[u] = i < n ? pidx[i] : 0x7fffffff;
    }
#pragma unroll
    for (int u = 0; u < AB; ++u)
      if (i0 + 1024 * u < n && argmax_better(v[u], j[u], b, ix)) { b = v[u]; ix = j[u]; }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ob = __shfl_xor(b, o, WAVE);
    const int oi = __shfl_xor(ix, o, WAVE);
    if (argmax_better(ob, oi, b, ix)) { b = ob; ix = oi; }
  }
  __shared__ float bv[16];
  __shared__ int bi[16];
  const int wv = threadIdx.x / WAVE;
  if ((threadIdx.x & (WAVE - 1)) == 0) { bv[wv] = b; bi[wv] = ix; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < 16; ++i)
      if (argmax_better(bv[i], bi[i], b, ix)) { b = bv[i]; ix = bi[i]; }
    return (b != b || ix == 0x7fffffff) ? vocab : ix;
  }
  return 0;
}

__global__ __launch_bounds__(1024) void k_argmax(const float* pval, const int* pidx, int n,
                                                 int vocab, int* out) {
  const int a = argmax_partials(pval, pidx, n, vocab);
  if (threadIdx.x == 0) *out = a;
}

// The token chain at the end of a replayed step (lps_step_finish), one launch: the
// argmax a; with s = state[1]: tok_hist[s] = a, the next input id t (feed[s + 1]
// while fed ids remain, else a) to *tok_cur and its embedding row to x_next (NaN for
// an id outside the table), then the position (unless it reached pos_limit: flag bit
// 0) and the step advance.  The state and the next id's feed entry are read before
// the partials are reduced, so their round trips overlap.
template <int WT>
__global__ __launch_bounds__(1024) void k_step_finish(const float* pval, const int* pidx, int n,
                                                      int vocab, int32_t* state, int pos_limit,
                                                      const int32_t* feed, int n_feed,
                                                      int32_t* tok_hist, int cap, int32_t* tok_cur,
                                                      int32_t* ring_tok, int slots,
                                                      const void* table, int d, float* x_next) {
  const int s = state[1], pos = state[0];
  const bool use_feed = s + 1 >= 0 && s + 1 < n_feed;
  const int fed = use_feed ? feed[s + 1] : -1;
  const int a = argmax_partials(pval, pidx, n, vocab);
  __shared__ int nxt;
  if (threadIdx.x == 0) {
    if (tok_hist && s >= 0 && s < cap) tok_hist[s] = a;
    if (ring_tok && s >= 0) ring_tok[s % slots] = a;
    const int t = use_feed ? fed : a;
    if (tok_cur) *tok_cur = t;
    nxt = t;
    if (pos + 1 < pos_limit) state[0] = pos + 1;
    else state[2] = state[2] | 1;
    state[1] = s + 1;
  }
  __syncthreads();
  const int t = nxt;
  const bool ok = t >= 0 && t < vocab;
  // the row's loads all go out before its stores (one round trip, not one per element)
  constexpr int EB = 4;
  for (int i0 = threadIdx.x; i0 < d; i0 += 1024 * EB) {
    float v[EB];
#pragma unroll
    for (int u = 0; u < EB; ++u) {
      const int i = i0 + 1024 * u;
      if (i >= d || !ok) v[u] = __uint_as_float(0x7FC00000u);
      else if (WT == LPS_F32) v[u] = static_cast<const float*>(table)[(long long)t * d + i];
      else v[u] = bf16_to_f32(static_cast<const uint16_t*>(table)[(long long)t * d + i]);
    }
#pragma unroll
    for (int u = 0; u < EB; ++u)
      if (i0 + 1024 * u < d) x_next[i0 + 1024 * u] = v[u];
  }
}

// ---- launch configuration ---------------------------------------------------
// DB: several batches per wave (double-buffered walk); otherwise each wave meets
// at most one batch and keeps a single set of registers.
template <int WT, int EPI, bool NORM>
static int launch_t(const GemvP& p, hipStream_t st, Stamp sp, int* waves) {
  constexpr int CH = Fmt<WT>::CH;
  const int per_lane = (p.K / CH + WAVE - 1) / WAVE;
  const size_t lds = WT == LPS_MXFP4 ? size_t(p.K / CH + 1) * MX16_XS * sizeof(_Float16)
                                     : (size_t(p.K) + CH) * sizeof(float);
#define LPS_GOB(UU, NTV, MAXBV)                                                                  \
  do {                                                                                           \
    constexpr int NW_ = (NTV) / WAVE;                                                            \
    if (WT == LPS_MXFP4 && p.K / 4 > mx16_maxr(UU, NTV) * (NTV))                                \
      return fail(LPS_EUNSUP, "gemv: MXFP4 K %d above %d", p.K, 4 * mx16_maxr(UU, NTV) * (NTV)); \
    int grid = (p.units + NW_ - 1) / NW_;                                                        \
    /* one unit per wave for the MoE down, and for launches whose units are one batch     \
       each and would come to fewer than two per wave under the cap (there the cap leaves \
       some waves a second unit after the others are done); otherwise capped */           \
    const bool each_ = EPI == EPI_MOEDN || (per_lane <= (UU) && p.units < 2 * (MAXBV) * NW_);  \
    if (!each_ && grid > (MAXBV)) grid = (MAXBV);                                              \
    if (grid < 1) grid = 1;                                                                      \
    const bool db = p.units > grid * NW_ || per_lane > (UU);                                     \
    if (waves) *waves = grid * NW_;                                                              \
    const void* fn_ = db ? (const void*)k_gemv_buf<WT, EPI, UU, NORM, NTV, true>                 \
                         : (const void*)k_gemv_buf<WT, EPI, UU, NORM, NTV, false>;               \
    int rc_ = ensure_lds(fn_, lds);                                                              \
    if (rc_) return rc_;                                                                         \
    if (db)                                                                                      \
      LPS_LAUNCH((k_gemv_buf<WT, EPI, UU, NORM, NTV, true>), dim3(grid), dim3(NTV), lds, st,     \
                 sp.start, sp.stop, p);                                                          \
    else                                                                                         \
      LPS_LAUNCH((k_gemv_buf<WT, EPI, UU, NORM, NTV, false>), dim3(grid), dim3(NTV), lds, st,    \
                 sp.start, sp.stop, p);                                                          \
  } while (0)
  if constexpr (WT == LPS_MXFP4) {
    if (per_lane <= 3) LPS_GOB(3, LPS_MX_NT, LPS_MX_MAXB);
    else if (per_lane <= 5) LPS_GOB(5, LPS_MX_NTL, LPS_MX_MAXBL);
    else if (per_lane <= 9) LPS_GOB(9, LPS_MX_NTL, LPS_MX_MAXBL);
    else LPS_GOB(4, LPS_MX_NT, LPS_MX_MAXB);
  } else {
    // gate/up and the residual-add projections (O, down) in 512-thread groups: half as
    // many groups stage the vector, and at the 8B slice every wave then takes exactly
    // one unit (gate/up 37.2 -> 36.8 us, down 21.0 -> 20.7 us); QKV keeps 256 threads
    // (12.6 us at 512 against 11.5); the head has its own shape (above)
    constexpr int NTB = (EPI == EPI_SWIGLU || EPI == EPI_ADD) ? 2 * LPS_BF_NT : LPS_BF_NT;
    if (per_lane <= 2) LPS_GOB(2, LPS_BF_NT, LPS_BF_MAXB);   // short rows: no empty chunk slots
    else if constexpr (EPI == EPI_LOGITS) LPS_GOB(LPS_BF_U, LPS_HEAD_NT, LPS_HEAD_MAXB);
    else LPS_GOB(LPS_BF_U, NTB, LPS_BF_MAXB);
  }
#undef LPS_GOB
  LPS_HIP(hipGetLastError());
  return LPS_OK;
}

template <int EPI, bool NORM>
static int launch_wt(int wdtype, const GemvP& p, hipStream_t st, Stamp sp, int* waves = nullptr) {
  switch (wdtype) {
    case LPS_F32: return launch_t<LPS_F32, EPI, NORM>(p, st, sp, waves);
    case LPS_BF16: return launch_t<LPS_BF16, EPI, NORM>(p, st, sp, waves);
    case LPS_MXFP4: return launch_t<LPS_MXFP4, EPI, NORM>(p, st, sp, waves);
  }
  return fail(LPS_EINVAL, "gemv: unknown wdtype %d", wdtype);
}

static void set_rows(GemvP& p, int wdtype, int K) {
  if (wdtype == LPS_F32) p.wrow = (long long)K * 4;
  else if (wdtype == LPS_BF16) p.wrow = (long long)K * 2;
  else { p.wrow = K / 2; p.srow = K / 32; }
}

int launch_gemv(int wdtype, const void* w, const uint8_t* s, int N, int K, const float* x,
                const float* g, float eps, float* y, int mode, hipStream_t st, Stamp sp,
                float* tee0, float* tee1) {
  GemvP p{};
  p.w = static_cast<const uint8_t*>(w);
  p.s = s;
  p.N = N;
  p.K = K;
  p.x = x;
  p.g = g;
  p.eps = eps;
  p.y = y;
  if (mode == EPI_ADD && tee0 && tee1) {
    p.tee0 = tee0;
    p.tee1 = tee1;
  }
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

int launch_moe_gu(const void* w_e, const void* w_s, const int32_t* eidx, int E, int kslots, int ff,
                  int d, const float* x, const float* g, float eps, float* y, hipStream_t st,
                  Stamp sp) {
  GemvP p{};
  p.w = static_cast<const uint8_t*>(w_e);
  p.w_s = static_cast<const uint8_t*>(w_s);
  p.eidx = eidx;
  p.E = E;
  p.kslots = kslots;
  p.ff = ff;
  p.estride = 2LL * ff * d * 2;
  p.N = 2 * ff;
  p.K = d;
  p.x = x;
  p.g = g;
  p.eps = eps;
  p.y = y;
  p.units = (kslots + 1) * ff;
  set_rows(p, LPS_BF16, d);
  return launch_wt<EPI_MOEGU, true>(LPS_BF16, p, st, sp);
}

int launch_moe_down(const void* w_e, const void* w_s, const int32_t* eidx, int E, int kslots,
                    int d, int ff, const float* m, float* z, hipStream_t st, Stamp sp) {
  GemvP p{};
  p.w = static_cast<const uint8_t*>(w_e);
  p.w_s = static_cast<const uint8_t*>(w_s);
  p.eidx = eidx;
  p.E = E;
  p.kslots = kslots;
  p.rps = d;
  p.estride = (long long)d * ff * 2;
  p.N = d;
  p.K = ff;
  p.x = m;
  p.y = z;
  p.units = (kslots + 1) * (d / 2);
  set_rows(p, LPS_BF16, ff);
  return launch_wt<EPI_MOEDN, false>(LPS_BF16, p, st, sp);
}

// cos, sin of pos * theta_i, theta_i = base^(-2i / hd), formed in double and
// rounded once to f32 (the angle reaches ~1e4 rad at long contexts)
void rope_cos_sin(float base, int hd, int pos, int i, float* cs) {
  const double theta = std::pow(double(base), -2.0 * double(i) / double(hd));
  const double ang = double(pos) * theta;
  cs[0] = float(std::cos(ang));
  cs[1] = float(std::sin(ang));
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
  // in double, once per launch, and hand the f32 values to every block (with a
  // device position, the same values come from the table rope_cs)
  p.pos_dev = a.pos_dev;
  p.rope_cs = L->rope_cs;
  for (int i = 0; a.pos_dev == nullptr && i < L->hd / 2; ++i)
    rope_cos_sin(L->rope_base, L->hd, a.pos, i, &p.rope[2 * i]);
  p.kc = L->k_cache;
  p.vc = L->v_cache;
  set_rows(p, L->wdtype, L->d);
  return launch_wt<EPI_QKV, true>(L->wdtype, p, st, sp);
}

// most per-wave (value, index) partials an LM-head launch can write
static size_t head_waves_max() {
  return std::max(size_t(LPS_BF_MAXB) * (LPS_BF_NT / WAVE),
                  size_t(LPS_HEAD_MAXB) * (LPS_HEAD_NT / WAVE));
}

size_t head_scratch(const lps_head_desc* h) {
  (void)h;
  return 2 * align256(head_waves_max() * 4);
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
  p.pidx = reinterpret_cast<int*>(sc + align256(head_waves_max() * 4));
  int waves = 0;
  int rc = launch_wt<EPI_LOGITS, true>(h->wdtype, p, st, Stamp{sp.start, nullptr}, &waves);
  if (rc) return rc;
  LPS_LAUNCH(k_argmax, dim3(1), dim3(1024), 0, st, nullptr, sp.stop, p.pval, p.pidx, waves,
             h->vocab, tok);
  LPS_HIP(hipGetLastError());
  return LPS_OK;
}

int launch_step_finish(const lps_head_desc* h, const float* x, float* logits, int32_t* state,
                       int32_t pos_limit, const int32_t* feed, int32_t n_feed, int32_t* tok_hist,
                       float* logits_hist, int32_t hist_cap, const void* embed, int32_t embed_dtype,
                       float* x_next, int32_t* tok_cur, float* ring_logits, int32_t* ring_tok,
                       int32_t ring_slots, void* scratch, hipStream_t st, Stamp sp) {
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
  p.pidx = reinterpret_cast<int*>(sc + align256(head_waves_max() * 4));
  int waves = 0;
  int rc = launch_wt<EPI_LOGITS, true>(h->wdtype, p, st, Stamp{sp.start, nullptr}, &waves);
  if (rc) return rc;
  // the history copy reads the step before the finish launch advances it
  rc = launch_step_advance_hist(state, logits, h->vocab, logits_hist, hist_cap, ring_logits,
                                ring_slots, st);
  if (rc) return rc;
  if (embed_dtype == LPS_F32)
    LPS_LAUNCH(k_step_finish<LPS_F32>, dim3(1), dim3(1024), 0, st, nullptr, sp.stop, p.pval, p.pidx,
               waves, h->vocab, state, pos_limit, feed, n_feed, tok_hist, hist_cap, tok_cur, ring_tok,
               ring_slots, embed, h->d, x_next);
  else
    LPS_LAUNCH(k_step_finish<LPS_BF16>, dim3(1), dim3(1024), 0, st, nullptr, sp.stop, p.pval, p.pidx,
               waves, h->vocab, state, pos_limit, feed, n_feed, tok_hist, hist_cap, tok_cur, ring_tok,
               ring_slots, embed, h->d, x_next);
  LPS_HIP(hipGetLastError());
  return LPS_OK;
}

}  // namespace lps
