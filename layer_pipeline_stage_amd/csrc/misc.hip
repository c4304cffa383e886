// Small kernels of the decode path: embedding gather, standalone RMSNorm, the
// boundary-slot copy, f32 <-> f16 piece conversions and the MoE combine.
#include "dev.h"
#include "internal.h"

#include <cmath>

namespace lps {

// ---- A2: x = E[tok] (the token is read on the device) ------------------------
template <int WT>
__global__ void k_embed(const void* table, int vocab, int d, const int32_t* tok, float* x) {
  const int t = *tok;
  const bool ok = t >= 0 && t < vocab;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < d; i += gridDim.x * blockDim.x) {
    float v;
    if (!ok) v = __uint_as_float(0x7FC00000u);
    else if (WT == LPS_F32) v = static_cast<const float*>(table)[(long long)t * d + i];
    else v = bf16_to_f32(static_cast<const uint16_t*>(table)[(long long)t * d + i]);
    x[i] = v;
  }
}

// ---- A3 standalone: y = x / sqrt(mean(x^2) + eps) * g (one workgroup) ----------
__global__ __launch_bounds__(256) void k_rmsnorm(const float* x, const float* g, float eps, int d,
                                                  float* y) {
  __shared__ float red[4];
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += 256) ss += x[i] * x[i];
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x / 64] = ss;
  __syncthreads();
  const float r = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / float(d) + eps);
  for (int i = threadIdx.x; i < d; i += 256) y[i] = x[i] * r * g[i];
}

// ---- A14 transport: plain copy ----------------------------------------------------
__global__ void k_copy(const float* __restrict__ src, float* __restrict__ dst, long long n) {
  const long long n4 = n / 4;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n4;
       i += (long long)gridDim.x * blockDim.x)
    reinterpret_cast<f32x4*>(dst)[i] = reinterpret_cast<const f32x4*>(src)[i];
  for (long long i = n4 * 4 + blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

// dst0 = dst1 = src (n floats, 16-byte aligned): the same-stream boundary hop
__global__ void k_copy2(const float* __restrict__ src, float* __restrict__ dst0,
                        float* __restrict__ dst1, long long n) {
  const long long n4 = n / 4;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n4;
       i += (long long)gridDim.x * blockDim.x) {
    const f32x4 v = reinterpret_cast<const f32x4*>(src)[i];
    reinterpret_cast<f32x4*>(dst0)[i] = v;
    reinterpret_cast<f32x4*>(dst1)[i] = v;
  }
  for (long long i = n4 * 4 + blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x)
    dst0[i] = dst1[i] = src[i];
}

// ---- A12: f32 -> f16 (RNE), f16 -> f32 (exact) ----------------------------------------
__global__ void k_f32_to_f16(const float* src, uint16_t* dst, long long n) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x) {
    const _Float16 h = static_cast<_Float16>(src[i]);
    dst[i] = __builtin_bit_cast(uint16_t, h);
  }
}
__global__ void k_f16_to_f32(const uint16_t* src, float* dst, long long lo, long long hi) {
  for (long long i = lo + blockIdx.x * (long long)blockDim.x + threadIdx.x; i < hi;
       i += (long long)gridDim.x * blockDim.x)
    dst[i] = static_cast<float>(__builtin_bit_cast(_Float16, src[i]));
}
// out = f32(x + ((shared + local) + bo)); out may be bo or x (no __restrict__):
// every element is read before it is written, by the same thread.
__global__ void k_combine(float* out, const float* x, const float* shared, const float* local,
                          const float* bo, long long n) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x) {
    const float y = (shared[i] + local[i]) + bo[i];
    const float v = x[i] + y;
    out[i] = v;
  }
}

// f16 -> f32 over [lo, hi), eight halves per thread access (lo, hi multiples of 8, both
// buffers 16-byte aligned); the halves are a last use and stream past the caches.
__global__ void k_f16_to_f32_8(const uint16_t* src, float* dst, long long lo, long long hi) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  const long long n8 = (hi - lo) / 8;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n8;
       i += (long long)gridDim.x * blockDim.x) {
    const long long e = lo + 8 * i;
    const h8 v = __builtin_bit_cast(h8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + e)));
    reinterpret_cast<f32x4*>(dst + e)[0] = f32x4{float(v[0]), float(v[1]), float(v[2]), float(v[3])};
    reinterpret_cast<f32x4*>(dst + e)[1] = f32x4{float(v[4]), float(v[5]), float(v[6]), float(v[7])};
  }
}

// The same, four elements per thread access (all five buffers 16-byte aligned, n a
// multiple of 4); shared, local and bo are last uses and stream past the caches.
__global__ void k_combine4(float* out, const float* x, const float* shared, const float* local,
                           const float* bo, long long n4) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n4;
       i += (long long)gridDim.x * blockDim.x) {
    const f32x4 sv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(shared) + i);
    const f32x4 lv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(local) + i);
    const f32x4 bv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(bo) + i);
    const f32x4 xv = reinterpret_cast<const f32x4*>(x)[i];
    f32x4 v;
    v.x = xv.x + ((sv.x + lv.x) + bv.x);
    v.y = xv.y + ((sv.y + lv.y) + bv.y);
    v.z = xv.z + ((sv.z + lv.z) + bv.z);
    v.w = xv.w + ((sv.w + lv.w) + bv.w);
    reinterpret_cast<f32x4*>(out)[i] = v;
  }
}

static dim3 grid_for(long long n, int threads = 256) {
  long long b = (n + threads - 1) / threads;
  if (b < 1) b = 1;
  if (b > 4096) b = 4096;
  return dim3(unsigned(b));
}

// ---- HBM read calibration: stream every 16-byte chunk once -------------------------------
// STREAM_BLOCKS workgroups of 256 threads; block b reads the contiguous chunk range
// [b * per, (b + 1) * per) with 8 loads of 1 KiB per wave in flight (nontemporal, as
// the GEMVs read weights).  Contiguous per-block ranges reach ~7.0 TB/s on a 4 GiB
// buffer where a grid-stride walk reaches ~5.6-6.2.  The words are folded by XOR so
// nothing is dead code; block b writes its fold to sink[b], and the XOR of the sink
// is the XOR of every 32-bit word of the buffer, whatever the order (exact).
constexpr int STREAM_BLOCKS = LPS_STREAM_SINK;

__global__ __launch_bounds__(256) void k_stream_read(const u32x4* __restrict__ src, long long n16,
                                                     uint32_t* __restrict__ sink) {
  constexpr int UNR = 8;
  const long long per = (n16 + gridDim.x - 1) / gridDim.x;
  const long long b0 = (long long)blockIdx.x * per;
  const long long b1 = b0 + per < n16 ? b0 + per : n16;
  uint32_t acc = 0;
  long long i = b0 + threadIdx.x;
  for (; i + (UNR - 1) * 256 < b1; i += UNR * 256) {
    u32x4 v[UNR];
#pragma unroll
    for (int k = 0; k < UNR; ++k) v[k] = ld_stream16(src + i + k * 256);
#pragma unroll
    for (int k = 0; k < UNR; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < b1; i += 256) {
    const u32x4 v = ld_stream16(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, WAVE);
  __shared__ uint32_t red[4];
  if ((threadIdx.x & (WAVE - 1)) == 0) red[threadIdx.x / WAVE] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// ---- device-side step state of a replayed decode step ----------------------------------
// state[0] = position, state[1] = step, state[2] = flags (bit 0: the position
// reached its limit and stayed).  Both kernels read the step from state[1], so
// the copy runs before the advance in stream order.
// ring (optional): host memory the device addresses directly (a pinned ring of
// `slots` rows); row s % slots receives the logits too, stored from here so no
// copy on another stream has to wait for the step
__global__ void k_hist_logits(const int32_t* state, const float* logits, int vocab, float* hist,
                              int cap, float* ring, int slots) {
  const int s = state[1];
  float* dst = hist && s >= 0 && s < cap ? hist + (long long)s * vocab : nullptr;
  float* rdst = ring && s >= 0 ? ring + (long long)(s % slots) * vocab : nullptr;
  const int stride = gridDim.x * blockDim.x;
  if ((vocab & 3) == 0 && ((reinterpret_cast<uintptr_t>(logits) | reinterpret_cast<uintptr_t>(dst) |
                            reinterpret_cast<uintptr_t>(rdst)) & 15) == 0) {
    // 16 bytes per lane: the ring row crosses to host memory in whole-line writes
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < vocab / 4; i += stride) {
      const f32x4 v = reinterpret_cast<const f32x4*>(logits)[i];
      if (dst) reinterpret_cast<f32x4*>(dst)[i] = v;
      if (rdst) reinterpret_cast<f32x4*>(rdst)[i] = v;
    }
    return;
  }
  // a thread's HB values are loaded before any is stored (one round trip, not one per
  // value: the stores could alias the loads, so they would otherwise wait in turn)
  constexpr int HB = 4;
  for (int i0 = blockIdx.x * blockDim.x + threadIdx.x; i0 < vocab; i0 += stride * HB) {
    float v[HB];
#pragma unroll
    for (int u = 0; u < HB; ++u) v[u] = i0 + stride * u < vocab ? logits[i0 + stride * u] : 0.f;
#pragma unroll
    for (int u = 0; u < HB; ++u) {
      const int i = i0 + stride * u;
      if (i < vocab) {
        if (dst) dst[i] = v[u];
        if (rdst) rdst[i] = v[u];
      }
    }
  }
}

__global__ void k_step_advance(int32_t* state, int pos_limit, const int32_t* argmax,
                               int32_t* tok_cur, const int32_t* feed, int n_feed,
                               int32_t* tok_hist, int cap) {
  if (threadIdx.x != 0) return;
  const int s = state[1];
  if (argmax) {   // a model with a vocabulary: the token chain
    const int a = *argmax;
    if (tok_hist && s >= 0 && s < cap) tok_hist[s] = a;
    // the next step's input: the fed id while ids remain, else this step's argmax
    *tok_cur = (s + 1 >= 0 && s + 1 < n_feed) ? feed[s + 1] : a;
  }
  const int pos = state[0];
  if (pos + 1 < pos_limit) state[0] = pos + 1;
  else state[2] = state[2] | 1;
  state[1] = s + 1;
}

int launch_step_advance_hist(const int32_t* state, const float* logits, int32_t vocab,
                             float* logits_hist, int32_t hist_cap, float* ring_logits,
                             int32_t ring_slots, hipStream_t st) {
  if (!(logits_hist && hist_cap > 0)) logits_hist = nullptr;
  if (logits_hist || ring_logits) {
    hipLaunchKernelGGL(k_hist_logits, grid_for(vocab / 4 + 1), dim3(256), 0, st, state, logits,
                       vocab, logits_hist, hist_cap, ring_logits, ring_slots);
    LPS_HIP(hipGetLastError());
  }
  return LPS_OK;
}

int launch_step_advance(int32_t* state, int32_t pos_limit, const int32_t* argmax, int32_t* tok_cur,
                        const int32_t* feed, int32_t n_feed, int32_t* tok_hist, int32_t hist_cap,
                        const float* logits, int32_t vocab, float* logits_hist, hipStream_t st) {
  int rc = launch_step_advance_hist(state, logits, vocab, logits_hist, hist_cap, nullptr, 0, st);
  if (rc) return rc;
  hipLaunchKernelGGL(k_step_advance, dim3(1), dim3(64), 0, st, state, pos_limit, argmax, tok_cur,
                     feed, n_feed, tok_hist, hist_cap);
  LPS_HIP(hipGetLastError());
  return LPS_OK;
}

// dst[s * dst_stride + i] = src[s * src_stride + i], i < n, at the device step
// s = state[1] clamped into [0, n_rows - 1] (a stride of 0 pins that side)
__global__ void k_row_at_step(const int32_t* state, const float* src, long long src_stride,
                              float* dst, long long dst_stride, int n, int n_rows) {
  const int s = min(max(state[1], 0), n_rows - 1);
  const float* a = src + (long long)s * src_stride;
  float* b = dst + (long long)s * dst_stride;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) b[i] = a[i];
}

int launch_row_at_step(const int32_t* state, const float* src, int64_t src_stride, float* dst,
                       int64_t dst_stride, int32_t n, int32_t n_rows, hipStream_t st) {
  hipLaunchKernelGGL(k_row_at_step, grid_for(n), dim3(256), 0, st, state, src,
                     (long long)src_stride, dst, (long long)dst_stride, n, n_rows);
  LPS_HIP(hipGetLastError());
  return LPS_OK;
}

int launch_copy2_f32(const float* src, float* dst0, float* dst1, int64_t n, hipStream_t st) {
  if (n == 0) return LPS_OK;
  hipLaunchKernelGGL(k_copy2, grid_for(n / 4 + 1), dim3(256), 0, st, src, dst0, dst1, (long long)n);
  LPS_HIP(hipGetLastError());
  return LPS_OK;
}

int launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t st) {
  if (n == 0) return LPS_OK;
  hipLaunchKernelGGL(k_copy, grid_for(n / 4 + 1), dim3(256), 0, st, src, dst, (long long)n);
  LPS_HIP(hipGetLastError());
  return LPS_OK;
}

}  // namespace lps

using namespace lps;

extern "C" int lps_hbm_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  LPS_REQUIRE(src && sink, LPS_EINVAL, "lps_hbm_stream_read: null pointer");
  LPS_REQUIRE(bytes > 0 && bytes % 16 == 0, LPS_EINVAL,
              "lps_hbm_stream_read: bytes %lld must be a positive multiple of 16", (long long)bytes);
  LPS_REQUIRE((reinterpret_cast<uintptr_t>(src) & 15) == 0, LPS_EINVAL,
              "lps_hbm_stream_read: src must be 16-byte aligned");
  hipLaunchKernelGGL(k_stream_read, dim3(STREAM_BLOCKS), dim3(256), 0, as_stream(stream),
                     static_cast<const u32x4*>(src), (long long)(bytes / 16), sink);
  LPS_HIP(hipGetLastError());
  return LPS_OK;
}

extern "C" int lps_embed(const void* table, int32_t wdtype, int32_t vocab, int32_t d,
                         const int32_t* tok, float* x, void* stream) {
  LPS_REQUIRE(table && tok && x, LPS_EINVAL, "lps_embed: null pointer");
  LPS_REQUIRE(vocab > 0 && d > 0, LPS_EINVAL, "lps_embed: vocab %d / d %d must be > 0", vocab, d);
  LPS_REQUIRE(wdtype == LPS_F32 || wdtype == LPS_BF16, LPS_EINVAL,
              "lps_embed: table dtype %d (f32 or bf16 only)", wdtype);
  const dim3 grid = grid_for(d);
  if (wdtype == LPS_F32)
    hipLaunchKernelGGL(k_embed<LPS_F32>, grid, dim3(256), 0, as_stream(stream), table, vocab, d, tok, x);
  else
    hipLaunchKernelGGL(k_embed<LPS_BF16>, grid, dim3(256), 0, as_stream(stream), table, vocab, d, tok, x);
  LPS_HIP(hipGetLastError());
  return LPS_OK;
}

extern "C" int lps_rmsnorm(const float* x, const float* g, float eps, int32_t d, float* y,
                           void* stream) {
  LPS_REQUIRE(x && g && y, LPS_EINVAL, "lps_rmsnorm: null pointer");
  LPS_REQUIRE(d > 0, LPS_EINVAL, "lps_rmsnorm: d %d must be > 0", d);
  hipLaunchKernelGGL(k_rmsnorm, dim3(1), dim3(256), 0, as_stream(stream), x, g, eps, d, y);
  LPS_HIP(hipGetLastError());
  return LPS_OK;
}

extern "C" int lps_copy_f32(const float* src, float* dst, int64_t n, void* stream) {
  LPS_REQUIRE(n >= 0, LPS_EINVAL, "lps_copy_f32: n %lld < 0", (long long)n);
  LPS_REQUIRE(n == 0 || (src && dst), LPS_EINVAL, "lps_copy_f32: null pointer");
  LPS_REQUIRE(n == 0 || ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0,
              LPS_EINVAL, "lps_copy_f32: src and dst must be 16-byte aligned");
  return launch_copy_f32(src, dst, n, as_stream(stream));
}

extern "C" int lps_f32_to_f16(const float* src, uint16_t* dst, int64_t n, void* stream) {
  LPS_REQUIRE(n >= 0, LPS_EINVAL, "lps_f32_to_f16: n %lld < 0", (long long)n);
  if (n == 0) return LPS_OK;
  LPS_REQUIRE(src && dst, LPS_EINVAL, "lps_f32_to_f16: null pointer");
  hipLaunchKernelGGL(k_f32_to_f16, grid_for(n), dim3(256), 0, as_stream(stream), src, dst, (long long)n);
  LPS_HIP(hipGetLastError());
  return LPS_OK;
}

// strata PR #3648, Approach (sums; the combine kernel; piece bounds): the FP16
// sums are widened into bo one piece at a time on the remote stream, an event
// after each piece; the main stream waits the last event and then combines.
extern "C" int lps_moe_combine(float* out, const float* x, const float* shared,
                               const float* local, const uint16_t* remote16, float* bo, int32_t T,
                               int32_t d, int32_t n_pieces, void* s_remote, void* s_main) {
  LPS_REQUIRE(T >= 0 && d > 0, LPS_EINVAL, "lps_moe_combine: T %d / d %d", T, d);
  LPS_REQUIRE(n_pieces >= 1 && n_pieces <= 64, LPS_EINVAL,
              "lps_moe_combine: n_pieces %d outside [1, 64]", n_pieces);
  if (T == 0) return LPS_OK;
  LPS_REQUIRE(out && x && shared && local && remote16 && bo, LPS_EINVAL,
              "lps_moe_combine: null pointer");
  LPS_REQUIRE(bo != local && bo != shared && (const void*)bo != (const void*)remote16, LPS_EINVAL,
              "lps_moe_combine: bo must not be shared, local or remote16 (they are read after bo is written)");
  hipStream_t sr = as_stream(s_remote), sm = as_stream(s_main);
  hipEvent_t start, done;
  // device-side ordering between the two streams only: no system-scope fence
  LPS_HIP(hipEventCreateWithFlags(&start, hipEventDisableTiming | hipEventDisableSystemFence));
  LPS_HIP(hipEventCreateWithFlags(&done, hipEventDisableTiming | hipEventDisableSystemFence));
  // the remote stream may only overwrite bo once the main stream's earlier work
  // (which may still read bo or local) is done
  LPS_HIP(hipEventRecord(start, sm));
  LPS_HIP(hipStreamWaitEvent(sr, start, 0));
  int pieces = 0;
  for (int pc = 0; pc < n_pieces; ++pc) {
    const long long lo = (long long)pc * T / n_pieces, hi = (long long)(pc + 1) * T / n_pieces;
    if (hi > lo) {
      const long long a = lo * d, b = hi * d;
      if (a % 8 == 0 && b % 8 == 0 && ((reinterpret_cast<uintptr_t>(remote16) | reinterpret_cast<uintptr_t>(bo)) & 15) == 0)
        hipLaunchKernelGGL(k_f16_to_f32_8, grid_for((b - a) / 8), dim3(256), 0, sr, remote16, bo, a, b);
      else
        hipLaunchKernelGGL(k_f16_to_f32, grid_for(b - a), dim3(256), 0, sr, remote16, bo, a, b);
      LPS_HIP(hipGetLastError());
      ++pieces;
    }
  }
  LPS_HIP(hipEventRecord(done, sr));
  LPS_HIP(hipStreamWaitEvent(sm, done, 0));
  const long long n = (long long)T * d;
  const auto a16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  if (n % 4 == 0 && a16(out) && a16(x) && a16(shared) && a16(local) && a16(bo))
    hipLaunchKernelGGL(k_combine4, grid_for(n / 4), dim3(256), 0, sm, out, x, shared, local, bo, n / 4);
  else
    hipLaunchKernelGGL(k_combine, grid_for(n), dim3(256), 0, sm, out, x, shared, local, bo, n);
  LPS_HIP(hipGetLastError());
  // events are released once they have fired (the runtime keeps them alive)
  LPS_HIP(hipEventDestroy(start));
  LPS_HIP(hipEventDestroy(done));
  count_pieces(pieces);
  return LPS_OK;
}
