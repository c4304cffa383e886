// Internal declarations shared by the liblps translation units (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/lps.h"

namespace lps {

// ---- errors -----------------------------------------------------------------
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

#define LPS_HIP(call)                                                                  \
  do {                                                                                 \
    hipError_t e_ = (call);                                                            \
    if (e_ != hipSuccess)                                                              \
      return ::lps::fail(LPS_EHIP, "%s: %s failed: %s", __func__, #call,               \
                         hipGetErrorString(e_));                                       \
  } while (0)

#define LPS_REQUIRE(cond, code, ...)                                                   \
  do {                                                                                 \
    if (!(cond)) return ::lps::fail((code), __VA_ARGS__);                              \
  } while (0)

// ---- counters -----------------------------------------------------------------
void count_stage_walk();
void count_send();
void count_recv();
void count_pieces(int64_t n);
void count_drain();

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Kernels whose dynamic LDS exceeds the default 64 KiB window must opt in once
// per function (gfx950 has 160 KiB per workgroup).  Returns a status.
int ensure_lds(const void* fn, size_t bytes);

// Benchmark timer: a pair of events the next launch of `kind` hands to
// hipExtLaunchKernelGGL, which stamps them with that dispatch's own start and
// end (nulls when no timer runs for this kind).
struct Stamp {
  hipEvent_t start = nullptr, stop = nullptr;
};
Stamp timer_take(int kind);

// A launch that stamps a timer's events when it carries any, and is a plain
// launch otherwise (the form a stream capture records).
#define LPS_LAUNCH(K, GRID, BLOCK, LDS, ST, E0, E1, ...)                        \
  do {                                                                          \
    if ((E0) != nullptr || (E1) != nullptr)                                     \
      hipExtLaunchKernelGGL(K, GRID, BLOCK, LDS, ST, E0, E1, 0, __VA_ARGS__);   \
    else                                                                        \
      hipLaunchKernelGGL(K, GRID, BLOCK, LDS, ST, __VA_ARGS__);                 \
  } while (0)

// ---- scratch carving ------------------------------------------------------------
inline size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// ---- launchers (each validates nothing; callers validate first) -------------------
struct QkvArgs {
  const lps_layer_desc* L;
  const float* x;
  int pos;
  float* q;
  const int32_t* pos_dev = nullptr;   // if set: the position is read here (RoPE from L->rope_cs)
};
// mode EPI_ADD with tee0 and tee1: every updated row of y is also stored to both
int launch_gemv(int wdtype, const void* w, const uint8_t* s, int N, int K, const float* x,
                const float* g, float eps, float* y, int mode, hipStream_t st, Stamp sp = {},
                float* tee0 = nullptr, float* tee1 = nullptr);
int launch_qkv(const QkvArgs& a, hipStream_t st, Stamp sp = {});
// cs[0], cs[1] = f32 cos, sin of pos * base^(-2i / hd) (the QKV launch's own values)
void rope_cos_sin(float base, int hd, int pos, int i, float* cs);
// MoE decode gate/up + SwiGLU over the k selected experts (eidx, device) and the
// shared one: y[(j, i)] = silu(gate) * up for slot j <= k, row i < ff
int launch_moe_gu(const void* w_e, const void* w_s, const int32_t* eidx, int E, int kslots, int ff,
                  int d, const float* x, const float* g, float eps, float* y, hipStream_t st, Stamp sp = {});
// MoE decode down projections: z[j * d + r] = W_j[r, :] . m[j, :] for slot j <= k
// (k selected experts by eidx, then the shared one); d even
int launch_moe_down(const void* w_e, const void* w_s, const int32_t* eidx, int E, int kslots,
                    int d, int ff, const float* m, float* z, hipStream_t st, Stamp sp = {});
int launch_head(const lps_head_desc* h, const float* x, float* logits, int32_t* tok,
                void* scratch, size_t bytes, hipStream_t st, Stamp sp = {});
size_t head_scratch(const lps_head_desc* h);

size_t attn_scratch(int nq, int nkv, int hd, int ctx_max);
// pos_dev set: the rows are 0 .. *pos_dev (read on the device), n_rows ignored
int launch_attention(int nq, int nkv, int hd, int kvdtype, const void* kc, const void* vc,
                     int ctx_max, int n_rows, const float* q, float* o, void* scratch,
                     hipStream_t st, Stamp sp = {}, const int32_t* pos_dev = nullptr);

int launch_row_at_step(const int32_t* state, const float* src, int64_t src_stride, float* dst,
                       int64_t dst_stride, int32_t n, int32_t n_rows, hipStream_t st);
int launch_copy2_f32(const float* src, float* dst0, float* dst1, int64_t n, hipStream_t st);
int launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t st);
// decode step state (pos, step, flags): see lps_step_advance
int launch_step_advance_hist(const int32_t* state, const float* logits, int32_t vocab,
                             float* logits_hist, int32_t hist_cap, float* ring_logits,
                             int32_t ring_slots, hipStream_t st);
// ring_logits / ring_tok: device addresses of a host ring of ring_slots rows (or NULL)
int launch_step_finish(const lps_head_desc* h, const float* x, float* logits, int32_t* state,
                       int32_t pos_limit, const int32_t* feed, int32_t n_feed, int32_t* tok_hist,
                       float* logits_hist, int32_t hist_cap, const void* embed, int32_t embed_dtype,
                       float* x_next, int32_t* tok_cur, float* ring_logits, int32_t* ring_tok,
                       int32_t ring_slots, void* scratch, hipStream_t st, Stamp sp = {});
int launch_step_advance(int32_t* state, int32_t pos_limit, const int32_t* argmax, int32_t* tok_cur,
                        const int32_t* feed, int32_t n_feed, int32_t* tok_hist, int32_t hist_cap,
                        const float* logits, int32_t vocab, float* logits_hist, hipStream_t st);

// ---- chunked dense prefill (prefill.hip) ---------------------------------------------
// scratch of one layer over T rows: bf16 rows [T, max(d, nq hd)] | qkv f32 | SwiGLU bf16
struct PrefillScratch {
  size_t xb, qkv, mb, total;
};
PrefillScratch prefill_scratch(const lps_layer_desc* L, int T);
int check_prefill_layer(const lps_layer_desc* L, int T, int p0, const char* who);
// one layer over the T rows of x [T, d] f32 (in place) at positions p0 .. p0 + T - 1
int prefill_layer(const lps_layer_desc* L, float* x, int T, int p0, void* scratch, hipStream_t st);
int launch_embed_rows(const void* table, int wdtype, int vocab, int d, const int32_t* tok, int T,
                      float* x, hipStream_t st);
void count_prefill_walk();
void count_act_pieces(int64_t n);

// validation helpers shared by entry points
int check_layer(const lps_layer_desc* L, const char* who);
// MoE FFN decode of one token (moe.hip): validation, scratch bytes, the launches
int check_moe_decode(const lps_moe_desc* m, const char* who);
size_t moe_decode_scratch(const lps_moe_desc* m);
// tee0 and tee1 (or NULL): the updated residual row is also stored to both
int moe_decode(const lps_moe_desc* m, float* x, void* scratch, hipStream_t st,
               float* tee0 = nullptr, float* tee1 = nullptr);

}  // namespace lps
