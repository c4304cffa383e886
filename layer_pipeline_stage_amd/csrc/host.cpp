// Host side of liblps: status text, the stage plan, liveness counters, boundary
// slots, deferred logits readback, the model handle and the layer / stage walks.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <cstdarg>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "internal.h"

namespace lps {

static thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}
void clear_error() { g_err[0] = 0; }

static std::atomic<long long> c_walks{0}, c_sends{0}, c_recvs{0}, c_pieces{0}, c_drains{0},
    c_prefill{0}, c_act_pieces{0};
void count_prefill_walk() { c_prefill.fetch_add(1, std::memory_order_relaxed); }
void count_act_pieces(int64_t n) { c_act_pieces.fetch_add(n, std::memory_order_relaxed); }
void count_stage_walk() { c_walks.fetch_add(1, std::memory_order_relaxed); }
void count_send() { c_sends.fetch_add(1, std::memory_order_relaxed); }
void count_recv() { c_recvs.fetch_add(1, std::memory_order_relaxed); }
void count_pieces(int64_t n) { c_pieces.fetch_add(n, std::memory_order_relaxed); }
void count_drain() { c_drains.fetch_add(1, std::memory_order_relaxed); }

int ensure_lds(const void* fn, size_t bytes) {
  if (bytes <= 65536) return LPS_OK;
  static std::mutex mu;
  static std::vector<std::pair<const void*, size_t>> done;
  std::lock_guard<std::mutex> lk(mu);
  for (auto& e : done)
    if (e.first == fn && e.second >= bytes) return LPS_OK;
  hipError_t err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
  if (err != hipSuccess) {
    (void)hipGetLastError();
    return fail(LPS_EUNSUP, "ensure_lds: %zu bytes of LDS refused: %s", bytes, hipGetErrorString(err));
  }
  done.emplace_back(fn, bytes);
  return LPS_OK;
}

// ---- benchmark timer ---------------------------------------------------------------
struct Timer {
  std::mutex mu;
  std::atomic<int> kind{0};
  std::vector<hipEvent_t> ev;   // 2 per launch
  int used = 0;
};
static Timer g_timer;

Stamp timer_take(int kind) {
  if (g_timer.kind.load(std::memory_order_relaxed) != kind) return {};
  std::lock_guard<std::mutex> lk(g_timer.mu);
  if (g_timer.kind.load() != kind || g_timer.used * 2 >= int(g_timer.ev.size())) return {};
  const int i = g_timer.used++;
  return Stamp{g_timer.ev[2 * i], g_timer.ev[2 * i + 1]};
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Id of the stream capture `st` takes part in, 0 when it is not capturing.
static int capture_of(hipStream_t st, unsigned long long* id) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  unsigned long long cid = 0;
  LPS_HIP(hipStreamGetCaptureInfo(st, &cs, &cid));
  LPS_REQUIRE(cs != hipStreamCaptureStatusInvalidated, LPS_ESTATE,
              "stream capture was invalidated by an earlier call");
  *id = cs == hipStreamCaptureStatusActive ? cid : 0;
  return LPS_OK;
}

static int chunk_of(int wdtype) { return wdtype == LPS_F32 ? 4 : wdtype == LPS_BF16 ? 8 : 32; }

// q heads per kv head that the attention kernel is instantiated for
static bool gqa_built(int g) { return g == 1 || g == 2 || g == 4 || g == 6 || g == 8; }

int check_layer(const lps_layer_desc* L, const char* who) {
  LPS_REQUIRE(L, LPS_EINVAL, "%s: null layer descriptor", who);
  LPS_REQUIRE(L->ffn_kind == LPS_FFN_DENSE || L->ffn_kind == LPS_FFN_MOE, LPS_EINVAL,
              "%s: ffn_kind %d", who, L->ffn_kind);
  LPS_REQUIRE(L->d > 0 && L->nq >= 0, LPS_EINVAL, "%s: d %d must be > 0 and nq %d >= 0", who, L->d,
              L->nq);
  LPS_REQUIRE(L->wdtype == LPS_F32 || L->wdtype == LPS_BF16 || L->wdtype == LPS_MXFP4, LPS_EINVAL,
              "%s: wdtype %d", who, L->wdtype);
  const int ch = chunk_of(L->wdtype);
  LPS_REQUIRE(L->d * 4 <= 160 * 1024, LPS_EUNSUP, "%s: d %d exceeds 160 KiB of LDS", who, L->d);
  if (L->nq > 0) {   // the attention sublayer
    LPS_REQUIRE(L->nkv > 0 && L->hd > 0, LPS_EINVAL, "%s: nkv %d and hd %d must be > 0", who,
                L->nkv, L->hd);
    LPS_REQUIRE(L->nq % L->nkv == 0 && gqa_built(L->nq / L->nkv), LPS_EUNSUP,
                "%s: nq / nkv = %d/%d: 1, 2, 4, 6 or 8 q heads per kv head are built", who, L->nq,
                L->nkv);
    LPS_REQUIRE(L->hd == 64 || L->hd == 128 || L->hd == 256, LPS_EUNSUP,  // RoPE table: hd/2 <= 128
                "%s: head dim %d not built (64, 128, 256)", who, L->hd);
    LPS_REQUIRE(L->kvdtype == LPS_F32 || L->kvdtype == LPS_BF16, LPS_EINVAL, "%s: kvdtype %d", who,
                L->kvdtype);
    LPS_REQUIRE(L->d % ch == 0 && (L->nq * L->hd) % ch == 0, LPS_EINVAL,
                "%s: d %d and nq*hd %d must be multiples of %d for this weight dtype", who, L->d,
                L->nq * L->hd, ch);
    LPS_REQUIRE(L->ctx_max > 0, LPS_EINVAL, "%s: ctx_max %d", who, L->ctx_max);
    if (L->kvdtype == LPS_BF16)   // whole 16-row V tiles; 32-bit byte offsets per head
      LPS_REQUIRE(L->ctx_max % 16 == 0 && L->ctx_max <= (1 << 22), LPS_EINVAL,
                  "%s: bf16 caches need ctx_max %d to be a multiple of 16 and at most 4194304", who,
                  L->ctx_max);
    LPS_REQUIRE(L->nq * L->hd * 4 <= 160 * 1024, LPS_EUNSUP,
                "%s: the attention output exceeds 160 KiB of LDS", who);
    LPS_REQUIRE(L->g_attn && L->w_qkv && L->w_o && L->k_cache && L->v_cache, LPS_EINVAL,
                "%s: null attention weight / gain / cache pointer", who);
    LPS_REQUIRE(aligned16(L->w_qkv) && aligned16(L->w_o) && aligned16(L->g_attn) &&
                    aligned16(L->k_cache) && aligned16(L->v_cache),
                LPS_EINVAL, "%s: weights, gains and caches must be 16-byte aligned", who);
    if (L->wdtype == LPS_MXFP4)
      LPS_REQUIRE(L->s_qkv && L->s_o, LPS_EINVAL, "%s: MXFP4 weights need their e8m0 scale arrays",
                  who);
  }
  if (L->ffn_kind == LPS_FFN_MOE) {   // the MoE FFN carries its own norm gain and weights
    LPS_REQUIRE(L->moe, LPS_EINVAL, "%s: ffn_kind MoE with a null moe descriptor", who);
    LPS_REQUIRE(L->moe->d == L->d, LPS_EINVAL, "%s: moe->d %d differs from d %d", who, L->moe->d,
                L->d);
    return check_moe_decode(L->moe, who);
  }
  LPS_REQUIRE(L->ff > 0 && L->d % ch == 0 && L->ff % ch == 0, LPS_EINVAL,
              "%s: d %d and ff %d must be positive multiples of %d for this weight dtype", who, L->d,
              L->ff, ch);
  LPS_REQUIRE(L->ff * 4 <= 160 * 1024, LPS_EUNSUP, "%s: ff %d exceeds 160 KiB of LDS", who, L->ff);
  LPS_REQUIRE(L->g_ffn && L->w_gu && L->w_d, LPS_EINVAL, "%s: null FFN weight / gain pointer", who);
  LPS_REQUIRE(aligned16(L->w_gu) && aligned16(L->w_d) && aligned16(L->g_ffn), LPS_EINVAL,
              "%s: weights and gains must be 16-byte aligned", who);
  if (L->wdtype == LPS_MXFP4)
    LPS_REQUIRE(L->s_gu && L->s_d, LPS_EINVAL, "%s: MXFP4 weights need their e8m0 scale arrays", who);
  return LPS_OK;
}

// scratch layout of one layer: q | o | attention partials (attention sublayer) and
// m (dense FFN) or the MoE FFN's scratch, each region after the previous one
struct LayerScratch {
  size_t q, o, attn, m, total;
};
static LayerScratch layer_scratch(const lps_layer_desc* L) {
  LayerScratch s{};
  size_t off = 0;
  if (L->nq > 0) {
    s.q = off;
    s.o = off += align256(size_t(L->nq) * L->hd * 4);
    s.attn = off += align256(size_t(L->nq) * L->hd * 4);
    off += align256(attn_scratch(L->nq, L->nkv, L->hd, L->ctx_max));
  }
  s.m = off;
  s.total = off + (L->ffn_kind == LPS_FFN_MOE ? moe_decode_scratch(L->moe)
                                               : align256(size_t(L->ff) * 4));
  return s;
}

// pos_dev set: the position is read on the device (pos unused).  tee0 / tee1 set: the
// layer's last launch also stores the updated residual row to both.
static int layer_forward(const lps_layer_desc* L, float* x, int pos, void* scratch, hipStream_t st,
                         const int32_t* pos_dev = nullptr, float* tee0 = nullptr,
                         float* tee1 = nullptr) {
  const LayerScratch s = layer_scratch(L);
  char* sc = static_cast<char*>(scratch);
  float* m = reinterpret_cast<float*>(sc + s.m);
  int rc;
  if (L->nq > 0) {
    float* q = reinterpret_cast<float*>(sc + s.q);
    float* o = reinterpret_cast<float*>(sc + s.o);
    void* at = sc + s.attn;
    QkvArgs qa{L, x, pos, q, pos_dev};
    rc = launch_qkv(qa, st, timer_take(LPS_KIND_QKV));
    if (rc) return rc;
    rc = launch_attention(L->nq, L->nkv, L->hd, L->kvdtype, L->k_cache, L->v_cache, L->ctx_max,
                          pos + 1, q, o, at, st, timer_take(LPS_KIND_ATTN), pos_dev);
    if (rc) return rc;
    rc = launch_gemv(L->wdtype, L->w_o, L->s_o, L->d, L->nq * L->hd, o, nullptr, 0.f, x,
                     LPS_EPI_ADD, st, timer_take(LPS_KIND_OPROJ));
    if (rc) return rc;
  }
  if (L->ffn_kind == LPS_FFN_MOE) return moe_decode(L->moe, x, m, st, tee0, tee1);
  rc = launch_gemv(L->wdtype, L->w_gu, L->s_gu, 2 * L->ff, L->d, x, L->g_ffn, L->eps, m,
                   LPS_EPI_SWIGLU, st, timer_take(LPS_KIND_GATEUP));
  if (rc) return rc;
  return launch_gemv(L->wdtype, L->w_d, L->s_d, L->d, L->ff, m, nullptr, 0.f, x, LPS_EPI_ADD, st,
                     timer_take(LPS_KIND_DOWN), tee0, tee1);
}

static int check_fence(const int32_t* fence, int32_t n_stages, int32_t n_layers, const char* who) {
  LPS_REQUIRE(fence, LPS_EINVAL, "%s: null fence", who);
  LPS_REQUIRE(n_stages >= 1, LPS_EINVAL, "%s: n_stages %d < 1", who, n_stages);
  LPS_REQUIRE(fence[0] == 0, LPS_EINVAL, "%s: fence[0] = %d, must be 0", who, fence[0]);
  if (n_layers >= 0)
    LPS_REQUIRE(fence[n_stages] == n_layers, LPS_EINVAL, "%s: fence[%d] = %d, must be n_layers %d",
                who, n_stages, fence[n_stages], n_layers);
  for (int s = 0; s < n_stages; ++s)
    LPS_REQUIRE(fence[s + 1] > fence[s], LPS_EINVAL,
                "%s: fence not strictly increasing at stage %d (%d -> %d)", who, s, fence[s],
                fence[s + 1]);
  return LPS_OK;
}

}  // namespace lps

struct lps_model {
  std::vector<lps_layer_desc> layers;
  std::vector<lps_moe_desc> moes;   // copies the MoE layers' descriptors point at
  size_t scratch = 0;
};

struct lps_boundary {
  int32_t n;
  float* slot[2];
  hipEvent_t ev_tx[2];
  hipEvent_t ev_rx[2];
  bool tx_recorded[2];
  bool rx_recorded[2];
  hipStream_t tx_stream[2];   // stream of the slot's last send
  hipStream_t rx_stream[2];   // stream of the slot's last receive
  // capture that made the event's last record (0: an eager record); a wait
  // only ever targets a record made in the waiting stream's own context
  unsigned long long tx_cap[2];   // context of the slot's last send
  unsigned long long rx_cap[2];
  int64_t next_send;
  int64_t next_recv;
};

struct lps_graph {
  hipGraphExec_t exec;
};

// A pending readback is a token, not an address: (generation << 32) | (slot + 1)
// into a table of slots.  A wait or a drop frees the slot and bumps its
// generation, so a second wait or drop on the same token (or one on a token
// that was never issued) is refused instead of touching freed state.
namespace lps {
struct PendingSlot {
  hipEvent_t drained = nullptr;
  uint32_t gen = 1;
  bool live = false;
};
static std::mutex g_pend_mu;
static std::vector<PendingSlot> g_pend;
static std::vector<uint32_t> g_pend_free;

static lps_pending* pending_token(uint32_t slot, uint32_t gen) {
  return reinterpret_cast<lps_pending*>((uintptr_t(gen) << 32) | uintptr_t(slot + 1));
}
// Takes the live slot a token names (marking it finished) and returns its event;
// nullptr when the token is not a live pending.
static hipEvent_t pending_take(lps_pending* p) {
  const uintptr_t v = reinterpret_cast<uintptr_t>(p);
  const uint32_t slot = uint32_t(v & 0xffffffffu) - 1u, gen = uint32_t(v >> 32);
  std::lock_guard<std::mutex> lk(g_pend_mu);
  if (slot >= g_pend.size() || !g_pend[slot].live || g_pend[slot].gen != gen) return nullptr;
  PendingSlot& e = g_pend[slot];
  hipEvent_t ev = e.drained;
  e.drained = nullptr;
  e.live = false;
  e.gen = e.gen == 0xffffffffu ? 1u : e.gen + 1u;
  g_pend_free.push_back(slot);
  return ev;
}
// The device address of pinned host memory (false for device memory, pageable
// host memory or an address the runtime does not know).
static bool pinned_host_on_device(void* p, void** dptr) {
  hipPointerAttribute_t a{};
  if (hipPointerGetAttributes(&a, p) != hipSuccess || a.type != hipMemoryTypeHost) {
    (void)hipGetLastError();
    return false;
  }
  if (hipHostGetDevicePointer(dptr, p, 0) != hipSuccess || *dptr == nullptr) {
    (void)hipGetLastError();
    return false;
  }
  return true;
}
// The checks and the wait of a same-stream hop of `step` across b, before anything
// writes the slot: the step is the next send and the next receive, and a slot whose
// last receive ran on another stream of the same capture context is waited for.
static int hop_begin(lps_boundary* b, int64_t step, hipStream_t st, unsigned long long* cid,
                     const char* who) {
  LPS_REQUIRE(step == b->next_send && step == b->next_recv, LPS_ESTATE,
              "%s: step %lld out of order (next send %lld, next receive %lld)", who,
              (long long)step, (long long)b->next_send, (long long)b->next_recv);
  const int k = int(step & 1);
  int rc = capture_of(st, cid);
  if (rc) return rc;
  if (b->rx_stream[k] && b->rx_stream[k] != st && b->rx_cap[k] == *cid) {
    if (!b->rx_recorded[k]) {
      unsigned long long rcid = 0;
      rc = capture_of(b->rx_stream[k], &rcid);
      if (rc) return rc;
      LPS_REQUIRE(rcid == *cid, LPS_ESTATE,
                  "%s: slot %d's last receive stream is in another capture context", who, k);
      LPS_HIP(hipEventRecord(b->ev_rx[k], b->rx_stream[k]));
      b->rx_recorded[k] = true;
    }
    LPS_HIP(hipStreamWaitEvent(st, b->ev_rx[k], 0));
  }
  return LPS_OK;
}
// The books of a same-stream hop whose row is in the slot: the slot was sent and
// received on st, in capture context cid.
static void hop_end(lps_boundary* b, int64_t step, hipStream_t st, unsigned long long cid) {
  const int k = int(step & 1);
  b->tx_recorded[k] = false;
  b->tx_stream[k] = b->rx_stream[k] = st;
  b->tx_cap[k] = b->rx_cap[k] = cid;
  b->rx_recorded[k] = false;
  b->next_send = b->next_recv = step + 1;
  count_send();
  count_recv();
}
// Registers an event as a live pending and hands out its token; on failure the
// event is destroyed.
static int pending_issue(hipEvent_t ev, lps_pending** out, const char* who) {
  std::lock_guard<std::mutex> lk(g_pend_mu);
  uint32_t slot;
  if (!g_pend_free.empty()) {
    slot = g_pend_free.back();
    g_pend_free.pop_back();
  } else {
    if (g_pend.size() >= 0xfffffffeu) {
      (void)hipEventDestroy(ev);
      return fail(LPS_ENOMEM, "%s: too many pending readbacks", who);
    }
    slot = uint32_t(g_pend.size());
    g_pend.emplace_back();
  }
  g_pend[slot].drained = ev;
  g_pend[slot].live = true;
  *out = pending_token(slot, g_pend[slot].gen);
  return LPS_OK;
}
}  // namespace lps

using namespace lps;

extern "C" {

const char* lps_last_error(void) { return g_err; }
const char* lps_version(void) { return "liblps 0.1 (gfx950)"; }

// ---- A1 ------------------------------------------------------------------------
int lps_stage_plan(int32_t n_layers, int32_t n_stages, const int32_t* cuts, int32_t n_cuts,
                   int32_t* fence_out) {
  LPS_REQUIRE(fence_out, LPS_EINVAL, "lps_stage_plan: null fence_out");
  LPS_REQUIRE(n_layers >= 1, LPS_EINVAL, "lps_stage_plan: n_layers %d < 1", n_layers);
  LPS_REQUIRE(n_stages >= 1 && n_stages <= n_layers, LPS_EINVAL,
              "lps_stage_plan: n_stages %d outside [1, n_layers=%d]", n_stages, n_layers);
  std::vector<int32_t> c;
  if (cuts == nullptr && n_cuts == 0) {
    for (int s = 1; s < n_stages; ++s) c.push_back(int32_t((int64_t)s * n_layers / n_stages));
  } else {
    LPS_REQUIRE(cuts, LPS_EINVAL, "lps_stage_plan: n_cuts %d with a null cuts array", n_cuts);
    LPS_REQUIRE(n_cuts == n_stages - 1, LPS_EINVAL,
                "lps_stage_plan: %d cuts given, n_stages %d needs %d", n_cuts, n_stages,
                n_stages - 1);
    c.assign(cuts, cuts + n_cuts);
  }
  int32_t prev = 0;
  for (size_t i = 0; i < c.size(); ++i) {
    LPS_REQUIRE(c[i] > 0 && c[i] < n_layers && c[i] > prev, LPS_EINVAL,
                "lps_stage_plan: cut %zu = %d must be strictly increasing inside (0, %d)", i, c[i],
                n_layers);
    prev = c[i];
  }
  fence_out[0] = 0;
  for (size_t i = 0; i < c.size(); ++i) fence_out[i + 1] = c[i];
  fence_out[n_stages] = n_layers;
  clear_error();
  return LPS_OK;
}

int lps_stage_plan_counts(int32_t n_layers, int32_t n_stages, const int32_t* counts,
                          int32_t* fence_out) {
  LPS_REQUIRE(counts && fence_out, LPS_EINVAL, "lps_stage_plan_counts: null pointer");
  LPS_REQUIRE(n_stages >= 1, LPS_EINVAL, "lps_stage_plan_counts: n_stages %d < 1", n_stages);
  std::vector<int32_t> cuts;
  int64_t acc = 0;
  for (int s = 0; s < n_stages; ++s) {
    LPS_REQUIRE(counts[s] >= 1, LPS_EINVAL, "lps_stage_plan_counts: counts[%d] = %d < 1", s,
                counts[s]);
    acc += counts[s];
    if (s < n_stages - 1) cuts.push_back(int32_t(acc));
  }
  LPS_REQUIRE(acc == n_layers, LPS_EINVAL, "lps_stage_plan_counts: counts sum to %lld, not %d",
              (long long)acc, n_layers);
  return lps_stage_plan(n_layers, n_stages, cuts.empty() ? nullptr : cuts.data(),
                        int32_t(cuts.size()), fence_out);
}

int lps_stage_of(const int32_t* fence, int32_t n_stages, int32_t layer) {
  int rc = check_fence(fence, n_stages, -1, "lps_stage_of");
  if (rc) return rc;
  LPS_REQUIRE(layer >= 0 && layer < fence[n_stages], LPS_ERANGE,
              "lps_stage_of: layer %d outside [0, %d)", layer, fence[n_stages]);
  for (int s = 0; s < n_stages; ++s)
    if (layer < fence[s + 1]) return s;
  return fail(LPS_ERANGE, "lps_stage_of: unreachable");
}

// ---- memory-balancing split (ninfer "Multi-GPU: layer pipeline stages", How it works:
// the most page groups every stage can hold, then the least-full stage) -------------
// Exact dynamic programs over contiguous splits, backward so that the forward
// reconstruction can take, stage by stage, the smallest cut that still completes
// an optimal split (the lexicographically smallest optimal fence):
//  1. P = max over splits of min over stages of the groups a stage can hold;
//  2. among splits where every stage holds P groups, minimise the largest fill
//     (overhead + fixed + P * kv) / free, compared exactly as fractions.
int lps_stage_solve(int32_t n_layers, int32_t n_stages, const int64_t* stage_free,
                    const int64_t* stage_overhead, const int64_t* layer_fixed,
                    const int64_t* layer_kv, int64_t max_groups, int32_t* fence_out,
                    int64_t* groups_out) {
  LPS_REQUIRE(n_layers >= 1 && n_layers <= 4096, LPS_EINVAL, "lps_stage_solve: n_layers %d", n_layers);
  LPS_REQUIRE(n_stages >= 1 && n_stages <= n_layers, LPS_EINVAL,
              "lps_stage_solve: n_stages %d outside [1, n_layers %d]", n_stages, n_layers);
  LPS_REQUIRE(stage_free && stage_overhead && layer_fixed && layer_kv && fence_out && groups_out,
              LPS_EINVAL, "lps_stage_solve: null pointer");
  LPS_REQUIRE(max_groups >= 0 && max_groups <= (int64_t(1) << 40), LPS_EINVAL,
              "lps_stage_solve: max_groups %lld outside [0, 2^40]", (long long)max_groups);
  const int L = n_layers, N = n_stages;
  for (int s = 0; s < N; ++s)
    LPS_REQUIRE(stage_free[s] > 0 && stage_free[s] <= (int64_t(1) << 50) && stage_overhead[s] >= 0 &&
                    stage_overhead[s] <= (int64_t(1) << 50),
                LPS_EINVAL, "lps_stage_solve: stage %d free %lld / overhead %lld", s,
                (long long)stage_free[s], (long long)stage_overhead[s]);
  for (int l = 0; l < L; ++l)
    LPS_REQUIRE(layer_fixed[l] >= 0 && layer_fixed[l] <= (int64_t(1) << 40) && layer_kv[l] >= 0 &&
                    layer_kv[l] <= (int64_t(1) << 40),
                LPS_EINVAL, "lps_stage_solve: layer %d fixed %lld / kv %lld", l,
                (long long)layer_fixed[l], (long long)layer_kv[l]);
  std::vector<int64_t> pf(L + 1, 0), pk(L + 1, 0);   // prefix sums (< 2^52)
  for (int l = 0; l < L; ++l) {
    pf[l + 1] = pf[l] + layer_fixed[l];
    pk[l + 1] = pk[l] + layer_kv[l];
  }
  auto groups = [&](int s, int a, int b) -> int64_t {   // page groups stage s holds for [a, b)
    const int64_t need = stage_overhead[s] + pf[b] - pf[a];
    if (need > stage_free[s]) return -1;
    const int64_t per = pk[b] - pk[a];
    if (per == 0) return max_groups;
    const int64_t g = (stage_free[s] - need) / per;
    return g < max_groups ? g : max_groups;
  };
  const int64_t NEG = -2;
  // best1[s][a]: max over splits of [a, L) into stages s..N-1 of the min groups
  std::vector<int64_t> best1(size_t(N + 1) * (L + 1), NEG);
  auto B1 = [&](int s, int a) -> int64_t& { return best1[size_t(s) * (L + 1) + a]; };
  B1(N, L) = max_groups;
  for (int s = N - 1; s >= 0; --s)
    for (int a = s; a <= L - (N - s); ++a) {
      int64_t best = NEG;
      for (int b = a + 1; b <= L - (N - s - 1); ++b) {
        const int64_t rest = B1(s + 1, b);
        if (rest == NEG) continue;
        const int64_t g = groups(s, a, b);
        const int64_t v = g < rest ? g : rest;
        if (v > best) best = v;
      }
      B1(s, a) = best;
    }
  const int64_t P = B1(0, 0);
  LPS_REQUIRE(P >= 0, LPS_EUNSUP, "lps_stage_solve: no split of %d layers over %d stages fits", L, N);
  // fill of stage s over [a, b) at P groups as a fraction num / den (den = free > 0)
  struct Frac { __int128 num, den; };
  auto less = [](const Frac& x, const Frac& y) { return x.num * y.den < y.num * x.den; };
  auto fill = [&](int s, int a, int b) {
    return Frac{__int128(stage_overhead[s] + pf[b] - pf[a]) + __int128(P) * (pk[b] - pk[a]),
                __int128(stage_free[s])};
  };
  // best2[s][a]: min over P-feasible splits of [a, L) of the largest fill (den 0: none)
  std::vector<Frac> best2(size_t(N + 1) * (L + 1), Frac{0, 0});
  auto B2 = [&](int s, int a) -> Frac& { return best2[size_t(s) * (L + 1) + a]; };
  B2(N, L) = Frac{0, 1};
  for (int s = N - 1; s >= 0; --s)
    for (int a = s; a <= L - (N - s); ++a) {
      Frac best{0, 0};
      for (int b = a + 1; b <= L - (N - s - 1); ++b) {
        const Frac rest = B2(s + 1, b);
        if (rest.den == 0 || groups(s, a, b) < P) continue;
        const Frac f = fill(s, a, b);
        const Frac v = less(f, rest) ? rest : f;
        if (best.den == 0 || less(v, best)) best = v;
      }
      B2(s, a) = best;
    }
  // forward: the smallest cut whose stage stays within the optimum F and whose
  // remainder can (the lexicographically smallest of the optimal fences)
  const Frac F = B2(0, 0);
  fence_out[0] = 0;
  int a = 0;
  for (int s = 0; s < N; ++s) {
    int pick = -1;
    for (int b = a + 1; b <= L - (N - s - 1); ++b) {
      const Frac rest = B2(s + 1, b);
      if (rest.den == 0 || groups(s, a, b) < P) continue;
      if (!less(F, fill(s, a, b)) && !less(F, rest)) { pick = b; break; }
    }
    LPS_REQUIRE(pick > 0, LPS_ESTATE, "lps_stage_solve: reconstruction failed at stage %d", s);
    fence_out[s + 1] = pick;
    a = pick;
  }
  *groups_out = P;
  return LPS_OK;
}

// ---- counters ---------------------------------------------------------------------
int lps_counters(lps_counters_t* out) {
  LPS_REQUIRE(out, LPS_EINVAL, "lps_counters: null out");
  out->stage_walks = c_walks.load();
  out->boundary_sends = c_sends.load();
  out->boundary_recvs = c_recvs.load();
  out->pieces = c_pieces.load();
  out->drains = c_drains.load();
  out->prefill_walks = c_prefill.load();
  out->act_pieces = c_act_pieces.load();
  return LPS_OK;
}
int lps_counters_reset(void) {
  c_walks = 0;
  c_sends = 0;
  c_recvs = 0;
  c_pieces = 0;
  c_drains = 0;
  c_prefill = 0;
  c_act_pieces = 0;
  return LPS_OK;
}

// ---- layer / model / stage walk ------------------------------------------------------
size_t lps_layer_scratch_bytes(const lps_layer_desc* L) {
  if (check_layer(L, "lps_layer_scratch_bytes")) return 0;
  return layer_scratch(L).total;
}

int lps_layer_forward(const lps_layer_desc* L, float* x, int32_t pos, void* scratch,
                      size_t scratch_bytes, void* stream) {
  int rc = check_layer(L, "lps_layer_forward");
  if (rc) return rc;
  LPS_REQUIRE(x && scratch, LPS_EINVAL, "lps_layer_forward: null x or scratch");
  LPS_REQUIRE(aligned16(x) && aligned16(scratch), LPS_EINVAL,
              "lps_layer_forward: x and scratch must be 16-byte aligned");
  LPS_REQUIRE(L->nq == 0 || (pos >= 0 && pos < L->ctx_max), LPS_ERANGE,
              "lps_layer_forward: pos %d outside [0, %d)", pos, L->ctx_max);
  LPS_REQUIRE(scratch_bytes >= layer_scratch(L).total, LPS_EINVAL,
              "lps_layer_forward: scratch %zu bytes < %zu needed", scratch_bytes,
              layer_scratch(L).total);
  return layer_forward(L, x, pos, scratch, as_stream(stream));
}

int lps_model_create(const lps_layer_desc* layers, int32_t n_layers, lps_model** out) {
  LPS_REQUIRE(out, LPS_EINVAL, "lps_model_create: null out");
  LPS_REQUIRE(layers && n_layers >= 1, LPS_EINVAL, "lps_model_create: need >= 1 layer");
  size_t mx = 0;
  for (int i = 0; i < n_layers; ++i) {
    char who[64];
    snprintf(who, sizeof who, "lps_model_create(layer %d)", i);
    int rc = check_layer(&layers[i], who);
    if (rc) return rc;
    mx = std::max(mx, layer_scratch(&layers[i]).total);
  }
  lps_model* m = new (std::nothrow) lps_model;
  LPS_REQUIRE(m, LPS_ENOMEM, "lps_model_create: out of host memory");
  m->layers.assign(layers, layers + n_layers);
  m->moes.reserve(size_t(n_layers));   // no reallocation: the layers point into it
  for (auto& L : m->layers)
    if (L.ffn_kind == LPS_FFN_MOE) {
      m->moes.push_back(*L.moe);
      L.moe = &m->moes.back();
    }
  m->scratch = mx;
  *out = m;
  return LPS_OK;
}

int lps_model_destroy(lps_model* m) {
  delete m;
  return LPS_OK;
}

size_t lps_model_scratch_bytes(const lps_model* m) { return m ? m->scratch : 0; }

int lps_stage_forward(const lps_model* m, const int32_t* fence, int32_t n_stages, int32_t stage,
                      float* x, int32_t pos, void* scratch, size_t scratch_bytes, void* stream) {
  LPS_REQUIRE(m, LPS_EINVAL, "lps_stage_forward: null model");
  int rc = check_fence(fence, n_stages, int32_t(m->layers.size()), "lps_stage_forward");
  if (rc) return rc;
  LPS_REQUIRE(stage >= 0 && stage < n_stages, LPS_ERANGE, "lps_stage_forward: stage %d outside [0, %d)",
              stage, n_stages);
  LPS_REQUIRE(x && scratch, LPS_EINVAL, "lps_stage_forward: null x or scratch");
  LPS_REQUIRE(aligned16(x) && aligned16(scratch), LPS_EINVAL,
              "lps_stage_forward: x and scratch must be 16-byte aligned");
  LPS_REQUIRE(scratch_bytes >= m->scratch, LPS_EINVAL, "lps_stage_forward: scratch %zu < %zu needed",
              scratch_bytes, m->scratch);
  for (int l = fence[stage]; l < fence[stage + 1]; ++l)
    LPS_REQUIRE(m->layers[l].nq == 0 || (pos >= 0 && pos < m->layers[l].ctx_max), LPS_ERANGE,
                "lps_stage_forward: pos %d outside layer %d's cache [0, %d)", pos, l,
                m->layers[l].ctx_max);
  hipStream_t st = as_stream(stream);
  for (int l = fence[stage]; l < fence[stage + 1]; ++l) {
    rc = layer_forward(&m->layers[l], x, pos, scratch, st);
    if (rc) return rc;
  }
  count_stage_walk();
  return LPS_OK;
}

}  // extern "C"

// The arguments of a device-position walk of one stage (the fence and stage checked).
static int check_dpos_walk(const lps_model* m, const int32_t* fence, int32_t stage, const float* x,
                           const int32_t* pos_dev, const void* scratch, size_t scratch_bytes,
                           const char* who) {
  LPS_REQUIRE(x && scratch && pos_dev, LPS_EINVAL, "%s: null x, scratch or pos", who);
  LPS_REQUIRE(aligned16(x) && aligned16(scratch) && (reinterpret_cast<uintptr_t>(pos_dev) & 3) == 0,
              LPS_EINVAL, "%s: x and scratch must be 16-byte aligned, pos 4", who);
  LPS_REQUIRE(scratch_bytes >= m->scratch, LPS_EINVAL, "%s: scratch %zu < %zu needed", who,
              scratch_bytes, m->scratch);
  for (int l = fence[stage]; l < fence[stage + 1]; ++l) {
    if (m->layers[l].nq == 0) continue;   // no attention: no position is read
    const float* t = m->layers[l].rope_cs;
    LPS_REQUIRE(t && (reinterpret_cast<uintptr_t>(t) & 7) == 0, LPS_EINVAL,
                "%s: layer %d needs an 8-byte aligned rope_cs table", who, l);
  }
  return LPS_OK;
}

extern "C" {

int lps_stage_forward_dpos(const lps_model* m, const int32_t* fence, int32_t n_stages,
                           int32_t stage, float* x, const int32_t* pos_dev, void* scratch,
                           size_t scratch_bytes, void* stream) {
  LPS_REQUIRE(m, LPS_EINVAL, "lps_stage_forward_dpos: null model");
  int rc = check_fence(fence, n_stages, int32_t(m->layers.size()), "lps_stage_forward_dpos");
  if (rc) return rc;
  LPS_REQUIRE(stage >= 0 && stage < n_stages, LPS_ERANGE,
              "lps_stage_forward_dpos: stage %d outside [0, %d)", stage, n_stages);
  rc = check_dpos_walk(m, fence, stage, x, pos_dev, scratch, scratch_bytes, "lps_stage_forward_dpos");
  if (rc) return rc;
  hipStream_t st = as_stream(stream);
  for (int l = fence[stage]; l < fence[stage + 1]; ++l) {
    rc = layer_forward(&m->layers[l], x, 0, scratch, st, pos_dev);
    if (rc) return rc;
  }
  count_stage_walk();
  return LPS_OK;
}

}  // extern "C"

// ---- the stage walk without caller scratch ---------------------------------------------
// For callers that cannot allocate (code under graph capture, tight serving loops):
// the layer scratch lives in this file-scope device array instead, one copy per GPU,
// held until the process ends.  In host code `scratch` names a host-side stand-in,
// never the device memory: its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is used.
namespace lps {
constexpr size_t kStaticScratchBytes = size_t(8) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
static std::mutex g_static_mu;
static std::vector<void*> g_static_ptr;   // per device ordinal, nullptr until looked up

static int static_scratch(void** out) {
  int dev = -1;
  LPS_HIP(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lk(g_static_mu);
  if (size_t(dev) >= g_static_ptr.size()) g_static_ptr.resize(size_t(dev) + 1, nullptr);
  if (!g_static_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(LPS_EHIP, "lps_stage_forward_static: hipGetSymbolAddress(scratch) on device %d: %s",
                  dev, hipGetErrorString(e));
    g_static_ptr[dev] = ptr;
  }
  *out = g_static_ptr[dev];
  return LPS_OK;
}
}  // namespace lps

extern "C" {

int lps_stage_forward_static(const lps_model* m, const int32_t* fence, int32_t n_stages,
                             int32_t stage, float* x, int32_t pos, void* stream) {
  LPS_REQUIRE(m, LPS_EINVAL, "lps_stage_forward_static: null model");
  LPS_REQUIRE(m->scratch <= kStaticScratchBytes, LPS_ERANGE,
              "lps_stage_forward_static: the model's layers need %zu bytes of scratch, more than "
              "the %zu bytes of the library's static buffer (use lps_stage_forward)",
              m->scratch, kStaticScratchBytes);
  void* sc = nullptr;
  int rc = static_scratch(&sc);
  if (rc) return rc;
  return lps_stage_forward(m, fence, n_stages, stage, x, pos, sc, kStaticScratchBytes, stream);
}

size_t lps_prefill_scratch_bytes(const lps_model* m, int32_t T) {
  if (!m || T < 1) return 0;
  size_t mx = 0;
  for (const auto& L : m->layers) mx = std::max(mx, prefill_scratch(&L, T).total);
  return mx;
}

int lps_stage_prefill(const lps_model* m, const int32_t* fence, int32_t n_stages, int32_t stage,
                      float* x, int32_t T, int32_t p0, void* scratch, size_t scratch_bytes,
                      void* stream) {
  LPS_REQUIRE(m, LPS_EINVAL, "lps_stage_prefill: null model");
  int rc = check_fence(fence, n_stages, int32_t(m->layers.size()), "lps_stage_prefill");
  if (rc) return rc;
  LPS_REQUIRE(stage >= 0 && stage < n_stages, LPS_ERANGE,
              "lps_stage_prefill: stage %d outside [0, %d)", stage, n_stages);
  LPS_REQUIRE(x && scratch, LPS_EINVAL, "lps_stage_prefill: null x or scratch");
  LPS_REQUIRE(aligned16(x) && aligned16(scratch), LPS_EINVAL,
              "lps_stage_prefill: x and scratch must be 16-byte aligned");
  LPS_REQUIRE(T >= 1, LPS_EINVAL, "lps_stage_prefill: T %d < 1", T);
  for (int l = fence[stage]; l < fence[stage + 1]; ++l) {
    char who[64];
    snprintf(who, sizeof who, "lps_stage_prefill(layer %d)", l);
    rc = check_prefill_layer(&m->layers[l], T, p0, who);
    if (rc) return rc;
  }
  const size_t need = lps_prefill_scratch_bytes(m, T);
  LPS_REQUIRE(scratch_bytes >= need, LPS_EINVAL, "lps_stage_prefill: scratch %zu < %zu needed",
              scratch_bytes, need);
  hipStream_t st = as_stream(stream);
  for (int l = fence[stage]; l < fence[stage + 1]; ++l) {
    rc = prefill_layer(&m->layers[l], x, T, p0, scratch, st);
    if (rc) return rc;
  }
  count_prefill_walk();
  return LPS_OK;
}

int lps_embed_rows(const void* table, int32_t wdtype, int32_t vocab, int32_t d, const int32_t* tok,
                   int32_t T, float* x, void* stream) {
  LPS_REQUIRE(table && tok && x, LPS_EINVAL, "lps_embed_rows: null pointer");
  LPS_REQUIRE(vocab > 0 && d > 0 && T >= 1 && T <= 65535, LPS_EINVAL,
              "lps_embed_rows: vocab %d, d %d, T %d (1 .. 65535)", vocab, d, T);
  LPS_REQUIRE(wdtype == LPS_F32 || wdtype == LPS_BF16, LPS_EINVAL,
              "lps_embed_rows: table dtype %d (f32 or bf16 only)", wdtype);
  return launch_embed_rows(table, wdtype, vocab, d, tok, T, x, as_stream(stream));
}

int lps_rope_table(int32_t hd, float rope_base, int32_t n_pos, float* host_out) {
  LPS_REQUIRE(host_out, LPS_EINVAL, "lps_rope_table: null output");
  LPS_REQUIRE(hd > 0 && hd % 2 == 0, LPS_EINVAL, "lps_rope_table: head dim %d (positive, even)", hd);
  LPS_REQUIRE(n_pos >= 1, LPS_EINVAL, "lps_rope_table: n_pos %d < 1", n_pos);
  LPS_REQUIRE(rope_base > 0.f, LPS_EINVAL, "lps_rope_table: base %g must be positive", rope_base);
  const int half = hd / 2;
  for (int p = 0; p < n_pos; ++p)
    for (int i = 0; i < half; ++i) rope_cos_sin(rope_base, hd, p, i, host_out + 2 * (size_t(p) * half + i));
  return LPS_OK;
}

int lps_step_advance(int32_t* state, int32_t pos_limit, const int32_t* argmax, int32_t* tok_cur,
                     const int32_t* feed, int32_t n_feed, int32_t* tok_hist, int32_t hist_cap,
                     const float* logits, int32_t vocab, float* logits_hist, void* stream) {
  LPS_REQUIRE(state, LPS_EINVAL, "lps_step_advance: null state");
  LPS_REQUIRE((argmax == nullptr) == (tok_cur == nullptr), LPS_EINVAL,
              "lps_step_advance: argmax and tok_cur go together (both NULL: no token chain)");
  LPS_REQUIRE(argmax || (n_feed == 0 && !tok_hist && !logits_hist), LPS_EINVAL,
              "lps_step_advance: fed ids and histories need the token chain");
  LPS_REQUIRE(pos_limit >= 1, LPS_EINVAL, "lps_step_advance: pos_limit %d < 1", pos_limit);
  LPS_REQUIRE(n_feed >= 0 && (n_feed == 0 || feed), LPS_EINVAL,
              "lps_step_advance: %d fed ids need a feed array", n_feed);
  LPS_REQUIRE(hist_cap >= 0 && (hist_cap == 0 || tok_hist), LPS_EINVAL,
              "lps_step_advance: a history of %d steps needs tok_hist", hist_cap);
  LPS_REQUIRE(!logits_hist || (logits && vocab > 0), LPS_EINVAL,
              "lps_step_advance: a logits history needs logits and vocab > 0");
  return launch_step_advance(state, pos_limit, argmax, tok_cur, feed, n_feed, tok_hist, hist_cap,
                             logits, vocab, logits_hist, as_stream(stream));
}

int lps_row_at_step(const int32_t* state, const float* src, int64_t src_stride, float* dst,
                    int64_t dst_stride, int32_t n, int32_t n_rows, void* stream) {
  LPS_REQUIRE(state && src && dst, LPS_EINVAL, "lps_row_at_step: null state, src or dst");
  LPS_REQUIRE(n >= 1 && n_rows >= 1, LPS_EINVAL, "lps_row_at_step: n %d and n_rows %d must be >= 1", n,
              n_rows);
  LPS_REQUIRE(src_stride >= 0 && dst_stride >= 0 && (src_stride == 0 || src_stride >= n) &&
                  (dst_stride == 0 || dst_stride >= n),
              LPS_EINVAL, "lps_row_at_step: strides %lld / %lld (0, or at least n %d)",
              (long long)src_stride, (long long)dst_stride, n);
  return launch_row_at_step(state, src, src_stride, dst, dst_stride, n, n_rows, as_stream(stream));
}

// ---- whole-pass graphs --------------------------------------------------------------------
int lps_graph_begin(void* stream) {
  LPS_REQUIRE(g_timer.kind.load() == 0, LPS_ESTATE,
              "lps_graph_begin: a kernel timer is running (timed launches are not captured)");
  hipStream_t st = as_stream(stream);
  LPS_REQUIRE(st != nullptr, LPS_EINVAL, "lps_graph_begin: the null stream cannot be captured");
  unsigned long long cid = 0;
  int rc = capture_of(st, &cid);
  if (rc) return rc;
  LPS_REQUIRE(cid == 0, LPS_ESTATE, "lps_graph_begin: the stream is already capturing");
  // relaxed: the walk may call hipFuncSetAttribute the first time a shape runs
  LPS_HIP(hipStreamBeginCapture(st, hipStreamCaptureModeRelaxed));
  return LPS_OK;
}

int lps_graph_end(void* stream, void* const* join, int32_t n_join, lps_graph** out) {
  LPS_REQUIRE(out, LPS_EINVAL, "lps_graph_end: null out");
  *out = nullptr;
  LPS_REQUIRE(n_join >= 0 && (n_join == 0 || join), LPS_EINVAL, "lps_graph_end: bad join list");
  hipStream_t st = as_stream(stream);
  unsigned long long cid = 0;
  int rc = capture_of(st, &cid);
  hipError_t jerr = hipSuccess;
  std::vector<hipEvent_t> evs;
  if (!rc && cid == 0) rc = fail(LPS_ESTATE, "lps_graph_end: the stream is not capturing");
  // join every forked stream of this capture back into the origin stream
  for (int i = 0; !rc && jerr == hipSuccess && i < n_join; ++i) {
    hipStream_t j = as_stream(join[i]);
    if (j == st || j == nullptr) continue;
    unsigned long long jc = 0;
    rc = capture_of(j, &jc);
    if (rc || jc == 0) continue;   // never forked into the capture: nothing to join
    if (jc != cid) {
      rc = fail(LPS_ESTATE, "lps_graph_end: join stream %d is in another capture", i);
      break;
    }
    hipEvent_t e;
    jerr = hipEventCreateWithFlags(&e, hipEventDisableTiming);
    if (jerr != hipSuccess) break;
    evs.push_back(e);
    jerr = hipEventRecord(e, j);
    if (jerr == hipSuccess) jerr = hipStreamWaitEvent(st, e, 0);
  }
  // the capture always ends here, also after a failure, so the stream is usable again
  hipGraph_t graph = nullptr;
  hipError_t eerr = cid ? hipStreamEndCapture(st, &graph) : hipSuccess;
  for (auto e : evs) (void)hipEventDestroy(e);
  if (!rc && jerr != hipSuccess) rc = fail(LPS_EHIP, "lps_graph_end: join: %s", hipGetErrorString(jerr));
  if (!rc && eerr != hipSuccess)
    rc = fail(LPS_EHIP, "lps_graph_end: hipStreamEndCapture: %s", hipGetErrorString(eerr));
  if (!rc && graph == nullptr) rc = fail(LPS_EHIP, "lps_graph_end: the capture produced no graph");
  hipGraphExec_t exec = nullptr;
  if (!rc) {
    hipError_t ierr = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    if (ierr != hipSuccess) rc = fail(LPS_EHIP, "lps_graph_end: hipGraphInstantiate: %s", hipGetErrorString(ierr));
  }
  if (graph) (void)hipGraphDestroy(graph);
  if (rc) {
    (void)hipGetLastError();
    return rc;
  }
  lps_graph* g = new (std::nothrow) lps_graph;
  if (!g) {
    (void)hipGraphExecDestroy(exec);
    return fail(LPS_ENOMEM, "lps_graph_end: out of host memory");
  }
  g->exec = exec;
  *out = g;
  return LPS_OK;
}

int lps_graph_launch(lps_graph* g, void* stream) {
  LPS_REQUIRE(g, LPS_EINVAL, "lps_graph_launch: null graph");
  LPS_HIP(hipGraphLaunch(g->exec, as_stream(stream)));
  return LPS_OK;
}

int lps_graph_destroy(lps_graph* g) {
  if (!g) return LPS_OK;
  hipError_t e = hipGraphExecDestroy(g->exec);
  delete g;
  if (e != hipSuccess) return fail(LPS_EHIP, "lps_graph_destroy: %s", hipGetErrorString(e));
  return LPS_OK;
}

// ---- step-level entry points -----------------------------------------------------------
int lps_gemv(int32_t wdtype, const void* w, const uint8_t* s, int32_t N, int32_t K, const float* x,
             const float* norm_g, float eps, float* y, int32_t mode, void* stream) {
  LPS_REQUIRE(wdtype == LPS_F32 || wdtype == LPS_BF16 || wdtype == LPS_MXFP4, LPS_EINVAL,
              "lps_gemv: wdtype %d", wdtype);
  LPS_REQUIRE(mode == LPS_EPI_STORE || mode == LPS_EPI_ADD || mode == LPS_EPI_SWIGLU, LPS_EINVAL,
              "lps_gemv: mode %d", mode);
  LPS_REQUIRE(N > 0 && K > 0, LPS_EINVAL, "lps_gemv: N %d / K %d must be > 0", N, K);
  LPS_REQUIRE(K % chunk_of(wdtype) == 0, LPS_EINVAL, "lps_gemv: K %d must be a multiple of %d", K,
              chunk_of(wdtype));
  LPS_REQUIRE(mode != LPS_EPI_SWIGLU || N % 2 == 0, LPS_EINVAL, "lps_gemv: SwiGLU needs an even N (%d)", N);
  LPS_REQUIRE(size_t(K) * 4 <= 160 * 1024, LPS_EUNSUP, "lps_gemv: K %d exceeds the LDS vector", K);
  LPS_REQUIRE(w && x && y, LPS_EINVAL, "lps_gemv: null w, x or y");
  LPS_REQUIRE(wdtype != LPS_MXFP4 || s, LPS_EINVAL, "lps_gemv: MXFP4 needs scales");
  LPS_REQUIRE(aligned16(w) && aligned16(x) && (!norm_g || aligned16(norm_g)), LPS_EINVAL,
              "lps_gemv: w, x and norm_g must be 16-byte aligned");
  return launch_gemv(wdtype, w, s, N, K, x, norm_g, eps, y, mode, as_stream(stream));
}

int lps_qkv_rope_append(const lps_layer_desc* L, const float* x, int32_t pos, float* q,
                        void* stream) {
  int rc = check_layer(L, "lps_qkv_rope_append");
  if (rc) return rc;
  LPS_REQUIRE(L->nq > 0, LPS_EINVAL, "lps_qkv_rope_append: the layer has no attention (nq 0)");
  LPS_REQUIRE(x && q && aligned16(x), LPS_EINVAL, "lps_qkv_rope_append: null or unaligned x / q");
  LPS_REQUIRE(pos >= 0 && pos < L->ctx_max, LPS_ERANGE,
              "lps_qkv_rope_append: pos %d outside [0, %d)", pos, L->ctx_max);
  QkvArgs qa{L, x, pos, q};
  return launch_qkv(qa, as_stream(stream));
}

size_t lps_attention_scratch_bytes(int32_t nq, int32_t nkv, int32_t hd, int32_t ctx_max) {
  if (nq <= 0 || nkv <= 0 || nq % nkv || hd <= 0 || ctx_max <= 0) return 0;
  return attn_scratch(nq, nkv, hd, ctx_max);
}

int lps_attention_decode(int32_t nq, int32_t nkv, int32_t hd, int32_t kvdtype, const void* k_cache,
                         const void* v_cache, int32_t ctx_max, int32_t n_rows, const float* q,
                         float* o, void* scratch, size_t scratch_bytes, void* stream) {
  LPS_REQUIRE(nq > 0 && nkv > 0 && nq % nkv == 0, LPS_EUNSUP,
              "lps_attention_decode: nq %d must be a multiple of nkv %d", nq, nkv);
  LPS_REQUIRE(hd == 64 || hd == 128 || hd == 256, LPS_EUNSUP, "lps_attention_decode: head dim %d", hd);
  LPS_REQUIRE(kvdtype == LPS_F32 || kvdtype == LPS_BF16, LPS_EINVAL, "lps_attention_decode: kvdtype %d",
              kvdtype);
  LPS_REQUIRE(n_rows >= 1 && n_rows <= ctx_max, LPS_ERANGE,
              "lps_attention_decode: n_rows %d outside [1, ctx_max=%d]", n_rows, ctx_max);
  LPS_REQUIRE(kvdtype != LPS_BF16 || (ctx_max % 16 == 0 && ctx_max <= (1 << 22)), LPS_EINVAL,
              "lps_attention_decode: bf16 caches need ctx_max %d to be a multiple of 16 and at "
              "most 4194304", ctx_max);
  LPS_REQUIRE(k_cache && v_cache && q && o && scratch, LPS_EINVAL, "lps_attention_decode: null pointer");
  LPS_REQUIRE(aligned16(k_cache) && aligned16(v_cache), LPS_EINVAL,
              "lps_attention_decode: caches must be 16-byte aligned");
  LPS_REQUIRE(scratch_bytes >= attn_scratch(nq, nkv, hd, ctx_max), LPS_EINVAL,
              "lps_attention_decode: scratch %zu < %zu", scratch_bytes,
              attn_scratch(nq, nkv, hd, ctx_max));
  return launch_attention(nq, nkv, hd, kvdtype, k_cache, v_cache, ctx_max, n_rows, q, o, scratch,
                          as_stream(stream));
}

size_t lps_head_scratch_bytes(const lps_head_desc* h) { return h ? head_scratch(h) : 0; }

int lps_head_forward(const lps_head_desc* h, const float* x, float* logits, int32_t* tok_out,
                     void* scratch, size_t scratch_bytes, void* stream) {
  LPS_REQUIRE(h, LPS_EINVAL, "lps_head_forward: null head");
  LPS_REQUIRE(h->d > 0 && h->vocab > 0, LPS_EINVAL, "lps_head_forward: d %d / vocab %d", h->d, h->vocab);
  LPS_REQUIRE(h->wdtype == LPS_F32 || h->wdtype == LPS_BF16, LPS_EINVAL,
              "lps_head_forward: wdtype %d (f32 or bf16)", h->wdtype);
  LPS_REQUIRE(h->d % chunk_of(h->wdtype) == 0 && h->d <= 8192, LPS_EINVAL,
              "lps_head_forward: d %d (a multiple of the weight chunk, at most 8192)", h->d);
  LPS_REQUIRE(h->g_out && h->w_lm && x && logits && tok_out && scratch, LPS_EINVAL,
              "lps_head_forward: null pointer");
  LPS_REQUIRE(aligned16(h->w_lm) && aligned16(h->g_out) && aligned16(x), LPS_EINVAL,
              "lps_head_forward: weights, gain and x must be 16-byte aligned");
  LPS_REQUIRE(scratch_bytes >= head_scratch(h), LPS_EINVAL, "lps_head_forward: scratch %zu < %zu",
              scratch_bytes, head_scratch(h));
  return launch_head(h, x, logits, tok_out, scratch, scratch_bytes, as_stream(stream),
                     timer_take(LPS_KIND_HEAD));
}

int lps_step_finish(const lps_head_desc* h, const float* x, float* logits, int32_t* state,
                    int32_t pos_limit, const int32_t* feed, int32_t n_feed, int32_t* tok_hist,
                    float* logits_hist, int32_t hist_cap, const void* embed, int32_t embed_dtype,
                    float* x_next, int32_t* tok_cur, const lps_host_ring* ring, void* scratch,
                    size_t scratch_bytes, void* stream) {
  LPS_REQUIRE(h, LPS_EINVAL, "lps_step_finish: null head");
  LPS_REQUIRE(h->d > 0 && h->vocab > 0, LPS_EINVAL, "lps_step_finish: d %d / vocab %d", h->d, h->vocab);
  LPS_REQUIRE(h->wdtype == LPS_F32 || h->wdtype == LPS_BF16, LPS_EINVAL,
              "lps_step_finish: wdtype %d (f32 or bf16)", h->wdtype);
  LPS_REQUIRE(h->d % chunk_of(h->wdtype) == 0 && h->d <= 8192, LPS_EINVAL,
              "lps_step_finish: d %d (a multiple of the weight chunk, at most 8192)", h->d);
  LPS_REQUIRE(embed_dtype == LPS_F32 || embed_dtype == LPS_BF16, LPS_EINVAL,
              "lps_step_finish: embed_dtype %d (f32 or bf16)", embed_dtype);
  LPS_REQUIRE(h->g_out && h->w_lm && x && logits && state && embed && x_next && scratch, LPS_EINVAL,
              "lps_step_finish: null pointer");
  LPS_REQUIRE(aligned16(h->w_lm) && aligned16(h->g_out) && aligned16(x), LPS_EINVAL,
              "lps_step_finish: weights, gain and x must be 16-byte aligned");
  LPS_REQUIRE(pos_limit >= 1, LPS_EINVAL, "lps_step_finish: pos_limit %d < 1", pos_limit);
  LPS_REQUIRE(n_feed >= 0 && (n_feed == 0 || feed), LPS_EINVAL,
              "lps_step_finish: %d fed ids need a feed array", n_feed);
  LPS_REQUIRE(hist_cap >= 0 && (hist_cap == 0 || tok_hist), LPS_EINVAL,
              "lps_step_finish: a history of %d steps needs tok_hist", hist_cap);
  LPS_REQUIRE(scratch_bytes >= head_scratch(h), LPS_EINVAL, "lps_step_finish: scratch %zu < %zu",
              scratch_bytes, head_scratch(h));
  float* ring_l = nullptr;
  int32_t* ring_t = nullptr;
  int32_t slots = 0;
  if (ring) {
    LPS_REQUIRE(ring->slots >= 1 && (ring->logits || ring->tok), LPS_EINVAL,
                "lps_step_finish: a host ring needs slots >= 1 and logits or tok (slots %d)",
                ring->slots);
    // the kernels store through the device's mapping of the pinned rows
    if (ring->logits && !pinned_host_on_device(ring->logits, reinterpret_cast<void**>(&ring_l)))
      return fail(LPS_EINVAL, "lps_step_finish: ring logits are not pinned host memory");
    if (ring->tok && !pinned_host_on_device(ring->tok, reinterpret_cast<void**>(&ring_t)))
      return fail(LPS_EINVAL, "lps_step_finish: ring tok is not pinned host memory");
    slots = ring->slots;
  }
  return launch_step_finish(h, x, logits, state, pos_limit, feed, n_feed, tok_hist, logits_hist,
                            hist_cap, embed, embed_dtype, x_next, tok_cur, ring_l, ring_t, slots,
                            scratch, as_stream(stream), timer_take(LPS_KIND_HEAD));
}

// ---- benchmark timer ----------------------------------------------------------------------
int lps_timer_start(int32_t kind, int32_t capacity) {
  LPS_REQUIRE(kind >= LPS_KIND_QKV && kind <= LPS_KIND_MOE_GEMM2, LPS_EINVAL, "lps_timer_start: kind %d",
              kind);
  LPS_REQUIRE(capacity >= 1 && capacity <= 1 << 16, LPS_EINVAL, "lps_timer_start: capacity %d", capacity);
  std::lock_guard<std::mutex> lk(g_timer.mu);
  LPS_REQUIRE(g_timer.kind.load() == 0, LPS_ESTATE, "lps_timer_start: a timer is already running");
  g_timer.ev.assign(size_t(2) * capacity, nullptr);
  // timing-only events: no system-scope fence (cache writeback / invalidate) when
  // they complete, which would otherwise be timed with, and slow, the kernels
  for (auto& e : g_timer.ev) {
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) {
      for (auto& f : g_timer.ev)
        if (f) (void)hipEventDestroy(f);
      g_timer.ev.clear();
      return fail(LPS_EHIP, "lps_timer_start: hipEventCreate failed");
    }
  }
  g_timer.used = 0;
  g_timer.kind.store(kind);
  return LPS_OK;
}

int lps_timer_stop(float* ms_out, int32_t cap, int32_t* n_out) {
  LPS_REQUIRE(n_out && (cap == 0 || ms_out), LPS_EINVAL, "lps_timer_stop: null output");
  std::lock_guard<std::mutex> lk(g_timer.mu);
  LPS_REQUIRE(g_timer.kind.load() != 0, LPS_ESTATE, "lps_timer_stop: no timer is running");
  g_timer.kind.store(0);
  int rc = LPS_OK;
  int n = 0;
  for (int i = 0; i < g_timer.used; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(g_timer.ev[2 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms, g_timer.ev[2 * i], g_timer.ev[2 * i + 1]) != hipSuccess) {
      rc = fail(LPS_EHIP, "lps_timer_stop: reading event pair %d failed", i);
      break;
    }
    if (n < cap) ms_out[n] = ms;
    ++n;
  }
  for (auto& e : g_timer.ev) (void)hipEventDestroy(e);
  g_timer.ev.clear();
  g_timer.used = 0;
  *n_out = n < cap ? n : cap;
  return rc;
}

// ---- A14 boundaries ----------------------------------------------------------------------
int lps_boundary_create(int32_t n_elems, float* slot0, float* slot1, lps_boundary** out) {
  LPS_REQUIRE(out, LPS_EINVAL, "lps_boundary_create: null out");
  LPS_REQUIRE(n_elems > 0, LPS_EINVAL, "lps_boundary_create: n_elems %d", n_elems);
  LPS_REQUIRE(slot0 && slot1 && slot0 != slot1, LPS_EINVAL,
              "lps_boundary_create: need two distinct slots");
  LPS_REQUIRE(aligned16(slot0) && aligned16(slot1), LPS_EINVAL,
              "lps_boundary_create: slots must be 16-byte aligned");
  lps_boundary* b = new (std::nothrow) lps_boundary;
  LPS_REQUIRE(b, LPS_ENOMEM, "lps_boundary_create: out of host memory");
  b->n = n_elems;
  b->slot[0] = slot0;
  b->slot[1] = slot1;
  b->next_send = 0;
  b->next_recv = 0;
  for (int k = 0; k < 2; ++k) {
    b->tx_recorded[k] = b->rx_recorded[k] = false;
    b->tx_stream[k] = b->rx_stream[k] = nullptr;
    b->tx_cap[k] = b->rx_cap[k] = 0;
    // device-side ordering between the stage streams only: no system-scope fence
    // (an L2 writeback for the host) when they are recorded
    hipError_t e1 = hipEventCreateWithFlags(&b->ev_tx[k], hipEventDisableTiming | hipEventDisableSystemFence);
    hipError_t e2 = hipEventCreateWithFlags(&b->ev_rx[k], hipEventDisableTiming | hipEventDisableSystemFence);
    if (e1 != hipSuccess || e2 != hipSuccess) {
      delete b;
      return fail(LPS_EHIP, "lps_boundary_create: hipEventCreate failed");
    }
  }
  *out = b;
  return LPS_OK;
}

int lps_boundary_send(lps_boundary* b, const float* x, int64_t step, void* producer) {
  LPS_REQUIRE(b && x, LPS_EINVAL, "lps_boundary_send: null boundary or x");
  LPS_REQUIRE(aligned16(x), LPS_EINVAL, "lps_boundary_send: x must be 16-byte aligned");
  LPS_REQUIRE(step == b->next_send, LPS_ESTATE,
              "lps_boundary_send: step %lld sent out of order (expected %lld)", (long long)step,
              (long long)b->next_send);
  LPS_REQUIRE(step - b->next_recv < 2, LPS_ESTATE,
              "lps_boundary_send: step %lld would overwrite slot %d before step %lld was received",
              (long long)step, int(step & 1), (long long)(step - 2));
  const int k = int(step & 1);
  hipStream_t st = as_stream(producer);
  unsigned long long cid = 0;
  int rc = capture_of(st, &cid);
  if (rc) return rc;
  // a wait on the own stream is implied by stream order (the same-stream seam);
  // a receive recorded in another context (eager vs a capture) is not waited:
  // ordering eager work against a graph launch is the caller's.  A receive made
  // on its producer's stream recorded no event; when the slot's next producer is
  // another stream, ev_rx is recorded now on the receiving stream, after all its
  // work so far, which covers that receive's copy.
  if (b->rx_stream[k] && b->rx_stream[k] != st && b->rx_cap[k] == cid) {
    if (!b->rx_recorded[k]) {
      unsigned long long rcid = 0;
      rc = capture_of(b->rx_stream[k], &rcid);
      if (rc) return rc;
      LPS_REQUIRE(rcid == cid, LPS_ESTATE,
                  "lps_boundary_send: slot %d's last receive stream is in another capture context",
                  k);
      LPS_HIP(hipEventRecord(b->ev_rx[k], b->rx_stream[k]));
      b->rx_recorded[k] = true;
    }
    LPS_HIP(hipStreamWaitEvent(st, b->ev_rx[k], 0));
  }
  rc = launch_copy_f32(x, b->slot[k], b->n, st);
  if (rc) return rc;
  // ev_tx is recorded by the receive, on this stream, when the consumer turns out to
  // be another stream: a marker after all work enqueued here so far, which covers
  // the copy above (nothing in between can un-write the slot)
  b->tx_recorded[k] = false;
  b->tx_stream[k] = st;
  b->tx_cap[k] = cid;
  b->next_send = step + 1;
  count_send();
  return LPS_OK;
}

int lps_boundary_recv(lps_boundary* b, float* x, int64_t step, void* consumer) {
  LPS_REQUIRE(b && x, LPS_EINVAL, "lps_boundary_recv: null boundary or x");
  LPS_REQUIRE(aligned16(x), LPS_EINVAL, "lps_boundary_recv: x must be 16-byte aligned");
  LPS_REQUIRE(step == b->next_recv, LPS_ESTATE,
              "lps_boundary_recv: step %lld received out of order (expected %lld)", (long long)step,
              (long long)b->next_recv);
  LPS_REQUIRE(step < b->next_send, LPS_ESTATE, "lps_boundary_recv: step %lld was never sent",
              (long long)step);
  const int k = int(step & 1);
  hipStream_t st = as_stream(consumer);
  unsigned long long ccid = 0, tcid = 0;
  int rc = capture_of(st, &ccid);
  if (!rc) rc = capture_of(b->tx_stream[k], &tcid);
  if (rc) return rc;
  // send and receive of one step belong to one context: both eager, or both in
  // one capture (a consumer stream that is not capturing yet joins the
  // producer's capture through the wait below)
  LPS_REQUIRE(tcid == b->tx_cap[k] && (ccid == 0 || ccid == tcid), LPS_ESTATE,
              "lps_boundary_recv: step %lld was sent in another capture context than it is "
              "received in", (long long)step);
  if (b->tx_stream[k] != st) {
    LPS_HIP(hipEventRecord(b->ev_tx[k], b->tx_stream[k]));
    b->tx_recorded[k] = true;
    LPS_HIP(hipStreamWaitEvent(st, b->ev_tx[k], 0));
  }
  rc = launch_copy_f32(b->slot[k], x, b->n, st);
  if (rc) return rc;
  // the producer's next use of slot k waits this event only from another stream
  if (b->tx_stream[k] != st) {
    LPS_HIP(hipEventRecord(b->ev_rx[k], st));
    b->rx_recorded[k] = true;
  } else {
    b->rx_recorded[k] = false;
  }
  b->rx_cap[k] = tcid;   // the consumer now records in the producer's context
  b->rx_stream[k] = st;
  b->next_recv = step + 1;
  count_recv();
  return LPS_OK;
}

int lps_boundary_hop(lps_boundary* b, const float* x, float* x_out, int64_t step, void* stream) {
  LPS_REQUIRE(b && x && x_out, LPS_EINVAL, "lps_boundary_hop: null boundary, x or x_out");
  LPS_REQUIRE(aligned16(x) && aligned16(x_out), LPS_EINVAL,
              "lps_boundary_hop: x and x_out must be 16-byte aligned");
  hipStream_t st = as_stream(stream);
  unsigned long long cid = 0;
  int rc = hop_begin(b, step, st, &cid, "lps_boundary_hop");
  if (rc) return rc;
  rc = launch_copy2_f32(x, b->slot[step & 1], x_out, b->n, st);
  if (rc) return rc;
  hop_end(b, step, st, cid);
  return LPS_OK;
}

int lps_stage_forward_dpos_hop(const lps_model* m, const int32_t* fence, int32_t n_stages,
                               int32_t stage, float* x, const int32_t* pos_dev, void* scratch,
                               size_t scratch_bytes, lps_boundary* b, float* x_out, int64_t step,
                               void* stream) {
  LPS_REQUIRE(m, LPS_EINVAL, "lps_stage_forward_dpos_hop: null model");
  int rc = check_fence(fence, n_stages, int32_t(m->layers.size()), "lps_stage_forward_dpos_hop");
  if (rc) return rc;
  LPS_REQUIRE(stage >= 0 && stage < n_stages, LPS_ERANGE,
              "lps_stage_forward_dpos_hop: stage %d outside [0, %d)", stage, n_stages);
  rc = check_dpos_walk(m, fence, stage, x, pos_dev, scratch, scratch_bytes,
                       "lps_stage_forward_dpos_hop");
  if (rc) return rc;
  LPS_REQUIRE(b && x_out, LPS_EINVAL, "lps_stage_forward_dpos_hop: null boundary or x_out");
  LPS_REQUIRE(aligned16(x_out), LPS_EINVAL, "lps_stage_forward_dpos_hop: x_out must be 16-byte aligned");
  const lps_layer_desc& last = m->layers[fence[stage + 1] - 1];
  LPS_REQUIRE(b->n == last.d, LPS_EINVAL,
              "lps_stage_forward_dpos_hop: boundary rows of %d values, the stage's rows are %d",
              b->n, last.d);
  hipStream_t st = as_stream(stream);
  unsigned long long cid = 0;
  rc = hop_begin(b, step, st, &cid, "lps_stage_forward_dpos_hop");
  if (rc) return rc;
  for (int l = fence[stage]; l < fence[stage + 1]; ++l) {
    const bool tail = l == fence[stage + 1] - 1;
    rc = layer_forward(&m->layers[l], x, 0, scratch, st, pos_dev, tail ? b->slot[step & 1] : nullptr,
                       tail ? x_out : nullptr);
    if (rc) return rc;
  }
  hop_end(b, step, st, cid);
  count_stage_walk();
  return LPS_OK;
}

int lps_boundary_destroy(lps_boundary* b) {
  if (!b) return LPS_OK;
  int rc = LPS_OK;
  for (int k = 0; k < 2; ++k) {
    if (hipEventSynchronize(b->ev_tx[k]) != hipSuccess) rc = LPS_EHIP;
    if (hipEventSynchronize(b->ev_rx[k]) != hipSuccess) rc = LPS_EHIP;
    (void)hipEventDestroy(b->ev_tx[k]);
    (void)hipEventDestroy(b->ev_rx[k]);
  }
  delete b;
  if (rc) return fail(rc, "lps_boundary_destroy: hipEventSynchronize failed");
  return LPS_OK;
}

// ---- A16 deferred readback ------------------------------------------------------------------
int lps_logits_defer(const float* logits, const int32_t* tok, int32_t vocab, void* last_stage,
                     void* readback, float* host_logits, int32_t* host_tok, lps_pending** out) {
  LPS_REQUIRE(out, LPS_EINVAL, "lps_logits_defer: null out");
  LPS_REQUIRE(logits || tok, LPS_EINVAL, "lps_logits_defer: nothing to read back");
  LPS_REQUIRE(!logits || (host_logits && vocab > 0), LPS_EINVAL,
              "lps_logits_defer: logits need host_logits and vocab > 0");
  LPS_REQUIRE(!tok || host_tok, LPS_EINVAL, "lps_logits_defer: tok needs host_tok");
  *out = nullptr;
  hipStream_t ls = as_stream(last_stage), rb = as_stream(readback);
  hipEvent_t done = nullptr, drained = nullptr;
  // done orders the copies after the step on the device (no system-scope fence on
  // the last stage's stream); drained is what the host waits on, with the fence that
  // makes the copied bytes visible to it
  hipError_t e = hipEventCreateWithFlags(&done, hipEventDisableTiming | hipEventDisableSystemFence);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&drained, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventRecord(done, ls);
  if (e == hipSuccess) e = hipStreamWaitEvent(rb, done, 0);
  if (e == hipSuccess && logits)
    e = hipMemcpyAsync(host_logits, logits, size_t(vocab) * 4, hipMemcpyDeviceToHost, rb);
  if (e == hipSuccess && tok) e = hipMemcpyAsync(host_tok, tok, 4, hipMemcpyDeviceToHost, rb);
  if (e == hipSuccess) e = hipEventRecord(drained, rb);
  if (done) (void)hipEventDestroy(done);
  if (e != hipSuccess) {
    if (drained) (void)hipEventDestroy(drained);
    return fail(LPS_EHIP, "lps_logits_defer: %s", hipGetErrorString(e));
  }
  return pending_issue(drained, out, "lps_logits_defer");
}

int lps_pending_mark(void* stream, lps_pending** out) {
  LPS_REQUIRE(out, LPS_EINVAL, "lps_pending_mark: null out");
  *out = nullptr;
  // the system-scope fence of this event is what makes the device's stores to host
  // memory visible to the host once it has fired
  hipEvent_t ev = nullptr;
  hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventRecord(ev, as_stream(stream));
  if (e != hipSuccess) {
    if (ev) (void)hipEventDestroy(ev);
    return fail(LPS_EHIP, "lps_pending_mark: %s", hipGetErrorString(e));
  }
  return pending_issue(ev, out, "lps_pending_mark");
}

int lps_pending_order(lps_pending* p, void* stream) {
  LPS_REQUIRE(p, LPS_EINVAL, "lps_pending_order: null pending");
  const uintptr_t v = reinterpret_cast<uintptr_t>(p);
  const uint32_t slot = uint32_t(v & 0xffffffffu) - 1u, gen = uint32_t(v >> 32);
  std::lock_guard<std::mutex> lk(g_pend_mu);
  LPS_REQUIRE(slot < g_pend.size() && g_pend[slot].live && g_pend[slot].gen == gen, LPS_ESTATE,
              "lps_pending_order: the pending was already waited or dropped (or never issued)");
  LPS_HIP(hipStreamWaitEvent(as_stream(stream), g_pend[slot].drained, 0));
  return LPS_OK;
}

int lps_pending_wait(lps_pending* p) {
  LPS_REQUIRE(p, LPS_EINVAL, "lps_pending_wait: null pending");
  hipEvent_t ev = pending_take(p);
  LPS_REQUIRE(ev, LPS_ESTATE,
              "lps_pending_wait: the pending was already waited or dropped (or never issued)");
  hipError_t e = hipEventSynchronize(ev);
  (void)hipEventDestroy(ev);
  count_drain();
  if (e != hipSuccess) return fail(LPS_EHIP, "lps_pending_wait: %s", hipGetErrorString(e));
  return LPS_OK;
}

int lps_pending_drop(lps_pending* p) {
  LPS_REQUIRE(p, LPS_EINVAL, "lps_pending_drop: null pending");
  hipEvent_t ev = pending_take(p);
  LPS_REQUIRE(ev, LPS_ESTATE,
              "lps_pending_drop: the pending was already waited or dropped (or never issued)");
  // the copies stay enqueued; destroying the event defers its release until it fires
  (void)hipEventDestroy(ev);
  count_drain();
  return LPS_OK;
}

}  // extern "C"
