/*
 * lps.h — C ABI of liblps, the MI355X (gfx950) staged single-token decode path.
 *
 * A transformer's layers are cut into contiguous ranges ("stages").  Each
 * stage walks its own layers on its own HIP stream; the only tensor that
 * crosses a stage boundary is the [n_embd] f32 hidden state, passed through
 * two persistent, event-ordered slots per boundary; the last stage's logits
 * are read back later on a dedicated stream.  (memra-engine `pp` module docs:
 * header, the stage map / boundary runtimes / ownership across a boundary /
 * deferred readback; functions pp_cuts, stage_of, pp2_overlap.)
 *
 * Conventions for every entry point:
 *  - Return value: LPS_OK (0) or a negative LPS_E* status.  On error nothing
 *    has been enqueued, and lps_last_error() names the call and the argument
 *    at fault (thread-local text, valid until the next failing call on the
 *    same thread).  No entry point aborts, exits or silently falls back.
 *  - Pointers marked (dev) are device memory of the current HIP device,
 *    (host) are host memory.  The caller owns every buffer passed in; the
 *    library never allocates or frees caller memory.  The library owns only
 *    the opaque handles it creates (and the hipEvents inside them).
 *  - `stream` arguments are hipStream_t values passed as void*; NULL is the
 *    null stream.  Work is enqueued, never waited for, unless stated.
 *  - Row-major layouts: a weight "[N, K]" has row n at offset n*K elements.
 *    bf16 values are raw 16-bit patterns; MXFP4 is OCP MX v1.0: codes
 *    u8 [N, K/2] (element 2b in the low nibble of byte b, 2b+1 in the high
 *    nibble) plus e8m0 scales u8 [N, K/32] (value 2^(s-127)).
 */
#ifndef LPS_H
#define LPS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status ------------------------------------------------------------- */
enum {
  LPS_OK = 0,
  LPS_EINVAL = -1,  /* a bad argument (null pointer, shape, dtype, plan) */
  LPS_ERANGE = -2,  /* an index or size outside what the objects allow */
  LPS_ESTATE = -3,  /* a call out of protocol order (e.g. recv of an unsent step) */
  LPS_EHIP = -4,    /* a HIP runtime call failed; the text names it */
  LPS_ENOMEM = -5,  /* a host-side allocation for a handle failed */
  LPS_EUNSUP = -6   /* a combination this build does not implement */
};

/* Text of the last failure on this thread ("" when none). */
const char* lps_last_error(void);

/* Library version string; never fails. */
const char* lps_version(void);

/* ---- dtypes and epilogue modes ----------------------------------------- */
enum { LPS_F32 = 0, LPS_BF16 = 1, LPS_MXFP4 = 2 };
enum { LPS_EPI_STORE = 0, LPS_EPI_ADD = 1, LPS_EPI_SWIGLU = 2 };

/* ---- A1: stage plan (host only; needs no GPU) ------------------------------
 * memra `pp` module docs, header (stage map) and fn pp_cuts; ninfer "Multi-GPU:
 * layer pipeline stages", How it works (StagePlan, per-stage layer counts).
 *
 * lps_stage_plan: writes the fence [0, c1, .., cN-1, n_layers] (n_stages + 1
 * int32 into fence_out, host).  cuts == NULL with n_cuts == 0 selects the even
 * split cut_s = floor(s * n_layers / n_stages).  Explicit cuts must number
 * n_stages - 1, be strictly increasing and lie in (0, n_layers).  n_stages must
 * lie in [1, n_layers].  Any violation -> LPS_EINVAL (never a silent N = 1).
 */
int lps_stage_plan(int32_t n_layers, int32_t n_stages, const int32_t* cuts, int32_t n_cuts,
                   int32_t* fence_out);
/* Per-stage layer counts (each >= 1, summing to n_layers) -> fence. */
int lps_stage_plan_counts(int32_t n_layers, int32_t n_stages, const int32_t* counts,
                          int32_t* fence_out);
/* The stage s with fence[s] <= layer < fence[s+1] (>= 0), or a negative status
 * for an invalid fence or a layer outside [0, fence[n_stages]). (fn stage_of) */
int lps_stage_of(const int32_t* fence, int32_t n_stages, int32_t layer);

/* Memory-balancing split (host only): ninfer "Multi-GPU: layer pipeline
 * stages", How it works (solve_stage_plan: the most KV page groups every stage
 * can hold, then the least-full stage) and Verification (a brute-force partition
 * oracle).  Bytes, host arrays: stage_free[s] > 0 and stage_overhead[s] >= 0
 * (n_stages each: what the device has free and what the stage needs besides its
 * layers, e.g. the head on the head stage), layer_fixed[l] (weights and fixed
 * state) and layer_kv[l] (KV bytes per page group), n_layers each.  Every stage
 * holds the same number P of page groups of its own layers' KV; the split
 * maximises P (capped at max_groups, which a stage without KV layers reports),
 * then minimises the largest (overhead + fixed + P * kv) / free, then takes the
 * lexicographically smallest fence.  Writes fence_out (n_stages + 1 int32) and
 * *groups_out = P.  LPS_EINVAL on bad arguments, LPS_EUNSUP if no split holds
 * even the layers' fixed bytes. */
int lps_stage_solve(int32_t n_layers, int32_t n_stages, const int64_t* stage_free,
                    const int64_t* stage_overhead, const int64_t* layer_fixed,
                    const int64_t* layer_kv, int64_t max_groups, int32_t* fence_out,
                    int64_t* groups_out);

/* ---- A2-A9, A17: one decoder layer ----------------------------------------
 * The pre-norm block: h = RMSNorm(x)*g_attn; [q|k|v] = W_qkv h; RoPE on the
 * pairs (i, i+hd/2) of every q and k head at position pos; k, v stored at row
 * pos of this layer's caches; q head j attends kv head j / (nq/nkv) over rows
 * 0..pos; x += W_o o; h' = RMSNorm(x)*g_ffn; x += W_d (silu(W_g h') * W_u h')
 * with W_gu holding the ff gate rows and then the ff up rows.  (TP3 zero-padded
 * dummy heads plan, Geometry and Weight-padding design for the GQA map and the
 * padded-head layout; ninfer pipeline stages, Tensor parallelism: status, for
 * the gate-then-up row order.)
 * A layer with nq == 0 has no attention sublayer (the attention fields are then
 * ignored): an FFN-only block, as in the MoE layer stack.  ffn_kind LPS_FFN_MOE
 * replaces the dense FFN by the MoE FFN of *moe (its own norm gain; the dense
 * FFN fields are then ignored): x += MoE(RMSNorm(x)) as lps_moe_layer_decode
 * computes it (strata PR #3648, Problem and result: MoE layers whose sums cross
 * a stage; memra pp docs, header: any layer range is a stage).
 */
struct lps_moe_desc;
enum { LPS_FFN_DENSE = 0, LPS_FFN_MOE = 1 };
typedef struct lps_layer_desc {
  int32_t d;          /* n_embd */
  int32_t nq, nkv;    /* q heads, kv heads (nq % nkv == 0) */
  int32_t hd;         /* head dim (even; 64, 128, 256 supported) */
  int32_t ff;         /* FFN width */
  int32_t wdtype;     /* LPS_F32 | LPS_BF16 | LPS_MXFP4 for every matrix */
  int32_t kvdtype;    /* LPS_F32 | LPS_BF16 */
  int32_t ctx_max;    /* rows allocated per kv head in each cache */
  float eps;          /* RMSNorm epsilon */
  float rope_base;    /* RoPE base (theta_i = base^(-2i/hd)) */
  const float* g_attn;             /* (dev) [d] f32 */
  const void* w_qkv; const uint8_t* s_qkv;   /* (dev) [(nq+2nkv)hd, d] (+ scales) */
  const void* w_o;   const uint8_t* s_o;     /* (dev) [d, nq*hd] */
  const float* g_ffn;              /* (dev) [d] f32 */
  const void* w_gu;  const uint8_t* s_gu;    /* (dev) [2ff, d] gate rows, then up rows */
  const void* w_d;   const uint8_t* s_d;     /* (dev) [d, ff] */
  void* k_cache;     /* (dev) kvdtype, owned by this layer's stage.  LPS_F32:
                      * [nkv, ctx_max, hd].  LPS_BF16: 16-row tiles of 8-dim groups,
                      * [nkv, ctx_max/16, hd/8, 16, 8]: element (head j, row r, dim e) at
                      * ((j*(ctx_max/16) + r/16)*(hd/8) + e/8)*128 + (r%16)*8 + e%8 */
  void* v_cache;     /* (dev) LPS_F32: [nkv, ctx_max, hd].  LPS_BF16: 16-row tiles,
                      * transposed, [nkv, ctx_max/16, hd, 16]: element (j, r, e) at
                      * ((j*(ctx_max/16) + r/16)*hd + e)*16 + r%16.  (The bf16 layouts are
                      * the matrix-core operand order: a 16-row tile of K or V is one
                      * contiguous block.)  bf16 caches need ctx_max % 16 == 0 */
  const float* rope_cs;  /* (dev, optional) [ctx_max, hd/2, 2] f32: cos, sin of pos * theta_i
                          * (lps_rope_table); required by the device-position entry points */
  int32_t ffn_kind;      /* LPS_FFN_DENSE (0: g_ffn, w_gu, w_d, ff) | LPS_FFN_MOE (moe) */
  const struct lps_moe_desc* moe;   /* (host) LPS_FFN_MOE: the layer's MoE FFN; copied by
                                     * lps_model_create, read during the call otherwise */
} lps_layer_desc;

/* Scratch bytes lps_layer_forward needs for this layer (0 on invalid desc). */
size_t lps_layer_scratch_bytes(const lps_layer_desc* L);

/* One layer on `stream`: x (dev, [d] f32) is updated in place; pos in
 * [0, ctx_max) is a by-value position (no device scalar is read).  scratch
 * (dev) of at least lps_layer_scratch_bytes(L) bytes; its contents on entry do
 * not matter; it must not be used by another stream while this call's work
 * runs.  Scales (s_*) are required for LPS_MXFP4 and ignored otherwise.
 * MXFP4 needs d, nq*hd and ff to be multiples of 32; bf16 multiples of 8;
 * f32 multiples of 4. */
int lps_layer_forward(const lps_layer_desc* L, float* x, int32_t pos, void* scratch,
                      size_t scratch_bytes, void* stream);

/* ---- a model handle and the stage walk ----------------------------------- */
typedef struct lps_model lps_model;
/* Copies the n_layers descriptors, and the MoE descriptors they point at (the
 * device buffers they point at stay the caller's).  *out receives the handle. */
int lps_model_create(const lps_layer_desc* layers, int32_t n_layers, lps_model** out);
int lps_model_destroy(lps_model* m);
/* Max scratch over the model's layers. */
size_t lps_model_scratch_bytes(const lps_model* m);
/* Walks layers [fence[stage], fence[stage+1]) of the model on `stream` over x
 * (dev [d] f32, in place) at position pos.  The fence is validated (as
 * lps_stage_plan would produce) before anything is enqueued.  Bumps the
 * stage_walks counter.  (ninfer pipeline stages, How it works: run_staged.) */
int lps_stage_forward(const lps_model* m, const int32_t* fence, int32_t n_stages, int32_t stage,
                      float* x, int32_t pos, void* scratch, size_t scratch_bytes, void* stream);

/* lps_stage_forward without caller scratch, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  The layer scratch is a static device buffer inside the
 * library, 8 MiB, one per GPU, held until the process ends; its address is
 * looked up on the first call on each device.  Nothing is allocated and
 * nothing in it needs clearing (every scratch value is written before it is
 * read).  A model whose layers need more scratch than the buffer holds
 * (lps_model_scratch_bytes(m) > 8 MiB) is refused with LPS_ERANGE before
 * anything is enqueued.  Every call on one GPU shares that GPU's buffer: calls
 * whose work overlaps on one GPU (other streams, or other threads) race on it;
 * the caller keeps them ordered. */
int lps_stage_forward_static(const lps_model* m, const int32_t* fence, int32_t n_stages,
                             int32_t stage, float* x, int32_t pos, void* stream);

/* ---- chunked dense prefill through the stages -------------------------------
 * memra pp module docs (functions on the prime split: the chunked prompt walk
 * takes the same per-stage layer ranges as decode) and ninfer pipeline stages
 * (What is not covered yet: a prefill chunk runs through the stages in turn).
 * lps_stage_prefill walks layers [fence[stage], fence[stage+1]) over the T rows
 * of x (dev [T, d] f32, in place) at positions p0 .. p0 + T - 1: per layer the
 * rows' RMSNorm, the QKV, O, gate/up and down products as bf16 GEMMs on the
 * matrix cores (the normed rows, the attention output and the SwiGLU output
 * are rounded to bf16 as their inputs; f32 accumulation and residual), RoPE
 * from the layer's rope_cs table, the chunk's K and V rows appended to the
 * caches, and causal attention of row t over cache rows 0 .. p0 + t on the
 * matrix cores (q and the unnormalised softmax weights enter as bf16 operands,
 * a precision deviation from the plain softmax(S) V of the decode path; f32
 * accumulation, the softmax sum over the f32 weights).  Cache rows at or past
 * p0 + T are never used, whatever they hold.  Bumps the prefill_walks counter.
 * Needs bf16 weights and bf16 caches, 1, 2, 4 or 8 q heads per kv head,
 * d % 256 == 0, (nq + 2 nkv) hd % 256 == 0, nq hd % 128 == 0, ff % 128 == 0,
 * rope_cs, p0 + T <= ctx_max, and every operand of the chunk (T rows of bf16
 * activations, f32 QKV and residual rows; the weights) below 2 GiB, the reach of
 * the kernels' 32-bit offsets (LPS_EUNSUP / LPS_EINVAL / LPS_ERANGE otherwise,
 * before anything is enqueued).  scratch (dev) of at least
 * lps_prefill_scratch_bytes(m, T) bytes, contents irrelevant. */
size_t lps_prefill_scratch_bytes(const lps_model* m, int32_t T);
int lps_stage_prefill(const lps_model* m, const int32_t* fence, int32_t n_stages, int32_t stage,
                      float* x, int32_t T, int32_t p0, void* scratch, size_t scratch_bytes,
                      void* stream);
/* x rows (dev [T, d] f32) = E[tok[t]] for the T ids tok (dev int32), as lps_embed
 * (an id outside [0, vocab) writes a NaN row); 1 <= T <= 65535. */
int lps_embed_rows(const void* table, int32_t wdtype, int32_t vocab, int32_t d, const int32_t* tok,
                   int32_t T, float* x, void* stream);

/* ---- device-position walk, step state and whole-pass graphs ----------------
 * ninfer pipeline stages, How it works (StageLink): the small control values
 * the layers read (the position among them) travel as device data, and decode
 * captures the whole staged pass into one graph.  A replayed step can only
 * differ from the last through device memory, so these entry points read the
 * position from the device and advance it there.
 *
 * lps_stage_forward_dpos: lps_stage_forward with the position read on the
 * device from *pos_dev (dev int32, 4-byte aligned) by every kernel of the
 * walk.  Each walked layer needs its rope_cs table (lps_rope_table, uploaded
 * by the caller).  The kernels clamp the position into [0, ctx_max - 1], so a
 * stale value cannot address memory outside the caches; keeping it in range is
 * the caller's (lps_step_advance stops it at pos_limit).  Attention is launched
 * over all ctx_max rows' chunks and the chunks past the position exit at once. */
int lps_stage_forward_dpos(const lps_model* m, const int32_t* fence, int32_t n_stages,
                           int32_t stage, float* x, const int32_t* pos_dev, void* scratch,
                           size_t scratch_bytes, void* stream);

/* host_out (host) [n_pos, hd/2, 2] f32 = cos, sin of p * base^(-2i/hd) for
 * p < n_pos, i < hd/2: formed in double and rounded once, the same values the
 * by-value QKV launch uses at position p (so both walks agree bit for bit).
 * Errors: LPS_EINVAL for a null output, odd or non-positive hd, n_pos < 1 or a
 * non-positive base.  Host only. */
int lps_rope_table(int32_t hd, float rope_base, int32_t n_pos, float* host_out);

/* Advances a decode step's device state, on `stream`, after the head wrote
 * this step's argmax (models without a vocabulary pass argmax = tok_cur = NULL,
 * n_feed 0 and no histories: only the position and the step advance).  state (dev int32 [3]): [0] position, [1] step, [2] flags
 * (bit 0: the position reached pos_limit - 1 and stayed there).  With s =
 * state[1]:
 *  - tok_hist[s] = *argmax when s < hist_cap (tok_hist dev, may be NULL when
 *    hist_cap is 0);
 *  - logits_hist[s * vocab ...] = logits[0 .. vocab) when logits_hist is not
 *    NULL and s < hist_cap (the copy precedes the advance in stream order);
 *  - *tok_cur = feed[s + 1] while s + 1 < n_feed (teacher-forced ids, dev),
 *    else *argmax: the next step's input token (read by lps_embed);
 *  - state[0] += 1 unless that reaches pos_limit (then flag bit 0); state[1] += 1.
 * Errors: LPS_EINVAL for null required pointers, pos_limit < 1 or
 * inconsistent feed / history arguments. */
int lps_step_advance(int32_t* state, int32_t pos_limit, const int32_t* argmax, int32_t* tok_cur,
                     const int32_t* feed, int32_t n_feed, int32_t* tok_hist, int32_t hist_cap,
                     const float* logits, int32_t vocab, float* logits_hist, void* stream);

/* The hidden-row input and output of a replayed step for models without a
 * vocabulary: with s = state[1] (dev int32, the step of lps_step_advance)
 * clamped into [0, n_rows - 1], dst[s * dst_stride + i] = src[s * src_stride + i]
 * for i < n, on `stream` (all dev f32).  A stride of 0 pins that side: src rows
 * [n_rows, src_stride] -> the stage-0 hidden (dst_stride 0) before the walk; the
 * last stage's hidden (src_stride 0) -> output rows after it.  Errors: LPS_EINVAL
 * for null pointers, n or n_rows < 1, or a nonzero stride below n. */
int lps_row_at_step(const int32_t* state, const float* src, int64_t src_stride, float* dst,
                    int64_t dst_stride, int32_t n, int32_t n_rows, void* stream);

/* Whole-pass graph capture.  lps_graph_begin starts a relaxed-mode capture on
 * `stream` (not the null stream; LPS_ESTATE while a kernel timer runs or the
 * stream already captures).  Everything then enqueued on it, and on every
 * stream that joins through an event (a boundary receive on another stream
 * joins it), is recorded rather than run.  lps_graph_end joins each stream of
 * `join` (host array of n_join streams; streams that never joined are skipped)
 * back into `stream`, ends the capture, and instantiates the graph into *out.
 * It always ends the capture, also when a captured call failed (it then
 * returns that failure's status and *out = NULL).
 * Boundaries in a capture: a wait targets only a record made in the same
 * context (eager, or that capture).  Ordering eager work against a graph
 * launch, in either direction, is the caller's (e.g. a stream or device
 * synchronize between them).
 * lps_graph_launch enqueues one replay on `stream`; replays on one stream run
 * one after the other.  lps_graph_destroy frees the graph (NULL is a no-op). */
typedef struct lps_graph lps_graph;
int lps_graph_begin(void* stream);
int lps_graph_end(void* stream, void* const* join, int32_t n_join, lps_graph** out);
int lps_graph_launch(lps_graph* g, void* stream);
int lps_graph_destroy(lps_graph* g);

/* ---- A2: embedding gather ------------------------------------------------
 * x[0..d) = E[*tok] widened to f32; tok (dev int32) is read on the device so a
 * previous step's argmax can feed it.  table (dev) [vocab, d] of wdtype
 * (LPS_F32 | LPS_BF16).  A token outside [0, vocab) writes NaN into x (the
 * host cannot see the device token; the NaN poisons the step loudly). */
int lps_embed(const void* table, int32_t wdtype, int32_t vocab, int32_t d, const int32_t* tok,
              float* x, void* stream);

/* ---- A15, A16: final RMSNorm + LM head + argmax --------------------------
 * logits (dev [vocab] f32) = W_lm (RMSNorm(x) * g_out); *tok_out (dev int32) =
 * the lowest index of the maximum logit.  Logits holding a NaN have no maximum:
 * *tok_out = vocab, an id outside the table, which lps_embed turns into a NaN
 * row, so a poisoned step poisons the next one instead of feeding a valid id.
 * memra pp docs: output_norm and the LM head live with the last stage. */
typedef struct lps_head_desc {
  int32_t d, vocab, wdtype;  /* wdtype LPS_F32 | LPS_BF16 */
  float eps;
  const float* g_out;        /* (dev) [d] */
  const void* w_lm;          /* (dev) [vocab, d] */
} lps_head_desc;
size_t lps_head_scratch_bytes(const lps_head_desc* h);
int lps_head_forward(const lps_head_desc* h, const float* x, float* logits, int32_t* tok_out,
                     void* scratch, size_t scratch_bytes, void* stream);
/* The end of a replayed greedy step (ninfer "Multi-GPU: layer pipeline stages", How
 * it works: the whole pass as one replayed graph) in three launches instead of
 * lps_head_forward, lps_step_advance and the next step's lps_embed: the final
 * RMSNorm and LM head into logits (dev [vocab] f32) as lps_head_forward; with
 * s = state[1] (dev), the logits copied to logits_hist[s * vocab ..] when
 * logits_hist is given and s < hist_cap; then one launch takes the lowest-index
 * argmax (vocab when no finite maximum), stores it to tok_hist[s] (s < hist_cap),
 * picks the next input id (feed[s + 1] while fed ids remain, else the argmax; to
 * *tok_cur when tok_cur is not NULL), writes that id's row of the embedding table
 * (dev, h->vocab rows of h->d values of embed_dtype, LPS_F32 or LPS_BF16; a NaN row
 * for an id outside it, as lps_embed) to x_next (dev [d] f32; may be x, which the
 * head has read by then), and advances
 * the position (unless it would reach pos_limit: flag bit 0 of state[2]) and the
 * step.  A run seeds x_next with lps_embed before its first replay.
 * ring (may be NULL): the step's own kernels also store its logits to
 * ring->logits[(s % slots) * vocab ..] and its argmax to ring->tok[s % slots]
 * (see lps_host_ring), so a replayed step is read back without a copy on another
 * stream.  Errors as lps_head_forward and lps_step_advance (LPS_EINVAL), also for
 * a ring with slots < 1, with neither row, or rows that are not pinned host memory. */
/* A pinned host ring the replayed step writes into (memra pp docs, struct
 * PendingLogits: the step's logits reach the host later, without blocking it;
 * ninfer pipeline stages, How it works: StageLink's ring of pinned host slots).
 * Rows are host memory the device addresses (pinned: hipHostMalloc, a pinned
 * tensor); logits [slots, vocab] f32 and tok [slots] int32, either may be NULL.
 * Step s's row is visible to the host once a pending marked after the step
 * (lps_pending_mark on the step's stream) has been waited; the caller waits step
 * s before it launches step s + slots, which reuses the row. */
typedef struct lps_host_ring {
  float* logits;
  int32_t* tok;
  int32_t slots;
} lps_host_ring;
int lps_step_finish(const lps_head_desc* h, const float* x, float* logits, int32_t* state,
                    int32_t pos_limit, const int32_t* feed, int32_t n_feed, int32_t* tok_hist,
                    float* logits_hist, int32_t hist_cap, const void* embed, int32_t embed_dtype,
                    float* x_next, int32_t* tok_cur, const lps_host_ring* ring, void* scratch,
                    size_t scratch_bytes, void* stream);

/* ---- step-level entry points (the pieces lps_layer_forward launches) ------ */
/* A3: y = x / sqrt(mean(x^2) + eps) * g, all (dev) [d] f32. */
int lps_rmsnorm(const float* x, const float* g, float eps, int32_t d, float* y, void* stream);
/* A4/A7/A8/A9/A17: y = W x' with x' = RMSNorm(x)*norm_g when norm_g != NULL, else x.
 *  mode LPS_EPI_STORE:  y[n] = (W x')[n], n < N
 *  mode LPS_EPI_ADD:    y[n] += (W x')[n]          (the residual add)
 *  mode LPS_EPI_SWIGLU: y[i] = silu(r_i) * r_{N/2+i}, i < N/2, r = W x' (N even)
 * W (dev) [N, K] of wdtype, s (dev) its e8m0 scales for LPS_MXFP4.  x (dev)
 * [K] f32.  The K tail is handled per 32-value group for MXFP4 (no read past a
 * row's end whatever K % 128 is: TP3 plan, Implementation status, item 1).
 * MXFP4 rows meet x' as an f16 operand (rounded once to nearest; f32
 * accumulation), f32 and bf16 rows meet it in f32.  MXFP4 K is at most 24576
 * (LPS_EUNSUP beyond). */
int lps_gemv(int32_t wdtype, const void* w, const uint8_t* s, int32_t N, int32_t K,
             const float* x, const float* norm_g, float eps, float* y, int32_t mode, void* stream);
/* A3+A4+A5: q (dev [nq*hd] f32) = RoPE(W_q h); RoPE(W_k h) and W_v h are written
 * to row pos of the layer's caches; h = RMSNorm(x)*g_attn.  Uses the layer desc's
 * shapes, weights and caches. */
int lps_qkv_rope_append(const lps_layer_desc* L, const float* x, int32_t pos, float* q,
                        void* stream);
/* A6: o (dev [nq*hd] f32) = softmax(q K^T / sqrt(hd)) V per q head over cache
 * rows 0..n_rows-1 of kv head j/(nq/nkv).  Caches (dev) in the layouts of
 * lps_layer_desc.k_cache / v_cache (16-row tiles for LPS_BF16, which also needs
 * ctx_max % 16 == 0).  Rows at or past n_rows are never used, whatever they
 * hold.
 * scratch (dev) of lps_attention_scratch_bytes(nq, nkv, hd, ctx_max) bytes. */
size_t lps_attention_scratch_bytes(int32_t nq, int32_t nkv, int32_t hd, int32_t ctx_max);
int lps_attention_decode(int32_t nq, int32_t nkv, int32_t hd, int32_t kvdtype,
                         const void* k_cache, const void* v_cache, int32_t ctx_max,
                         int32_t n_rows, const float* q, float* o, void* scratch,
                         size_t scratch_bytes, void* stream);

/* ---- A14: boundary slots -------------------------------------------------
 * memra pp docs, header: each boundary runtime has TWO persistent
 * double-buffered slots with ev_tx / ev_rx per slot; fn pp2_overlap: the slots
 * alternate per step.  Slot k = step & 1.
 *  send(step t): the producer stream waits ev_rx[k] (slot k drained by the
 *    recv of step t-2) and copies x -> slot[k].  When that recv ran on its own
 *    producer's stream (no event was recorded then) and this send comes from
 *    another stream, ev_rx[k] is recorded first on the receiving stream.
 *  recv(step t): ev_tx[k] is recorded on the producer stream (after the send's
 *    copy and whatever the host enqueued there since), the consumer stream waits
 *    it, copies slot[k] -> x and records ev_rx[k].
 * When producer and consumer are the same stream (memra pp docs, fn
 * pp2_streams_off: the same-stream seam), stream order already gives both
 * orderings and no event is recorded or waited for that step.
 * Steps must be sent in order 0, 1, 2, ... and received in the same order;
 * a recv of a step that was not sent, or out of order, is LPS_ESTATE.
 * The two slots (dev [n_elems] f32 each) are the caller's. */
typedef struct lps_boundary lps_boundary;
int lps_boundary_create(int32_t n_elems, float* slot0, float* slot1, lps_boundary** out);
int lps_boundary_send(lps_boundary* b, const float* x, int64_t step, void* producer);
int lps_boundary_recv(lps_boundary* b, float* x, int64_t step, void* consumer);
/* The same-stream seam in one call: send(step) and recv(step) with producer ==
 * consumer == `stream`, as one kernel that writes slot[step & 1] and x_out (dev
 * [n_elems] f32) from x; the same order rules (step must be the next send and the
 * next receive), the same waits (for an earlier receive of that slot on another
 * stream) and counters (a send and a receive) as the two calls. */
int lps_boundary_hop(lps_boundary* b, const float* x, float* x_out, int64_t step, void* stream);
/* lps_stage_forward_dpos of `stage` followed by lps_boundary_hop(b, x, x_out, step,
 * stream), with the hop's copy folded into the stage's last launch (the down
 * projection's residual add, or the MoE combine): it stores every updated row of x
 * also to slot[step & 1] and to x_out, so no copy launch follows.  The same
 * checks as the two calls (the boundary's rows must be the stage's d values,
 * LPS_EINVAL otherwise), the same order rules, waits and counters as the hop
 * (ninfer pipeline stages, How it works: StageLink; memra pp docs, header: the
 * boundary slots and their events). */
int lps_stage_forward_dpos_hop(const lps_model* m, const int32_t* fence, int32_t n_stages,
                               int32_t stage, float* x, const int32_t* pos_dev, void* scratch,
                               size_t scratch_bytes, lps_boundary* b, float* x_out, int64_t step,
                               void* stream);
/* Synchronizes the boundary's events, then frees the handle. */
int lps_boundary_destroy(lps_boundary* b);

/* Achievable HBM read bandwidth, the calibration of every GB/s figure (TP3
 * zero-padded dummy heads plan, File-level changes (AR work) and AR phasing &
 * gates: a bandwidth microbenchmark is run before anything is tuned on it): reads
 * `bytes` (a positive
 * multiple of 16) at `src` (dev, 16-byte aligned) once, with the GEMVs' load
 * pattern, on `stream`.  sink (dev, LPS_STREAM_SINK uint32) receives per-block
 * XOR folds of the 32-bit words: their XOR is the XOR of the whole buffer.
 * Errors: LPS_EINVAL on null / unaligned pointers or a bad size. */
#define LPS_STREAM_SINK 2048
int lps_hbm_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);

/* A copy of n f32 values on `stream` (the slot transport, also usable alone). */
int lps_copy_f32(const float* src, float* dst, int64_t n, void* stream);

/* ---- A16: deferred logits readback ----------------------------------------
 * memra pp docs, struct PendingLogits: a step's logits stay on the device with
 * a completion event; wait() orders a dedicated readback stream behind it,
 * copies and synchronizes; dropping without waiting is safe.
 * lps_logits_defer records a completion event on `last_stage`, makes
 * `readback` wait it, enqueues the D2H copies of logits (dev [vocab] f32,
 * may be NULL) and *tok (dev int32, may be NULL) into host_logits / host_tok
 * (host; pinned for a truly asynchronous copy), and records a drained event.
 * The caller must not overwrite the device buffers until the pending is
 * drained: lps_pending_order(p, stream) makes `stream` wait the drained event.
 * *out is an opaque token, not an address: exactly one lps_pending_wait or
 * lps_pending_drop consumes it; any later use of the token (a second wait, a
 * drop after a wait, an order after either), or a token the library never
 * issued, is LPS_ESTATE (memra pp docs, fn pp_multi_stream_same_device: refuse
 * loudly rather than return silently-wrong logits).
 */
typedef struct lps_pending lps_pending;
int lps_logits_defer(const float* logits, const int32_t* tok, int32_t vocab, void* last_stage,
                     void* readback, float* host_logits, int32_t* host_tok, lps_pending** out);
/* A pending for everything enqueued on `stream` so far (an event with the
 * system-scope fence that makes the device's stores to host memory visible),
 * e.g. a replayed step whose kernels wrote an lps_host_ring: lps_pending_wait
 * then blocks until those rows are on the host.  Consumed and refused as the
 * pendings of lps_logits_defer. */
int lps_pending_mark(void* stream, lps_pending** out);
/* Makes `stream` wait until the pending's copies are done (no host block). */
int lps_pending_order(lps_pending* p, void* stream);
/* Blocks the host until host_logits / host_tok hold the step; consumes p. */
int lps_pending_wait(lps_pending* p);
/* Consumes p without waiting: its copies still complete on the readback
 * stream; the events are released once they have fired. */
int lps_pending_drop(lps_pending* p);

/* ---- A10-A12: MoE FFN layer ------------------------------------------------
 * strata PR #3648 (Problem and result; Approach): per-token sums of the
 * "remote" half of the experts travel as FP16, converted back exactly in
 * pieces; the combine adds in a fixed order and may write over an input.
 * Layer: h = RMSNorm(x)*g_ffn; router r = W_r h; pi = softmax(r); top_k by pi
 * (ties to the lower id), listed by descending pi; w = pi_sel / sum pi_sel;
 * e_j = W_d,j (silu(W_g,j h) * W_u,j h); local = sum of w_j e_j over selected
 * j < remote_from in ascending j; remote likewise over j >= remote_from;
 * shared = the shared expert's output; x += (shared + local) + f32(f16(remote)).
 */
typedef struct lps_moe_desc {
  int32_t d, n_experts, top_k, ff, remote_from;
  float eps;
  const float* g_ffn;    /* (dev) [d] f32 */
  const void* w_r;       /* (dev) [E, d] bf16 */
  const void* w_gu_e;    /* (dev) [E, 2ff, d] bf16: per expert gate rows then up rows */
  const void* w_d_e;     /* (dev) [E, d, ff] bf16 */
  const void* w_gu_s;    /* (dev) [2ff, d] bf16, the shared expert */
  const void* w_d_s;     /* (dev) [d, ff] bf16 */
} lps_moe_desc;

/* A10: for T rows of x (dev [T, d] f32): idx (dev [T, top_k] int32), w (dev
 * [T, top_k] f32).  top_k <= 16, n_experts <= 256, d <= 4096.  scratch (dev) of
 * lps_moe_route_scratch_bytes(m, T) bytes receives the router logits [T, E]. */
size_t lps_moe_route_scratch_bytes(const lps_moe_desc* m, int32_t T);
int lps_moe_route(const lps_moe_desc* m, const float* x, int32_t T, int32_t* idx, float* w,
                  void* scratch, size_t scratch_bytes, void* stream);
/* A12: out (dev [T, d]) = f32(x + ((shared + local) + bo)) where bo (dev [T, d]
 * f32) first receives f32(remote16), converted piece by piece on `s_remote`:
 * piece p covers rows [floor(pT/P), floor((p+1)T/P)); `s_remote` first waits
 * for the work already enqueued on `s_main`, and `s_main` waits an event
 * recorded after the last piece before it combines.  remote16 (dev [T, d])
 * holds f16 bit patterns.  out may be the same buffer as bo or as x (each
 * element is read before it is written, by the same thread); bo must not
 * overlap shared, local or remote16.  Bumps the pieces counter. */
int lps_moe_combine(float* out, const float* x, const float* shared, const float* local,
                    const uint16_t* remote16, float* bo, int32_t T, int32_t d, int32_t n_pieces,
                    void* s_remote, void* s_main);
/* f32 -> f16 bits (round to nearest even) of n values: the remote half's
 * "sums_to_f16" step (strata PR #3648, Approach: sums). */
int lps_f32_to_f16(const float* src, uint16_t* dst, int64_t n, void* stream);
/* A13: one whole MoE layer over a prefill chunk of T tokens; x (dev [T, d] f32)
 * is updated in place.  Route (as above) per token; group the (token, expert)
 * pairs per expert in token order (a stable counting sort); run the experts as
 * grouped GEMMs on the bf16 matrix cores: the normed rows and the SwiGLU output
 * are rounded to bf16 as matrix inputs, accumulation is f32; the shared expert
 * is one more group over all T rows; per token, the gate-weighted expert terms
 * are added in ascending expert id within each half, the remote half rounded to
 * f16 and widened back in n_pieces pieces on s_remote, and x += (shared + local)
 * + remote (lps_moe_combine).  The activation half of the piece transfer
 * (strata PR #3648, Approach: activations): as soon as the rows are normed, their
 * bf16 copy goes to the remote half's own buffer in n_pieces row pieces on
 * s_remote while s_main routes and groups; the remote experts' grouped GEMMs then
 * run on s_remote from that copy once the tile lists exist, the local experts and
 * the shared one on s_main, which waits for the remote experts before the
 * per-token halves.  Both halves read the same values, so every n_pieces (1..64)
 * gives the same bits.  Bumps act_pieces (and pieces, in the combine).  Built for
 * n_experts <= 64, top_k <= 16, d a multiple of 128, ff a multiple of 64, and
 * every operand below 2 GiB, the reach of the kernels' 32-bit offsets (e.g. T
 * <= 32767 at d 2048, top 8: the per-slot expert outputs [T, top_k, d] f32);
 * LPS_EUNSUP otherwise, before anything is enqueued.
 * scratch (dev) of lps_moe_prefill_scratch_bytes(m, T) bytes; its contents on
 * entry do not matter.  Work is enqueued on s_main and s_remote. */
size_t lps_moe_prefill_scratch_bytes(const lps_moe_desc* m, int32_t T);
int lps_moe_prefill(const lps_moe_desc* m, float* x, int32_t T, int32_t n_pieces, void* scratch,
                    size_t scratch_bytes, void* s_main, void* s_remote);
/* One whole MoE layer for one token (decode): x (dev [d]) updated in place:
 * route, the selected experts' and the shared expert's gate/up + SwiGLU and down
 * GEMVs, the ordered local / remote (f16) combine.  d a multiple of 8, at most
 * 4096 (LPS_EUNSUP otherwise). */
size_t lps_moe_layer_scratch_bytes(const lps_moe_desc* m);
int lps_moe_layer_decode(const lps_moe_desc* m, float* x, void* scratch, size_t scratch_bytes,
                         void* stream);

/* ---- liveness counters ------------------------------------------------------
 * memra pp docs, Statics (PRIME_SPLIT_CHUNKS and friends): counters that prove
 * the staged walker ran, so that bit-identity gates cannot pass vacuously.
 * Process-wide, bumped at enqueue time. */
typedef struct lps_counters_t {
  int64_t stage_walks;     /* lps_stage_forward calls that enqueued work */
  int64_t boundary_sends;
  int64_t boundary_recvs;
  int64_t pieces;          /* FP16 pieces converted by lps_moe_combine */
  int64_t drains;          /* pendings waited or dropped */
  int64_t prefill_walks;   /* lps_stage_prefill calls that enqueued work */
  int64_t act_pieces;      /* activation row pieces sent to the remote half by lps_moe_prefill */
} lps_counters_t;
int lps_counters(lps_counters_t* out);
int lps_counters_reset(void);

/* ---- kernel timing (benchmarks) -------------------------------------------
 * While a timer runs, every launch of the chosen kind made by lps_layer_forward,
 * lps_stage_forward, lps_head_forward, lps_moe_layer_decode or lps_moe_prefill
 * carries a pair of hipEvents that the
 * dispatch itself stamps at its start and end (hipExtLaunchKernelGGL), so the
 * durations are those of the kernels on their stream, without launch gaps.
 * capacity bounds the pairs recorded (later launches are not timed).  One timer
 * at a time per process. */
enum {
  LPS_KIND_QKV = 1,     /* RMSNorm + QKV GEMV + RoPE + KV append */
  LPS_KIND_ATTN = 2,    /* decode attention incl. the chunk merge */
  LPS_KIND_OPROJ = 3,   /* O projection + residual */
  LPS_KIND_GATEUP = 4,  /* RMSNorm + gate/up GEMV + SwiGLU */
  LPS_KIND_DOWN = 5,    /* down projection + residual */
  LPS_KIND_HEAD = 6,    /* final RMSNorm + LM head + argmax */
  LPS_KIND_MOE_GU = 7,  /* MoE decode: RMSNorm + the selected and shared experts' gate/up + SwiGLU */
  LPS_KIND_MOE_DOWN = 8,   /* MoE decode: every slot's down projection */
  LPS_KIND_MOE_GEMM1 = 9,  /* MoE prefill: grouped gate/up GEMM + SwiGLU (each half's launch) */
  LPS_KIND_MOE_GEMM2 = 10  /* MoE prefill: grouped down GEMM (each half's launch) */
};
int lps_timer_start(int32_t kind, int32_t capacity);
/* Synchronizes the recorded events, writes up to cap durations (milliseconds)
 * to ms_out (host) and their count to *n_out, and stops the timer. */
int lps_timer_stop(float* ms_out, int32_t cap, int32_t* n_out);

#ifdef __cplusplus
}
#endif
#endif /* LPS_H */
