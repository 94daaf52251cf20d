/*
 * jev.h -- C ABI of the shared-prefix, prefill-only branch scorer (MI355X, gfx950).
 *
 * The method (jdon.com openjev-sglang article, "inference flow" and
 * "prefill-only" sections; LLM2Jev shared-prefix page): a shared token prefix is
 * prefilled once into a paged KV cache; every branch (question / candidate)
 * continues from that prefix and computes only its own suffix tokens, attending
 * to the cached prefix pages plus its own causal suffix; only the last
 * position's logits at the requested candidate label ids are read and they are
 * renormalised with a max-subtracted softmax over the labels.  No token is
 * decoded.  Candidate sets given as full sequences are grouped by token prefix
 * and submitted in staged rounds (LLM2Jev shared-prefix page, staged-submission
 * section), each candidate scored exactly once and returned in input order.
 *
 * Conventions for every entry point:
 *  - Return value: JEV_OK (0) or a JEV_E* status.  jev_last_error() returns a
 *    thread-local message for the last failure of the calling thread.
 *  - Everything is validated before any device work is queued; a call that
 *    fails leaves the context unchanged (no pages taken, no handle created),
 *    except JEV_EHIP, after which the context is unusable (every later call
 *    returns JEV_EHIP).
 *  - Host arrays (tokens, offsets, labels, parents, handles) are read during
 *    the call only; the library keeps its own copies.
 *  - Device work is queued on the given HIP stream (NULL = default stream) and
 *    is asynchronous: device outputs are valid once that stream has reached
 *    the end of the call.  Calls on one context must not overlap (the context
 *    is not thread-safe); a call on a different stream than the previous one is
 *    ordered after the previous call's device work by the library.
 *  - Device buffers (weights, KV pool, workspace, outputs) are owned by the
 *    caller and must outlive the context.  The library owns only host state.
 */
#ifndef JEV_H
#define JEV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  JEV_OK = 0,
  JEV_EINVAL = 1,  /* bad argument: shapes, ids, offsets, label count, empty suffix */
  JEV_ENOMEM = 2,  /* not enough free KV pages or workspace for the whole call */
  JEV_EHANDLE = 3, /* unknown or already released prefix handle */
  JEV_EHIP = 4,    /* a HIP call failed; the context is dead */
  JEV_ESTATE = 5,  /* operation not available on this context (e.g. device work on a planning-only context) */
  JEV_EPENDING = 6 /* a scheduled request has not finished yet */
};

enum { JEV_DTYPE_F32 = 0, JEV_DTYPE_BF16 = 1 };

/* Tokens per KV page. */
#define JEV_PAGE_TOKENS 16
/* Label count bounds per branch (jdon.com article, limits section: 2..64 options). */
#define JEV_MIN_LABELS 2
#define JEV_MAX_LABELS 64

typedef int64_t jev_prefix; /* resident prefix handle; 0 = the empty prefix */
typedef struct jev_ctx jev_ctx;

/* Model shape.  Attention-only pre-norm stack:
 *   x = E[token]; per layer: h = RMSNorm(x) * g_l; q,k,v = h Wq^T, h Wk^T, h Wv^T;
 *   RoPE(q, k) at the logical position (rotate-half pairs (i, i+dh/2),
 *   inverse frequency theta^(-2i/dh)); causal attention with KV head
 *   floor(j / (Hq/Hkv)) for query head j, scale 1/sqrt(dh); x += o Wo^T;
 *   final: RMSNorm(x) * g_f, logits = . U^T.
 * bf16 models store activations in bf16 at: norm outputs, q/k after RoPE, v,
 * attention output, residual stream, final-norm output; accumulation is fp32. */
typedef struct {
  int32_t n_layers;
  int32_t d_model;
  int32_t n_q_heads;
  int32_t n_kv_heads;       /* divides n_q_heads; n_q_heads/n_kv_heads divides 128 */
  int32_t head_dim;         /* 64 or 128 */
  int32_t vocab;
  int32_t dtype;            /* JEV_DTYPE_F32 or JEV_DTYPE_BF16: weights, activations, KV pages */
  float rope_theta;
  float rms_eps;
  int32_t max_positions;    /* longest sequence (prefix + suffix) the context will see, <= 65536 */
  int32_t max_round_tokens; /* most new tokens computed in one round (sizes the activations) */
} jev_model_desc;

/* Device pointers to the weights, row-major, all of the model's dtype.
 * Matrices are [out][in]: embed/unembed [vocab][d], wq [Hq*dh][d],
 * wk/wv [Hkv*dh][d], wo [d][Hq*dh]; norms [d].  The per-layer members are host
 * arrays of n_layers device pointers (copied at create). */
typedef struct {
  const void* embed;
  const void* unembed;
  const void* final_norm;
  const void* const* attn_norm;
  const void* const* wq;
  const void* const* wk;
  const void* const* wv;
  const void* const* wo;
} jev_weights;

/* Bytes of device workspace jev_create needs for this model (activations for
 * max_round_tokens rows, LSE partial states, RoPE table, call descriptors). */
size_t jev_workspace_bytes(const jev_model_desc* desc);

/* Bytes of a KV pool of n_pages pages.  Layout, per element of the model dtype:
 * [layer][page][kv_head][K|V][16 * head_dim]; the K block of a page is
 * [slot][head_dim], the V block is [head_dim][slot] (transposed). */
size_t jev_kv_pool_bytes(const jev_model_desc* desc, int32_t n_pages);

/* Creates a context.  kv_pool: jev_kv_pool_bytes(desc, n_pages) bytes;
 * workspace: at least jev_workspace_bytes(desc) bytes, 256-byte aligned.
 * With weights == NULL, kv_pool == NULL and workspace == NULL the context is a
 * planning-only context: prefix/plan/page-table calls run on the host and
 * nothing touches a GPU (scoring calls return JEV_ESTATE).  n_pages in
 * [1, 2^26].
 * Errors: JEV_EINVAL (shape, n_pages), JEV_ENOMEM (workspace too small),
 * JEV_EHIP. */
int jev_create(const jev_model_desc* desc, const jev_weights* weights, void* kv_pool,
               int32_t n_pages, void* workspace, size_t workspace_bytes, jev_ctx** out);

/* Waits for the context's queued work and frees its host state. */
int jev_destroy(jev_ctx* ctx);

/* Prefills n prefixes (the "warm-up" prefill of the N+1 flow: jdon.com article,
 * N+1 section).  Prefix i continues resident prefix parents[i] (0 = none) with
 * tokens[offsets[i] .. offsets[i+1]) (host int32, offsets has n+1 entries,
 * offsets[0] = 0, every segment non-empty, ids in [0, vocab)).  All prefixes
 * are computed in one round.  A prefix identical to an existing child of the
 * same parent is not recomputed: its handle is returned with one more
 * reference.  out_handles[i] receives one caller reference each.
 * Errors: JEV_EINVAL, JEV_EHANDLE (unknown parent), JEV_ENOMEM (pages or
 * workspace for the whole call), JEV_EHIP. */
int jev_prefill_prefix(jev_ctx* ctx, int32_t n, const jev_prefix* parents, const int32_t* tokens,
                       const int64_t* offsets, jev_prefix* out_handles, void* hip_stream);

/* Scores n branches (jdon.com article, prefill-only section).  Branch i
 * continues resident prefix parents[i] with suffix tokens[tok_offsets[i] ..
 * tok_offsets[i+1]) (non-empty: the last scored position is always computed)
 * and reads the labels label_ids[label_offsets[i] .. label_offsets[i+1])
 * (host int32, 2..64 distinct ids in [0, vocab)).  probs (device float32,
 * label_offsets[n] entries) receives, per branch, the softmax over its labels
 * of the last position's logits, in label order.  Branch KV pages are taken for
 * the call and released when it ends.  Branches with the same parent share one
 * pass over the parent's pages.
 * Errors: JEV_EINVAL, JEV_EHANDLE, JEV_ENOMEM, JEV_EHIP, JEV_ESTATE. */
int jev_score_branches(jev_ctx* ctx, int32_t n, const jev_prefix* parents, const int32_t* tokens,
                       const int64_t* tok_offsets, const int32_t* label_ids,
                       const int64_t* label_offsets, float* probs, void* hip_stream);

/* jev_score_branches for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, results and errors; the kernels' scratch (the
 * attention partial states and the split-K partial tiles) lives in a 96 MiB
 * file-scope device array instead of the context's workspace, one copy per GPU
 * the library runs on, held until the process ends.  The call makes no
 * hipMalloc/hipFree and no allocating library call (profiling records of
 * jev_profile are not taken on this path).  A call whose round needs more
 * partial-state rows than the array holds fails with JEV_ENOMEM before
 * anything changes.  Every call on one GPU shares that GPU's array and finds
 * it as the previous call left it: calls that overlap on one GPU (contexts
 * driven on different streams at once) race. */
int jev_score_branches_noalloc(jev_ctx* ctx, int32_t n, const jev_prefix* parents, const int32_t* tokens,
                               const int64_t* tok_offsets, const int32_t* label_ids,
                               const int64_t* label_offsets, float* probs, void* hip_stream);

/* Scores n candidates given as full token sequences (LLM2Jev shared-prefix page,
 * staged-submission section).  Each candidate is matched against the resident
 * prefixes (longest full-node match leaving at least one token; where it leaves
 * a resident node inside it after at least one whole page, that node is split
 * at the last page boundary before the divergence and the candidate reuses the
 * pages before it (the split stays; the node's handle keeps the rest and still
 * names the whole prefix)), the rest are
 * grouped into a token-prefix tree and computed in staged rounds whose order
 * is the context's plan mode (jev_set_plan_mode); every candidate is read out
 * exactly once; probs as for jev_score_branches, in input order.  Pages of the
 * call's own tree nodes are released when it ends; with JEV_CACHE_LRU the
 * nodes its candidates share stay as cached prefixes instead (automatic
 * checkpoints of a repeated state, evicted least recently used first).
 * Errors: as jev_score_branches. */
int jev_score_candidates(jev_ctx* ctx, int32_t n, const int32_t* tokens, const int64_t* tok_offsets,
                         const int32_t* label_ids, const int64_t* label_offsets, float* probs,
                         void* hip_stream);

/* Round order of jev_score_candidates and jev_plan on this context (LLM2Jev
 * shared-prefix page, staged-submission section).
 *  JEV_PLAN_DEPTH (the default): round k computes every new tree node at depth
 *    k; a shared prefix is computed as a node of its own before the candidates
 *    that continue it.
 *  JEV_PLAN_CANDIDATE_FIRST: the page's own order.  Each round takes every node
 *    whose parent is already computed; a node without children is computed with
 *    all its candidates, while a shared node is built by one real candidate, its
 *    smallest index, whose path down to its own read-out is computed (and read
 *    out) in that round.  No candidate waits on a separate warmup node.
 * Both orders compute every node once.  Their probabilities agree to the
 * accumulation-order floor, not bitwise: a round of at most 256 tokens splits
 * the K dimension of its projections over workgroups and a larger round does
 * not, so a node's K/V can be summed in another order in another round.
 * Errors: JEV_EINVAL (NULL ctx, unknown mode). */
enum { JEV_PLAN_DEPTH = 0, JEV_PLAN_CANDIDATE_FIRST = 1 };
int jev_set_plan_mode(jev_ctx* ctx, int32_t mode);

/* Round-invariant numerics on this context (0 off, the default; 1 on).  By
 * default a token's values depend, within the accumulation-order floor, on
 * the round it is computed in: rounds of at most 256 rows split the
 * projections' K over workgroups and larger ones do not, and the number of
 * prefix chunks, the split of long causal tiles and the attention's wave
 * groups follow the round's occupancy.  With this on, every projection sums K
 * in the large rounds' order (no K split; the residual projection and the
 * next layer's norm as two kernels), prefix chunks are 32 pages (more when a
 * prefix would need over 8), long causal tiles are not split, and every round
 * splits each tile's steps over two wave groups: a token's K/V, attention
 * output and probabilities are then bitwise the same whichever round
 * computes it (both plan orders, any batch), at the cost of speed in rounds
 * of at most 256 rows.  Takes effect at the next call.
 * Errors: JEV_EINVAL (NULL ctx, on not 0 or 1). */
int jev_set_round_invariant(jev_ctx* ctx, int32_t on);

/* What happens to a prefix whose last caller reference is dropped
 * (openjev-multimodal performance page, repeated-state section: the KV at the
 * end of a state is kept for the next request that repeats it, and several
 * states can be kept and used in turn).
 *  JEV_CACHE_RELEASE (the default): its pages return to the pool at once
 *    (once it has no resident child either).
 *  JEV_CACHE_LRU: it stays resident as a cached prefix.  jev_prefill_prefix of
 *    the same segment under the same parent re-references it with no
 *    compute.  A call that is short of free pages evicts cached prefixes that
 *    have no resident children, least recently used first (ties: the smallest
 *    handle), never one on the path of a prefix the call uses; it fails with
 *    JEV_ENOMEM (evicting nothing) if that cannot make room.  An eviction made
 *    for a call stays even if the call then fails a later capacity check.  A
 *    prefix is used by a call that creates, re-references, scores under or
 *    releases a prefix on whose path it lies (jev_plan changes nothing; it
 *    reports the plan, evictions included, that scoring would run).
 * Setting JEV_CACHE_RELEASE evicts every cached prefix that can go.
 * Errors: JEV_EINVAL (NULL ctx, unknown policy). */
enum { JEV_CACHE_RELEASE = 0, JEV_CACHE_LRU = 1 };
int jev_set_cache_policy(jev_ctx* ctx, int32_t policy);

/* Drops one caller reference of each handle.  A prefix with no reference and
 * no resident child returns its pages to the pool (its parent may follow).
 * Pages are re-used only by later calls, which the library orders after the
 * device work that read them.  Errors: JEV_EHANDLE (nothing is released then). */
int jev_free_pages(jev_ctx* ctx, int32_t n, const jev_prefix* handles);

/* Host-only: the staged-round plan jev_score_candidates would execute now (in
 * the context's plan mode), serialised as int32: the round count; per round,
 * its node count and per node: id, parent id (-1: continues the resident
 * anchor), anchor handle, tree depth, smallest candidate index, segment start
 * (relative to the anchor), segment length, page count, the page ids, read-out
 * count, the read-out candidate indices; then the candidate count and per
 * candidate: anchor handle, tokens matched in the resident tree, id of its
 * read-out node.  out may be NULL to query *out_len.  Errors: JEV_EINVAL,
 * JEV_ENOMEM (pool too small for the plan; the plan is not returned). */
int jev_plan(jev_ctx* ctx, int32_t n, const int32_t* tokens, const int64_t* tok_offsets,
             int32_t* out, int64_t cap, int64_t* out_len);

/* Host-only: page ids and valid token counts of every page on the path from
 * the root to handle h (root first).  cap = room in page_ids/valid; *n gets the
 * count (also when cap is too small, with JEV_EINVAL). */
int jev_page_table(jev_ctx* ctx, jev_prefix h, int32_t* page_ids, int32_t* valid, int32_t cap,
                   int32_t* n);

/* Host-only: deepest resident prefix whose whole path is a prefix of tokens[0..n)
 * leaving at least one token; *matched = its length (0 and handle 0 if none). */
int jev_match(jev_ctx* ctx, const int32_t* tokens, int64_t n, jev_prefix* handle, int64_t* matched);

typedef struct {
  int64_t logical_tokens;   /* tokens of every scored sequence incl. cached prefix (last call) */
  int64_t computed_tokens;  /* tokens actually run through the model (last call) */
  int64_t cached_tokens;    /* logical - computed (last call) */
  int32_t rounds;           /* rounds of the last call */
  int32_t pages_in_use;
  int32_t pages_total;
  int32_t resident_prefixes;  /* resident prefixes, cached ones included */
  int64_t calls;
  int32_t cached_prefixes;    /* resident prefixes without caller references (cache policy) */
  int32_t cached_pages;       /* pages they hold (counted in pages_in_use) */
  int64_t evictions;          /* cached prefixes evicted so far */
  /* Timing of the last call that ran device work, split like the pages' server
   * timing (openjev-sglang article, response-header section: preparation,
   * shared prefill, branch inference; openjev-multimodal performance page,
   * server-side timing section). */
  int32_t last_call_kind;     /* JEV_CALL_* (JEV_CALL_NONE before the first such call) */
  uint32_t debug_flags;       /* jev_set_debug flags in force */
  int64_t last_prepare_ns;    /* host: call entry to its first enqueue (checks, matching, plan, descriptors) */
  int64_t last_enqueue_ns;    /* host: queueing its copies and kernels */
  double last_prefill_ms;     /* device: its rounds without read-outs (shared prefixes); with
                                 JEV_DEBUG_TIME_CALLS, else -1 */
  double last_branch_ms;      /* device: its rounds with read-outs (branch inference); with
                                 JEV_DEBUG_TIME_CALLS, else -1 */
} jev_stats_t;

enum { JEV_CALL_NONE = 0, JEV_CALL_PREFILL = 1, JEV_CALL_BRANCHES = 2, JEV_CALL_CANDIDATES = 3, JEV_CALL_SCHED_STEP = 4 };

/* Host-only statistics.  With JEV_DEBUG_TIME_CALLS the device times need the
 * last call's device work: jev_stats then waits for it.  Errors: JEV_EINVAL. */
int jev_stats(jev_ctx* ctx, jev_stats_t* out);

/* Debug modes (bit flags; 0 turns everything off):
 *  - JEV_DEBUG_POISON_FREED_PAGES: every KV page that a call (or
 *    jev_free_pages) leaves free after the call wrote or released it is filled
 *    with the byte 0x7F in every layer, on the call's stream after its kernels
 *    (jev_free_pages: the stream of the last call).  0x7F7F is a finite bf16
 *    (and 0x7F7F7F7F a finite fp32) near the type's maximum: masked key slots
 *    of a partly filled page still contribute exactly 0, while a kernel that
 *    reads a freed page as valid keys produces non-finite scores, so
 *    stale-page bugs show up as wrong (NaN) probabilities in any parity test.
 *    Costs one fill launch per call; results are unchanged.
 *  - JEV_DEBUG_TIME_CALLS: the device time of each call's rounds is recorded
 *    with events (two fence-free event records per round) for jev_stats.
 *  - JEV_DEBUG_FULL_LAST_LAYER: the last layer's attention and output
 *    projection run for every row of a round, as in the other layers.  By
 *    default (and unless a debug tap is registered) they run only for the rows
 *    whose final state is read out, or not at all in a round without
 *    read-outs: a prefill produces the KV cache at every position and the
 *    logits at the last one only (jdon.com article, prefill-only section), and
 *    nothing else reads a row's last-layer output.  A round's read-out rows
 *    get the tiles, chunks and wave groups they have in the whole round, so
 *    their probabilities are bitwise the same either way when the round has
 *    at most 256 rows (larger rounds project the whole round without a K
 *    split and the read-out rows with one: equal to the accumulation-order
 *    floor).
 * Errors: JEV_EINVAL (unknown bit, NULL ctx). */
enum { JEV_DEBUG_POISON_FREED_PAGES = 1, JEV_DEBUG_TIME_CALLS = 2, JEV_DEBUG_FULL_LAST_LAYER = 4 };
int jev_set_debug(jev_ctx* ctx, uint32_t flags);

/* Limits of a context (host-only; also on a planning-only context). */
typedef struct {
  int32_t page_tokens;          /* JEV_PAGE_TOKENS */
  int32_t min_labels;           /* JEV_MIN_LABELS */
  int32_t max_labels;           /* JEV_MAX_LABELS */
  int32_t max_positions;        /* longest sequence (prefix + suffix), from the model description */
  int32_t max_round_tokens;     /* most tokens computed in one round */
  int32_t n_pages;              /* KV pages of the pool */
  int32_t split_k_rows;         /* rounds of at most this many rows split the projections' K
                                   (0: none does, with round-invariant numerics) */
  int32_t max_tile_pages;       /* longest key list of one attention tile */
  int64_t noalloc_scratch_bytes;     /* static scratch of jev_score_branches_noalloc (per device) */
  int64_t noalloc_partial_rows;      /* attention partial-state rows it holds for this model (0: dry context) */
  int64_t workspace_partial_rows;    /* those the workspace holds */
} jev_limits_t;
int jev_limits(jev_ctx* ctx, jev_limits_t* out);

/* Projection kernel variants, for measurement (process-wide; 0 everywhere is
 * the default, which every call uses unless this is set).  Every variant
 * computes the same products (q/k/v with RoPE and page writes, the residual
 * projection) from the same bf16 operands with fp32 accumulation; a variant
 * can sum K in another order, so its probabilities agree with the default's
 * to the accumulation-order floor, not bitwise.
 *  large:  projections of rounds of more than 256 rows (bf16):
 *          0 = the default kernel (four MFMA waves fed by four loader waves
 *          that load straight into LDS, three stages), 1 = eight MFMA waves
 *          with register-staged loads, 2 / 3 = four MFMA waves loading
 *          straight into LDS themselves, two / three stages;
 *  splits: K splits of rounds of at most 256 rows (0 = as many as fill the
 *          CUs once, at most 6; else 1..8, capped by K / 128);
 *  bn:     column tile of the large projections (0 = automatic, 128, 160).
 * Set it only while no call is in flight; the next call uses it.
 * Errors: JEV_EINVAL (a value outside these ranges; nothing changes). */
int jev_set_gemm_variant(int32_t large, int32_t splits, int32_t bn);

/* Debug taps for parity tests.  Each call registers one tap (up to 16); a
 * NULL dst removes every tap.  what = JEV_TAP_ATTN: the attention output of
 * `layer` (after the log-sum-exp merge); what = JEV_TAP_RESID: the residual
 * stream entering `layer` (layer == n_layers: the stream entering the final
 * norm).  Rows are model-dtype [token][width] in the round's token order (nodes
 * grouped by parent, input order within a group); at most cap_rows rows are
 * copied to dst (device).  Taps apply to single-round calls only. */
enum { JEV_TAP_ATTN = 0, JEV_TAP_RESID = 1 };
int jev_debug_tap(jev_ctx* ctx, int32_t what, int32_t layer, void* dst, int64_t cap_rows);

/* Kernel timing for measurement.  While a kind is enabled (bit 1<<kind of the
 * mask), every launch of that kernel is bracketed by HIP events on the call's
 * stream and recorded with its algorithmic work: FLOPs for the contractions
 * (QKV and output projections: 2*M*N*K; attention: 4*head_dim per visible
 * query-key pair) and bytes for the memory-bound kernels (each input and
 * output element once).  jev_profile(ctx, 0) disables and clears the records.
 * jev_profile_read waits for the recorded events and copies up to cap records;
 * *n receives the number recorded.  jev_profile_rows is jev_profile restricted
 * to the launches of exactly `rows` token rows (rows = 0: every launch), so
 * that a measurement puts events on the launches it times and on no other
 * (an event pair costs the stream a short idle between kernels); errors:
 * JEV_EINVAL for rows < 0, otherwise those of jev_profile. */
enum {
  JEV_K_EMBED = 0,
  JEV_K_RMSNORM = 1,
  JEV_K_QKV = 2,
  JEV_K_ATTN = 3,
  JEV_K_MERGE = 4,
  JEV_K_OPROJ = 5,
  JEV_K_READOUT = 6,
  JEV_K_COUNT = 7
};
typedef struct {
  int32_t kind;
  int32_t layer;  /* -1 for per-round kernels */
  int64_t rows;   /* token rows (or readout items) of the launch */
  double flops;   /* algorithmic FLOPs (0 for memory-bound kernels) */
  double bytes;   /* algorithmic HBM bytes */
  float ms;       /* event-measured duration */
} jev_launch_record;
int jev_profile(jev_ctx* ctx, uint32_t kind_mask);
int jev_profile_rows(jev_ctx* ctx, uint32_t kind_mask, int64_t rows);
int jev_profile_read(jev_ctx* ctx, jev_launch_record* out, int64_t cap, int64_t* n);

/* Answer layer (jdon.com openjev-sglang article, "three question types" and
 * "confidence" sections), on the host.  Branch i's label distribution is
 * probs[label_offsets[i] .. label_offsets[i+1]) (host float32, K = 2..64
 * entries in label order, each finite and >= 0; offsets has n+1 entries,
 * offsets[0] = 0).  Per branch, with options numbered from 0:
 *   kinds[i] = JEV_ANSWER_NOUL:   value[i] = P(yes), the first label's probability;
 *   kinds[i] = JEV_ANSWER_CHOICE: value[i] = index of the largest probability
 *                                 (ties go to the lowest index);
 *   kinds[i] = JEV_ANSWER_SCORE:  value[i] = sum_j j * P_j.
 * choice[i] receives that argmax for every kind and confidence[i] receives
 * 1 - H(P) / ln K, H the Shannon entropy in natural log with 0 ln 0 = 0: 1 for
 * a one-hot P, 0 for the uniform one (a measure of concentration, not of
 * calibrated correctness).  value, choice and confidence are host arrays of n
 * entries; choice and confidence may be NULL.  Computed in double precision;
 * no context or device is involved.
 * Errors: JEV_EINVAL (n < 0, NULL probs/offsets/kinds/value, bad offsets,
 * K outside [2, 64], a negative or non-finite probability, unknown kind);
 * on error no output is written. */
enum { JEV_ANSWER_NOUL = 0, JEV_ANSWER_CHOICE = 1, JEV_ANSWER_SCORE = 2 };
int jev_answers(int32_t n, const float* probs, const int64_t* label_offsets, const int32_t* kinds, double* value,
                int32_t* choice, double* confidence);

/* ---------------------------------------------------------------------------
 * Round-level continuous batching of requests from many callers (shared-prefix
 * scoring article, "next steps" section: cross-request continuous batching
 * for throughput).  A request is a set of candidates as for
 * jev_score_candidates.  Callers on any thread submit requests; one driver
 * thread calls jev_sched_step.  Each step: the requests submitted since the
 * previous step join the active ones; the unfinished candidates of all active
 * requests (in submission order, then candidate order) are planned together
 * as one scoring call in depth rounds (shared prefixes across requests are
 * computed once, reuse inside resident prefixes and the cache policy as for
 * jev_score_candidates), and only the plan's first round runs.  That round's
 * nodes with children become resident prefixes held by the scheduler, so the
 * next step continues below them; candidates read out in the round are done.
 * Held prefixes that no unfinished candidate of a started request passes
 * through are then released.  Admission: jev_sched_submit refuses a request
 * that does not fit an empty pool of the context's size on its own
 * (JEV_ENOMEM); when a step's plan does not fit, the newest requests that have
 * not started yet wait for a later step, until it fits.  Every step therefore advances each active request by
 * one level of its candidate tree, and new requests join at their first level
 * in the same GPU round.  Probabilities equal those of scoring each request
 * alone, up to the rounding order of the bf16 kernels.
 *
 * The scheduler belongs to its context: make no other call on the context
 * while jev_sched_step runs.  Destroying the context first detaches its
 * schedulers (their requests are dropped): later calls on them fail with
 * JEV_ESTATE, jev_sched_status still answers, and jev_sched_destroy only frees
 * them.  Destroying a context while another thread uses one of its schedulers
 * is undefined. */
typedef struct jev_sched jev_sched;
enum { JEV_SCHED_QUEUED = 0, JEV_SCHED_ACTIVE = 1, JEV_SCHED_FINISHED = 2 };
int jev_sched_create(jev_ctx* ctx, jev_sched** out);
/* Waits for the context's last work, releases the held prefixes and frees the
 * scheduler; requests not collected are dropped. */
int jev_sched_destroy(jev_sched* s);
/* Thread-safe.  Queues a request of n >= 1 candidates (arguments as for
 * jev_score_candidates; copied, so the caller's arrays may be reused at once)
 * and returns its ticket.  Errors: JEV_EINVAL (as jev_score_candidates). */
int jev_sched_submit(jev_sched* s, int32_t n, const int32_t* tokens, const int64_t* tok_offsets,
                     const int32_t* label_ids, const int64_t* label_offsets, int64_t* ticket);
/* Runs one round on hip_stream (NULL: the default stream) and waits for it.
 * If plan_out is not NULL it receives the plan the round was taken from, in
 * jev_plan's format (candidates numbered in this step's order), and *plan_n
 * its length in int32 words (plan_cap is its capacity).  An idle step (no
 * unfinished candidate) does nothing and sets *plan_n = 0.  On a planning-only
 * context the tree work is done and no kernel runs.  Errors: JEV_ENOMEM (the
 * step's plan does not fit; nothing changes and the requests stay queued or
 * active), JEV_EINVAL (plan_out too small), JEV_EHIP. */
int jev_sched_step(jev_sched* s, void* hip_stream, int32_t* plan_out, int64_t plan_cap, int64_t* plan_n);
/* Thread-safe: *state = JEV_SCHED_QUEUED, _ACTIVE or _FINISHED.
 * Errors: JEV_EHANDLE (unknown ticket, or a result already collected). */
int jev_sched_status(jev_sched* s, int64_t ticket, int32_t* state);
/* Thread-safe: copies a finished request's probabilities (host float32, in
 * its label_offsets layout; cap = entries available) and forgets the request.
 * Errors: JEV_EPENDING (queued or active), JEV_EHANDLE (unknown or collected),
 * JEV_ESTATE (planning-only context), JEV_EINVAL (probs NULL or too small). */
int jev_sched_result(jev_sched* s, int64_t ticket, float* probs, int64_t cap);

const char* jev_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* JEV_H */
