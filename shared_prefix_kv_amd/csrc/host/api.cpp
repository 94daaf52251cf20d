// C ABI (include/jev.h) and the host engine that turns a call into rounds of
// kernel launches.
//
// A call is planned completely on the host first (validation, page
// assignment, the descriptors of every round), the descriptors go to the
// device in one copy, and then each round runs: embedding, per layer
// [RMSNorm -> QKV GEMM + RoPE + page write -> attention tiles -> LSE merge ->
// output projection + residual], then the label readout.
//
// Attention work of a round (the branch step the pages describe: each branch
// computes only its own suffix while attending to the cached prefix; LLM2Jev
// shared-prefix page, Radix Cache section; openjev-multimodal performance page,
// "what changed" and "next steps" sections, which batch several questions
// from one checkpoint):
//  * own part: each node's tokens against its own pages, causal;
//  * prefix part: all tokens of the sibling nodes that share a parent, packed
//    together, against the parent's whole page path, unmasked, split into page
//    chunks; the prefix pages are read once per sibling group and KV head
//    instead of once per branch;
//  * a node without a parent writes its output directly; otherwise every part
//    leaves a normalised partial state and a log2-sum-exp, merged exactly.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <set>
#include <string>
#include <vector>

#include "../../../include/jev.h"
#include "../kernels/launch.hpp"
#include "answers.hpp"
#include "tree.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

constexpr int kMaxChunks = jev::kMaxAncParts;  // prefix chunks per sibling group
// own causal tiles are split in two when a round has fewer (tile, KV head)
// pairs than the GPU has CUs (otherwise every CU already holds work)
constexpr int64_t kSplitTilesBelow = 256;
constexpr int kRowsPerTile = 128;
// attention rounds whose longest tile has at least this many pages run two
// wave groups per workgroup
constexpr int32_t kTwoGroupPages = 48;
// prefix chunk length of round-invariant numerics (jev_set_round_invariant)
constexpr int64_t kInvariantChunkPages = 32;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct WsLayout {
  size_t rope, x, h, q, o, part_o, part_lse, gemm_part, desc, total;
  size_t gemm_part_elems;
  int64_t part_rows;
  int64_t desc_ints;
};

int elt_size(const jev_model_desc& d) { return d.dtype == JEV_DTYPE_BF16 ? 2 : 4; }

WsLayout layout(const jev_model_desc& d) {
  WsLayout L{};
  const int64_t T = d.max_round_tokens;
  const int G = d.n_q_heads / d.n_kv_heads;
  const int64_t tt = kRowsPerTile / G;
  // partial rows: own tiles plus prefix-chunk tiles of a round, per KV head
  // (the chunk count is chosen so that tiles x chunks x Hkv stays within 512)
  L.part_rows = int64_t(kRowsPerTile) * (int64_t(d.n_kv_heads) * (2 * ((T + tt - 1) / tt) + 64) + 1024);
  L.desc_ints = 32 * T + 4 * int64_t(d.max_positions) + (1 << 18);
  const size_t e = elt_size(d);
  size_t off = 0;
  L.rope = off;
  off = align256(off + size_t(d.max_positions) * (d.head_dim / 2) * 2 * sizeof(float));
  L.x = off;
  off = align256(off + size_t(T) * d.d_model * e);
  L.h = off;
  off = align256(off + size_t(T) * d.d_model * e);
  L.q = off;
  off = align256(off + size_t(T) * d.n_q_heads * d.head_dim * e);
  L.o = off;
  off = align256(off + size_t(T) * d.n_q_heads * d.head_dim * e);
  L.part_o = off;
  off = align256(off + size_t(L.part_rows) * d.head_dim * sizeof(float));
  L.part_lse = off;
  off = align256(off + size_t(L.part_rows) * sizeof(float));
  // split-K scratch of the branch-phase GEMMs: one fp32 [256][N] partial tile
  // per K split
  const int64_t nmax = std::max<int64_t>(int64_t(d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim, d.d_model);
  L.gemm_part_elems = size_t(jev::kMaxSplits) * 256 * size_t(nmax);
  L.gemm_part = off;
  off = align256(off + L.gemm_part_elems * sizeof(float));
  L.desc = off;
  off = align256(off + size_t(L.desc_ints) * sizeof(int32_t));
  L.total = off;
  return L;
}

bool desc_ok(const jev_model_desc* d, std::string* why) {
  if (!d) return *why = "desc is NULL", false;
  if (d->n_layers < 1 || d->d_model < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->vocab < 1)
    return *why = "non-positive model dimension", false;
  if (d->n_q_heads % d->n_kv_heads) return *why = "n_kv_heads must divide n_q_heads", false;
  const int G = d->n_q_heads / d->n_kv_heads;
  if (G > kRowsPerTile || kRowsPerTile % G) return *why = "query heads per KV head must divide 128", false;
  if (!((d->dtype == JEV_DTYPE_BF16 && d->head_dim == 128) || (d->dtype == JEV_DTYPE_F32 && d->head_dim == 64)))
    return *why = "supported: bf16 with head_dim 128, f32 with head_dim 64", false;
  const int64_t nqkv = int64_t(d->n_q_heads + 2 * d->n_kv_heads) * d->head_dim;
  if (nqkv % 128 || d->d_model % 128) return *why = "projection widths must be multiples of 128", false;
  const int chunk_elems = 16 / elt_size(*d);
  if (d->d_model % (8 * chunk_elems) || (int64_t(d->n_q_heads) * d->head_dim) % (8 * chunk_elems))
    return *why = "reduction widths must be multiples of 128 bytes", false;
  if (d->d_model > 256 * 4 * chunk_elems) return *why = "d_model too large for the norm kernel", false;
  if (d->max_positions < 1 || d->max_round_tokens < 1) return *why = "max_positions/max_round_tokens < 1", false;
  if (d->max_positions > 65536) return *why = "max_positions above 65536", false;
  if (!(d->rope_theta > 0.f) || !(d->rms_eps >= 0.f)) return *why = "bad rope_theta or rms_eps", false;
  return true;
}

// ----------------------------------------------------------------- rounds

struct ReadSpec {
  int32_t cand;
  const int32_t* labels;
  int32_t k;
  int64_t out_off;
};

// A node computed in a round.
struct RNode {
  int64_t group;                   // nodes with the same parent share a group
  std::vector<jev::PageRef> anc;   // parent's page path (root first); empty: no parent
  const int32_t* tok;
  int64_t n;
  int64_t start;                   // logical position of tok[0]
  std::vector<int32_t> pages;
  std::vector<ReadSpec> reads;
};

struct RoundDesc {
  int32_t T = 0;
  int64_t off_tok = 0, off_pos = 0, off_slot = 0, off_plist = 0, off_tiles = 0, off_merge = 0,
          off_read = 0, off_labels = 0;
  int32_t n_tiles = 0, n_merge = 0, n_read = 0;
  int64_t part_slots = 0;
  double attn_pairs = 0;  // visible (query row, key) pairs of one layer
  int64_t n_part_rows = 0;
  int32_t attn_groups = 1;  // wave groups per attention workgroup
  // last layer: every row, none (only its K/V pages are needed), or the
  // read-out rows alone (ll_R of them, compacted: round rows at ll_off_rows,
  // positions at ll_off_pos, their own tiles and merges)
  int32_t last_mode = 0;
  int32_t ll_R = 0;
  int64_t ll_off_rows = 0, ll_off_pos = 0, ll_off_tiles = 0, ll_off_merge = 0;
  int32_t ll_n_tiles = 0, ll_n_merge = 0;
  int64_t ll_part_slots = 0;
  double ll_attn_pairs = 0;
};
enum { LAST_ALL = 0, LAST_NONE = 1, LAST_READ_ROWS = 2 };

// Device scratch of a call's kernels: attention partial states (rows of dh
// floats plus their log2-sum-exp) and the split-K partial tiles of the
// branch-round projections.
struct Scratch {
  float* part_o;
  float* part_lse;
  int64_t part_rows;
  jev::GemmWs gemm;
  bool no_alloc;  // the call may not create anything (profiling records are skipped)
};

}  // namespace

struct jev_ctx {
  jev_model_desc desc{};
  bool dry = true;
  bool dead = false;
  jev::PlanMode plan_mode = jev::PlanMode::DEPTH;
  bool round_invariant = false;  // jev_set_round_invariant
  uint64_t clock = 0;  // stamp of the last call (cache recency)
  jev::ModelDims dims{};
  std::vector<jev::LayerW> layers;
  const void* embed = nullptr;
  const void* unembed = nullptr;
  const void* final_norm = nullptr;
  char* pool = nullptr;
  WsLayout L{};
  char* ws = nullptr;
  char* static_scratch = nullptr;  // this device's copy of the file-scope scratch array
  // Pinned staging of a call's descriptors: two halves of L.desc_ints ints,
  // used by calls in turn.  A call reads its half on the device (the first
  // kernel copies it up) only before its end event, so the host rewrites a
  // half once the end event of the call before last that used it has passed:
  // no event between kernels.
  int32_t* desc_host = nullptr;
  int32_t* desc_host_dev = nullptr;  // its device-side address
  hipEvent_t done_ev[2] = {nullptr, nullptr};  // end of the latest call on each half
  int32_t desc_half = 0;                       // half of the next call
  hipEvent_t last_done = nullptr;              // end of the latest call (one of done_ev)
  bool have_last = false;
  hipStream_t last_stream = nullptr;
  jev::PagePool pages;
  std::unique_ptr<jev::ResidentTree> tree;
  jev_stats_t stats{};
  struct Tap {
    int32_t what, layer;
    void* dst;
    int64_t rows;
  };
  std::vector<Tap> taps;
  struct Prof {
    jev_launch_record rec;
    hipEvent_t e0, e1;
  };
  uint32_t prof_mask = 0;
  int64_t prof_rows = 0;  // only launches of this many rows are timed (0: all)
  std::vector<Prof> prof;
  std::vector<hipEvent_t> prof_free;  // events kept for re-use
  std::vector<jev_sched*> scheds;     // schedulers on this context (detached when it is destroyed)
  // debug modes and call timing (jev_set_debug, jev_stats)
  uint32_t debug = 0;
  int32_t call_kind = JEV_CALL_NONE;       // kind of the call in progress
  std::chrono::steady_clock::time_point call_t0{};
  std::vector<int32_t> call_written;       // KV pages the last run_rounds wrote
  std::vector<hipEvent_t> round_ev;        // round boundaries of the last timed call
  std::vector<char> round_reads;           // per round of it: has read-outs
  int32_t n_round_ev = 0;                  // events recorded by the last call (0: not timed)
};

namespace {

#define HIPCHK(expr)                                                              \
  do {                                                                            \
    hipError_t e_ = (expr);                                                       \
    if (e_ != hipSuccess) {                                                       \
      ctx->dead = true;                                                           \
      return fail(JEV_EHIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
    }                                                                             \
  } while (0)

int check_alive(jev_ctx* ctx) {
  if (!ctx) return fail(JEV_EINVAL, "ctx is NULL");
  if (ctx->dead) return fail(JEV_EHIP, "context is unusable after an earlier HIP failure");
  return JEV_OK;
}

// Start of an entry point that may run device work (timing of jev_stats).
void begin_call(jev_ctx* ctx, int32_t kind) {
  ctx->call_kind = kind;
  ctx->call_t0 = std::chrono::steady_clock::now();
}

int64_t ns_since(std::chrono::steady_clock::time_point t0) {
  return std::chrono::duration_cast<std::chrono::nanoseconds>(std::chrono::steady_clock::now() - t0).count();
}

// Free pages before a call, when its freed pages are to be poisoned.
std::set<int32_t> poison_before(const jev_ctx* ctx) {
  if (ctx->dry || !(ctx->debug & JEV_DEBUG_POISON_FREED_PAGES)) return {};
  return ctx->pages.snapshot();
}

// JEV_DEBUG_POISON_FREED_PAGES: after a call's kernels, on its stream, fills
// every page that is free now and that the call wrote (call_written) or freed
// (free now, not free before).  Runs of consecutive ids are filled by one
// launch each.
int poison_after(jev_ctx* ctx, const std::set<int32_t>& before, const std::vector<int32_t>& written,
                 hipStream_t s) {
  if (ctx->dry || !(ctx->debug & JEV_DEBUG_POISON_FREED_PAGES)) return JEV_OK;
  const std::set<int32_t> now = ctx->pages.snapshot();
  std::set<int32_t> pages;
  for (int32_t p : now)
    if (!before.count(p)) pages.insert(p);
  for (int32_t p : written)
    if (now.count(p)) pages.insert(p);
  if (pages.empty()) return JEV_OK;
  for (auto it = pages.begin(); it != pages.end();) {
    const int32_t first = *it;
    int32_t count = 0;
    while (it != pages.end() && *it == first + count) {
      ++count;
      ++it;
    }
    HIPCHK(jev::launch_poison_pages(ctx->dims, ctx->pool, first, count, s));
  }
  // the next call (possibly on another stream) is ordered after the fills
  HIPCHK(hipEventRecord(ctx->last_done, s));
  ctx->have_last = true;
  ctx->last_stream = s;
  return JEV_OK;
}

Scratch ws_scratch(const jev_ctx* ctx) {
  return Scratch{reinterpret_cast<float*>(ctx->ws + ctx->L.part_o), reinterpret_cast<float*>(ctx->ws + ctx->L.part_lse),
                 ctx->L.part_rows,
                 jev::GemmWs{reinterpret_cast<float*>(ctx->ws + ctx->L.gemm_part), ctx->L.gemm_part_elems}, false};
}

}  // namespace

// ----------------------------------------------------------------- static scratch
// Scratch of jev_score_branches_noalloc: a file-scope device array, one copy
// per GPU the library runs on, held until the process ends.  On the host its
// name is only a stand-in symbol, never a device address: jev_create looks up
// the current device's copy once with hipGetSymbolAddress, and every use goes
// through that pointer (kernel arguments).
constexpr size_t kNoAllocScratchBytes = size_t(96) << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

// This device's copy of the scratch array (looked up once per device).
int device_scratch(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(JEV_EHIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(JEV_EHIP, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(JEV_EHIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return JEV_OK;
}

// The static scratch laid out for a call: the split-K partial tiles first
// (sized like the workspace's), then as many attention partial-state rows as
// fit; JEV_ENOMEM if the call's rounds need more rows.
// Attention partial-state rows the static scratch holds after the split-K
// tiles (0 if those alone do not fit).
int64_t noalloc_rows(const jev_ctx* ctx) {
  const size_t gemm_bytes = align256(ctx->L.gemm_part_elems * sizeof(float));
  const size_t row_bytes = size_t(ctx->desc.head_dim + 1) * sizeof(float);
  if (gemm_bytes + 512 + row_bytes > kNoAllocScratchBytes) return 0;
  return int64_t((kNoAllocScratchBytes - gemm_bytes - 512) / row_bytes);
}

int static_scratch_for(const jev_ctx* ctx, const std::vector<RoundDesc>& rds, Scratch* out) {
  if (!ctx->static_scratch) return fail(JEV_ESTATE, "no static scratch on this context");
  const size_t gemm_bytes = align256(ctx->L.gemm_part_elems * sizeof(float));
  const int64_t rows = noalloc_rows(ctx);
  if (rows == 0) return fail(JEV_ENOMEM, "model too large for the 96 MiB static scratch");
  int64_t need = 0;
  for (const RoundDesc& rd : rds) need = std::max<int64_t>(need, rd.part_slots * ctx->desc.n_kv_heads * kRowsPerTile);
  if (need > rows)
    return fail(JEV_ENOMEM, "round needs " + std::to_string(need) + " partial-state rows; the 96 MiB static scratch holds " +
                                std::to_string(rows));
  char* base = ctx->static_scratch;
  const size_t o_bytes = align256(size_t(rows) * ctx->desc.head_dim * sizeof(float));
  *out = Scratch{reinterpret_cast<float*>(base + gemm_bytes), reinterpret_cast<float*>(base + gemm_bytes + o_bytes),
                 rows, jev::GemmWs{reinterpret_cast<float*>(base), ctx->L.gemm_part_elems}, true};
  return JEV_OK;
}

// Handles on the root..h paths of `hs`: prefixes a call uses, never evicted by it.
std::set<int64_t> path_set(const jev::ResidentTree& t, const std::vector<int64_t>& hs) {
  std::set<int64_t> out;
  for (int64_t h : hs)
    for (; h != 0 && !out.count(h); h = t.node(h).parent) out.insert(h);
  return out;
}

// Cached prefixes a call must evict to fit (cache policy on): least recently
// used first, none in `pinned`, found on copies of the tree and pool until
// fits(tree, pool) holds.  Nothing changes here; JEV_ENOMEM if they do not
// suffice.  The caller applies them together with the rest of its changes,
// once every check of the call has passed.
template <typename Fits>
int find_room(jev_ctx* ctx, const std::set<int64_t>& pinned, Fits fits, const char* what,
              std::vector<int64_t>* victims) {
  victims->clear();
  if (fits(*ctx->tree, ctx->pages)) return JEV_OK;  // a plan trial leaves the pool as it found it
  if (!ctx->tree->keep()) return fail(JEV_ENOMEM, what);
  jev::PagePool pool = ctx->pages;
  jev::ResidentTree tree = *ctx->tree;
  tree.rebind(&pool);
  while (!fits(tree, pool)) {
    const int64_t v = tree.evict_one(pinned);
    if (v == 0) return fail(JEV_ENOMEM, what);
    victims->push_back(v);
  }
  return JEV_OK;
}

// Stages the pages of a call's victims as free in the pool (the caller
// restores its snapshot after simulating its page allocation).
void release_victim_pages(jev_ctx* ctx, const std::vector<int64_t>& victims) {
  for (int64_t v : victims) ctx->pages.release(ctx->tree->node(v).pages);
}

// Resident prefixes the candidates of a plan continue (their match paths).
std::set<int64_t> plan_pins(const jev::ResidentTree& t, int32_t n, const int32_t* tok, const int64_t* off) {
  std::vector<int64_t> used;
  for (int32_t c = 0; c < n; ++c) {
    int64_t h, m;
    t.match(tok + off[c], off[c + 1] - off[c], &h, &m);
    used.push_back(h);
  }
  return path_set(t, used);
}

// The tree work of a candidate call, on copies of the tree and pool: each
// candidate in input order takes its anchor (splitting a resident node at a
// page boundary where it diverges inside it), then cached prefixes are evicted
// (cache policy) until the plan fits.  The caller commits the copies or drops
// them.
int stage_candidates(jev_ctx* ctx, int32_t n, const int32_t* tok, const int64_t* off, jev::PagePool* pool,
                     jev::ResidentTree* tree, jev::Plan* plan, jev::PlanMode mode) {
  *pool = ctx->pages;
  *tree = *ctx->tree;
  tree->rebind(pool);
  for (int32_t c = 0; c < n; ++c) {
    int64_t h, m;
    tree->match_split(tok + off[c], off[c + 1] - off[c], &h, &m);
  }
  const std::set<int64_t> pinned = plan_pins(*tree, n, tok, off);
  while (!jev::plan_candidates(*tree, pool, n, tok, off, plan, mode))
    if (!tree->keep() || tree->evict_one(pinned) == 0) return fail(JEV_ENOMEM, "not enough free KV pages for the plan");
  return JEV_OK;
}

int check_segments(const jev_ctx* ctx, int32_t n, const int32_t* tokens, const int64_t* off, const char* what) {
  if (n < 0) return fail(JEV_EINVAL, std::string(what) + ": n < 0");
  if (n == 0) return JEV_OK;
  if (!tokens || !off) return fail(JEV_EINVAL, std::string(what) + ": NULL tokens/offsets");
  if (off[0] != 0) return fail(JEV_EINVAL, std::string(what) + ": offsets[0] != 0");
  for (int32_t i = 0; i < n; ++i) {
    if (off[i + 1] <= off[i])
      return fail(JEV_EINVAL, std::string(what) + ": empty or decreasing segment " + std::to_string(i));
  }
  const int32_t V = ctx->desc.vocab;
  for (int64_t i = 0; i < off[n]; ++i)
    if (tokens[i] < 0 || tokens[i] >= V)
      return fail(JEV_EINVAL, std::string(what) + ": token id out of range at " + std::to_string(i));
  return JEV_OK;
}

int check_labels(const jev_ctx* ctx, int32_t n, const int32_t* labels, const int64_t* loff) {
  if (!labels || !loff) return fail(JEV_EINVAL, "NULL labels/label_offsets");
  if (loff[0] != 0) return fail(JEV_EINVAL, "label_offsets[0] != 0");
  for (int32_t i = 0; i < n; ++i) {
    const int64_t k = loff[i + 1] - loff[i];
    if (k < JEV_MIN_LABELS || k > JEV_MAX_LABELS)
      return fail(JEV_EINVAL, "branch " + std::to_string(i) + ": label count outside [2, 64]");
    for (int64_t a = loff[i]; a < loff[i + 1]; ++a) {
      if (labels[a] < 0 || labels[a] >= ctx->desc.vocab)
        return fail(JEV_EINVAL, "branch " + std::to_string(i) + ": label id out of range");
      for (int64_t b = loff[i]; b < a; ++b)
        if (labels[b] == labels[a]) return fail(JEV_EINVAL, "branch " + std::to_string(i) + ": duplicate label");
    }
  }
  return JEV_OK;
}

// Builds the descriptors of one round into hb (int32 words) and returns its layout.
int build_round(jev_ctx* ctx, std::vector<RNode>& nodes, std::vector<int32_t>& hb, RoundDesc* rd) {
  const int G = ctx->desc.n_q_heads / ctx->desc.n_kv_heads;
  const int TT = kRowsPerTile / G;
  // order nodes by group (groups in order of first appearance), stable
  std::vector<int64_t> gorder;
  for (auto& nd : nodes)
    if (std::find(gorder.begin(), gorder.end(), nd.group) == gorder.end()) gorder.push_back(nd.group);
  std::stable_sort(nodes.begin(), nodes.end(), [&](const RNode& a, const RNode& b) {
    return std::find(gorder.begin(), gorder.end(), a.group) < std::find(gorder.begin(), gorder.end(), b.group);
  });
  int64_t T = 0;
  for (auto& nd : nodes) T += nd.n;
  if (T > ctx->desc.max_round_tokens)
    return fail(JEV_ENOMEM, "round of " + std::to_string(T) + " tokens exceeds max_round_tokens");
  rd->T = int32_t(T);
  auto push = [&](int64_t words) {
    int64_t o = int64_t(hb.size());
    hb.resize(hb.size() + size_t(words), 0);
    return o;
  };
  rd->off_tok = push(T);
  rd->off_pos = push(T);
  rd->off_slot = push(T);
  std::vector<int64_t> node_t0(nodes.size());
  {
    int64_t t = 0;
    for (size_t i = 0; i < nodes.size(); ++i) {
      RNode& nd = nodes[i];
      node_t0[i] = t;
      for (int64_t j = 0; j < nd.n; ++j, ++t) {
        hb[rd->off_tok + t] = nd.tok[j];
        hb[rd->off_pos + t] = int32_t(nd.start + j);
        hb[rd->off_slot + t] = nd.pages[j / jev::kPage] * jev::kPage + int32_t(j % jev::kPage);
      }
    }
  }
  // page lists: own pages per node, parent path per group
  std::vector<int64_t> own_off(nodes.size());
  std::vector<int64_t> plist;  // pairs
  for (size_t i = 0; i < nodes.size(); ++i) {
    own_off[i] = int64_t(plist.size() / 2);
    const RNode& nd = nodes[i];
    for (size_t p = 0; p < nd.pages.size(); ++p) {
      int64_t v = nd.n - int64_t(jev::kPage) * int64_t(p);
      plist.push_back(nd.pages[p]);
      plist.push_back(int32_t(v < jev::kPage ? v : jev::kPage));
    }
  }
  struct Group {
    int64_t t0, t1, anc_off, anc_pages;
  };
  std::vector<Group> groups;
  for (size_t i = 0; i < nodes.size(); ++i) {
    if (i == 0 || nodes[i].group != nodes[i - 1].group) {
      Group g{node_t0[i], node_t0[i], int64_t(plist.size() / 2), int64_t(nodes[i].anc.size())};
      for (auto& pr : nodes[i].anc) {
        plist.push_back(pr.page);
        plist.push_back(pr.valid);
      }
      groups.push_back(g);
    }
    groups.back().t1 = node_t0[i] + nodes[i].n;
  }
  rd->off_plist = push(int64_t(plist.size()));
  std::copy(plist.begin(), plist.end(), hb.begin() + rd->off_plist);

  // chunking of the prefix part
  int64_t anc_qtiles = 0, min_anc_pages = INT64_MAX;
  for (auto& g : groups)
    if (g.anc_pages > 0) {
      anc_qtiles += (g.t1 - g.t0 + TT - 1) / TT;
      min_anc_pages = std::min(min_anc_pages, g.anc_pages);
    }
  int64_t own_qtiles = 0;
  for (auto& nd : nodes) own_qtiles += (nd.n + TT - 1) / TT;
  int64_t n_chunks = 1;
  if (anc_qtiles > 0) {
    // as many chunks as fit, with the own tiles, in one wave of the 512
    // workgroup slots (two per CU): a second, partial wave would add a
    // whole chunk's steps for a few tiles
    const int64_t slots = 512 - own_qtiles * ctx->desc.n_kv_heads;
    n_chunks = slots / (anc_qtiles * ctx->desc.n_kv_heads);
    n_chunks = std::max<int64_t>(1, std::min<int64_t>({n_chunks, kMaxChunks, min_anc_pages / 8}));
  }

  // When a round has too few attention tiles to occupy every CU, its time is
  // set by the longest causal tile; tiles longer than cpo pages are then split
  // in two: the pages before the tile's first query page (every key visible,
  // unmasked) and the rest (causal), merged like prefix chunks.
  int64_t n_own_tiles = 0, max_own_pages = 0;
  for (auto& nd : nodes) {
    n_own_tiles += (nd.n + TT - 1) / TT;
    max_own_pages = std::max<int64_t>(max_own_pages, (nd.n + jev::kPage - 1) / jev::kPage);
  }
  int64_t cpo = INT64_MAX;
  if (!ctx->round_invariant && n_own_tiles * ctx->desc.n_kv_heads < kSplitTilesBelow && max_own_pages >= 32) {
    cpo = (max_own_pages + 1) / 2;
    cpo += cpo & 1;
  }

  // One attention plan over a set of query tokens.  A query range is tokens
  // [i0, i0 + nt) of node `node`, whose first token is query row tq of the
  // launch (q, positions and output rows); `tile_i0` is the first token of the
  // round tile that holds it, which fixes the split point, so that a range
  // planned alone gets the same tiles, page steps and merge order as in the
  // whole round.  grows[g] are the query rows of group g.
  struct QRange {
    size_t node;
    int64_t i0, nt, tq, tile_i0;
  };
  struct AttnPlan {
    std::vector<jev::AttnTile> tiles;
    std::vector<jev::MergeItem> merges;
    int64_t slots = 0;
    double pairs = 0;
  };
  auto plan_attention = [&](const std::vector<QRange>& qr, int64_t n_rows,
                            const std::vector<std::pair<int64_t, int64_t>>& grows, AttnPlan* ap) {
    std::vector<jev::AttnTile>& tiles = ap->tiles;
    std::vector<jev::MergeItem>& merges = ap->merges;
    int64_t slot = 0;
    std::vector<int32_t> own_slot(size_t(n_rows), -1), own_ti(size_t(n_rows), -1), own_n(size_t(n_rows), 0);
    for (const QRange& r : qr) {
      const RNode& nd = nodes[r.node];
      const bool has_anc = !nd.anc.empty();
      const int64_t nt = r.nt, i0 = r.i0;
      const int64_t np = (i0 + nt - 1) / jev::kPage + 1;
      // split point of the round tile: an even page count, at or before its
      // first query's page
      const int64_t tile_nt = std::min<int64_t>(TT, nd.n - r.tile_i0);
      const int64_t tile_np = (r.tile_i0 + tile_nt - 1) / jev::kPage + 1;
      int64_t sp = 0;
      if (tile_np > cpo) sp = std::min<int64_t>(tile_np / 2, r.tile_i0 / jev::kPage) & ~int64_t(1);
      const bool partial = has_anc || sp > 0;
      // causal pairs of the range: token i0+j sees i0+j+1 own keys
      ap->pairs += double(G) * double(ctx->desc.n_kv_heads) * double(nt * i0 + nt * (nt + 1) / 2);
      if (partial)
        for (int64_t j = 0; j < nt; ++j) {
          own_slot[size_t(r.tq + j)] = int32_t(slot);
          own_ti[size_t(r.tq + j)] = int32_t(j);
          own_n[size_t(r.tq + j)] = sp > 0 ? 2 : 1;
        }
      if (sp > 0) {
        jev::AttnTile tl{};
        tl.t0 = int32_t(r.tq);
        tl.n_tok = int32_t(nt);
        tl.page_off = int32_t(own_off[r.node]);
        tl.n_pages = int32_t(sp);
        tl.causal = 0;
        tl.kv_pos0 = int32_t(nd.start);
        tl.out_mode = 1;
        tl.part_slot = int32_t(slot++);
        tiles.push_back(tl);
      }
      jev::AttnTile tl{};
      tl.t0 = int32_t(r.tq);
      tl.n_tok = int32_t(nt);
      tl.page_off = int32_t(own_off[r.node] + sp);
      tl.n_pages = int32_t(np - sp);
      tl.causal = 1;
      tl.kv_pos0 = int32_t(nd.start + jev::kPage * sp);
      tl.out_mode = partial ? 1 : 0;
      tl.part_slot = partial ? int32_t(slot++) : 0;
      tiles.push_back(tl);
    }
    std::vector<char> merged(size_t(n_rows), 0);
    for (size_t gi = 0; gi < groups.size(); ++gi) {
      const Group& g = groups[gi];
      const int64_t r0 = grows[gi].first, r1 = grows[gi].second;
      if (g.anc_pages == 0 || r1 <= r0) continue;
      int64_t cp = (g.anc_pages + n_chunks - 1) / n_chunks;
      if (ctx->round_invariant) {
        // chunks set by the prefix alone: kInvariantChunkPages pages, more
        // when that would exceed the merge's chunk count
        cp = std::max<int64_t>(kInvariantChunkPages, (g.anc_pages + jev::kMaxAncParts - 1) / jev::kMaxAncParts);
      }
      cp += cp & 1;  // whole two-page steps per chunk
      const int64_t nch = (g.anc_pages + cp - 1) / cp;
      int64_t anc_keys = 0;
      for (int64_t pi = 0; pi < g.anc_pages; ++pi) anc_keys += plist[2 * (g.anc_off + pi) + 1];
      ap->pairs += double(r1 - r0) * G * double(ctx->desc.n_kv_heads) * double(anc_keys);
      for (int64_t t0 = r0; t0 < r1; t0 += TT) {
        const int64_t nt = std::min<int64_t>(TT, r1 - t0);
        const int64_t slot0 = slot;
        for (int64_t c = 0; c < nch; ++c) {
          jev::AttnTile tl{};
          tl.t0 = int32_t(t0);
          tl.n_tok = int32_t(nt);
          tl.page_off = int32_t(g.anc_off + c * cp);
          tl.n_pages = int32_t(std::min(cp, g.anc_pages - c * cp));
          tl.causal = 0;
          tl.out_mode = 1;
          tl.part_slot = int32_t(slot++);
          tiles.push_back(tl);
        }
        for (int64_t j = 0; j < nt; ++j) {
          const size_t t = size_t(t0 + j);
          merges.push_back(jev::MergeItem{int32_t(t), own_slot[t], own_ti[t], own_n[t], int32_t(slot0),
                                          int32_t(j), int32_t(nch), 0});
          merged[t] = 1;
        }
      }
    }
    // rows of split tiles without a prefix part
    for (int64_t t = 0; t < n_rows; ++t)
      if (!merged[size_t(t)] && own_n[size_t(t)] > 1)
        merges.push_back(jev::MergeItem{int32_t(t), own_slot[size_t(t)], own_ti[size_t(t)], own_n[size_t(t)], 0,
                                        0, 0, 0});
    // heavy tiles first
    std::stable_sort(tiles.begin(), tiles.end(),
                     [](const jev::AttnTile& a, const jev::AttnTile& b) { return a.n_pages > b.n_pages; });
    ap->slots = slot;
  };

  // the whole round
  AttnPlan full;
  {
    std::vector<QRange> qr;
    for (size_t i = 0; i < nodes.size(); ++i)
      for (int64_t i0 = 0; i0 < nodes[i].n; i0 += TT)
        qr.push_back(QRange{i, i0, std::min<int64_t>(TT, nodes[i].n - i0), node_t0[i] + i0, i0});
    std::vector<std::pair<int64_t, int64_t>> grows;
    for (auto& g : groups) grows.emplace_back(g.t0, g.t1);
    plan_attention(qr, T, grows, &full);
  }
  if (full.slots * ctx->desc.n_kv_heads * kRowsPerTile > ctx->L.part_rows)
    return fail(JEV_ENOMEM, "round needs more partial-state rows than the workspace holds");
  rd->part_slots = full.slots;
  rd->n_part_rows = int64_t(full.merges.size());
  rd->attn_pairs = full.pairs;
  rd->n_tiles = int32_t(full.tiles.size());
  // a round whose longest tile has many steps splits every tile's steps over
  // two wave groups, halving the chain that sets the kernel's length
  rd->attn_groups = (!full.tiles.empty() && full.tiles.front().n_pages >= kTwoGroupPages) ? 2 : 1;
  // round-invariant numerics: every round splits each tile's steps over two
  // groups (a split that depends on the tile alone)
  if (ctx->round_invariant) rd->attn_groups = 2;
  rd->off_tiles = push(int64_t(full.tiles.size()) * 8);
  std::memcpy(hb.data() + rd->off_tiles, full.tiles.data(), full.tiles.size() * sizeof(jev::AttnTile));
  rd->n_merge = int32_t(full.merges.size());
  rd->off_merge = push(int64_t(full.merges.size()) * int64_t(sizeof(jev::MergeItem) / sizeof(int32_t)));
  std::memcpy(hb.data() + rd->off_merge, full.merges.data(), full.merges.size() * sizeof(jev::MergeItem));

  // The last layer.  Nothing reads a token's last-layer attention or output
  // projection except the read-out of its own final state, and later rounds
  // read only K/V pages: a round without read-outs skips them, and a round
  // whose read-out rows are few computes them for those rows only, with the
  // tiles they have in the whole round (same chunks, split points and wave
  // groups), so their values are bitwise those of the whole round.  The
  // debug taps and JEV_DEBUG_FULL_LAST_LAYER keep every row.
  int64_t R = 0;
  for (auto& nd : nodes) R += nd.reads.empty() ? 0 : 1;
  rd->last_mode = LAST_ALL;
  if (ctx->taps.empty() && !(ctx->debug & JEV_DEBUG_FULL_LAST_LAYER)) {
    if (R == 0)
      rd->last_mode = LAST_NONE;
    else if (4 * R <= T)
      rd->last_mode = LAST_READ_ROWS;
  }
  if (rd->last_mode == LAST_READ_ROWS) {
    // compact query rows, in round order (so grouped like the round's)
    std::vector<QRange> qr;
    std::vector<std::pair<int64_t, int64_t>> grows(groups.size(), {0, 0});
    std::vector<int32_t> rows, pos;
    size_t gi = 0;
    for (size_t i = 0; i < nodes.size(); ++i) {
      while (gi + 1 < groups.size() && node_t0[i] >= groups[gi].t1) ++gi;
      if (nodes[i].reads.empty()) continue;
      const int64_t r = int64_t(rows.size()), i0 = nodes[i].n - 1;
      if (grows[gi].second <= grows[gi].first)
        grows[gi] = {r, r + 1};
      else
        grows[gi].second = r + 1;
      qr.push_back(QRange{i, i0, 1, r, (i0 / TT) * TT});
      rows.push_back(int32_t(node_t0[i] + i0));
      pos.push_back(int32_t(nodes[i].start + i0));
    }
    AttnPlan ll;
    plan_attention(qr, R, grows, &ll);
    rd->ll_R = int32_t(R);
    rd->ll_off_rows = push(R);
    std::copy(rows.begin(), rows.end(), hb.begin() + rd->ll_off_rows);
    rd->ll_off_pos = push(R);
    std::copy(pos.begin(), pos.end(), hb.begin() + rd->ll_off_pos);
    rd->ll_part_slots = ll.slots;
    rd->ll_attn_pairs = ll.pairs;
    rd->ll_n_tiles = int32_t(ll.tiles.size());
    rd->ll_off_tiles = push(int64_t(ll.tiles.size()) * 8);
    std::memcpy(hb.data() + rd->ll_off_tiles, ll.tiles.data(), ll.tiles.size() * sizeof(jev::AttnTile));
    rd->ll_n_merge = int32_t(ll.merges.size());
    rd->ll_off_merge = push(int64_t(ll.merges.size()) * int64_t(sizeof(jev::MergeItem) / sizeof(int32_t)));
    std::memcpy(hb.data() + rd->ll_off_merge, ll.merges.data(), ll.merges.size() * sizeof(jev::MergeItem));
  }
  // readouts
  std::vector<jev::ReadoutItem> reads;
  std::vector<int32_t> labs;
  for (size_t i = 0; i < nodes.size(); ++i)
    for (auto& r : nodes[i].reads) {
      reads.push_back(jev::ReadoutItem{int32_t(node_t0[i] + nodes[i].n - 1), int32_t(labs.size()), r.k,
                                       int32_t(r.out_off)});
      labs.insert(labs.end(), r.labels, r.labels + r.k);
    }
  rd->n_read = int32_t(reads.size());
  rd->off_read = push(int64_t(reads.size()) * 4);
  std::memcpy(hb.data() + rd->off_read, reads.data(), reads.size() * sizeof(jev::ReadoutItem));
  rd->off_labels = push(int64_t(labs.size()));
  std::copy(labs.begin(), labs.end(), hb.begin() + rd->off_labels);
  return JEV_OK;
}

// Copies the descriptors of a call to the device and runs its rounds.
int run_rounds(jev_ctx* ctx, const std::vector<RoundDesc>& rds, const std::vector<int32_t>& hb, float* probs,
               hipStream_t s, const Scratch& sc) {
  if (int64_t(hb.size()) > ctx->L.desc_ints)
    return fail(JEV_ENOMEM, "call descriptors exceed the workspace descriptor region");
  for (const RoundDesc& rd : rds)
    if (std::max(rd.part_slots, rd.ll_part_slots) * ctx->desc.n_kv_heads * kRowsPerTile > sc.part_rows)
      return fail(JEV_ENOMEM, "round needs more partial-state rows than the scratch holds");
  const int64_t prepare_ns = ns_since(ctx->call_t0);
  const auto enqueue_t0 = std::chrono::steady_clock::now();
  // (the allocation-free entry point times a call only with events made earlier)
  const bool timed_call = (ctx->debug & JEV_DEBUG_TIME_CALLS) != 0 &&
                          !(sc.no_alloc && ctx->round_ev.size() < rds.size() + 1);
  if (timed_call)
    while (ctx->round_ev.size() < rds.size() + 1) {
      hipEvent_t e = nullptr;
      // read after the device work is done: no system-scope fence needed
      HIPCHK(hipEventCreateWithFlags(&e, hipEventDisableSystemFence));
      ctx->round_ev.push_back(e);
    }
  ctx->n_round_ev = 0;
  if (ctx->have_last && s != ctx->last_stream) HIPCHK(hipStreamWaitEvent(s, ctx->last_done, 0));
  // this call's staging half: free once the last call that used it has ended
  // (an event never recorded has nothing to wait for)
  const int32_t half = ctx->desc_half;
  HIPCHK(hipEventSynchronize(ctx->done_ev[half]));
  int32_t* const desc_host = ctx->desc_host + size_t(half) * size_t(ctx->L.desc_ints);
  const int32_t* const desc_host_dev = ctx->desc_host_dev + size_t(half) * size_t(ctx->L.desc_ints);
  if (timed_call) HIPCHK(hipEventRecord(ctx->round_ev[0], s));
  std::memcpy(desc_host, hb.data(), hb.size() * sizeof(int32_t));
  int32_t* dd = reinterpret_cast<int32_t*>(ctx->ws + ctx->L.desc);
  // No separate copy (a host-to-device copy on the stream left the GPU idle
  // for ~15 us per call): the first round's embedding kernel reads its tokens
  // from the pinned staging buffer and copies the descriptors up, in 16-byte
  // units (the buffers hold a multiple of 16 bytes), for the kernels after it.
  const int64_t up_bytes = (int64_t(hb.size()) * int64_t(sizeof(int32_t)) + 15) / 16 * 16;
  const bool upload = !rds.empty() && rds[0].T > 0;
  if (!upload) HIPCHK(hipMemcpyAsync(dd, desc_host, hb.size() * sizeof(int32_t), hipMemcpyHostToDevice, s));
  const jev::ModelDims& m = ctx->dims;
  void* x = ctx->ws + ctx->L.x;
  void* h = ctx->ws + ctx->L.h;
  void* q = ctx->ws + ctx->L.q;
  void* o = ctx->ws + ctx->L.o;
  float* rope = reinterpret_cast<float*>(ctx->ws + ctx->L.rope);
  float* part_o = sc.part_o;
  float* part_lse = sc.part_lse;
  jev::GemmWs gws = sc.gemm;
  gws.no_split = ctx->round_invariant;
  const size_t elt = size_t(elt_size(ctx->desc));
  // times one launch with events when its kind is being profiled
  auto timed = [&](int kind, int layer, int64_t rows, double flops, double bytes, auto&& launch) -> hipError_t {
    if (sc.no_alloc || !(ctx->prof_mask & (1u << kind)) || (ctx->prof_rows > 0 && rows != ctx->prof_rows))
      return launch();
    jev_ctx::Prof p;
    p.rec = jev_launch_record{kind, layer, rows, flops, bytes, 0.f};
    for (hipEvent_t* e : {&p.e0, &p.e1}) {
      if (!ctx->prof_free.empty()) {
        *e = ctx->prof_free.back();
        ctx->prof_free.pop_back();
      } else {
        // timing only, read after the caller has synchronised the stream: no
        // system-scope fence (it costs a cache writeback between kernels)
        hipError_t err = hipEventCreateWithFlags(e, hipEventDisableSystemFence);
        if (err != hipSuccess) return err;
      }
    }
    // the launcher's own dispatches carry the events (no separate event
    // packets between kernels); a launcher that launched nothing gets a pair
    // of plain records
    jev::g_launch_timing = jev::LaunchTiming{p.e0, p.e1};
    hipError_t err = launch();
    const bool launched = jev::g_launch_timing.start == nullptr;
    jev::g_launch_timing = jev::LaunchTiming{nullptr, nullptr};
    if (err == hipSuccess && !launched) {
      err = hipEventRecord(p.e0, s);
      if (err == hipSuccess) err = hipEventRecord(p.e1, s);
    }
    ctx->prof.push_back(p);
    return err;
  };
  auto tap = [&](int what, int layer, const void* src, int64_t T, size_t width) -> int {
    if (rds.size() != 1) return JEV_OK;
    for (const auto& tp : ctx->taps)
      if (tp.what == what && tp.layer == layer) {
        const int64_t rows = std::min<int64_t>(T, tp.rows);
        HIPCHK(hipMemcpyAsync(tp.dst, src, size_t(rows) * width * elt, hipMemcpyDeviceToDevice, s));
      }
    return JEV_OK;
  };
  const double D = m.d, HD = double(m.hq) * m.dh, NQKV = double(m.hq + 2 * m.hkv) * m.dh, E = double(elt);
  ctx->call_written.clear();
  ctx->round_reads.clear();
  for (const RoundDesc& rd : rds) {
    for (int64_t t = 0; t < rd.T; ++t) ctx->call_written.push_back(hb[size_t(rd.off_slot + t)] >> 4);
    ctx->round_reads.push_back(rd.n_read > 0);
    const bool first = upload && &rd == &rds[0];
    const int32_t* tok = (first ? desc_host_dev : dd) + rd.off_tok;
    const double T = rd.T;
    // the embedding gather also writes layer 0's normalised input
    HIPCHK(timed(JEV_K_EMBED, -1, rd.T, 0, 3 * T * D * E + 4 * T, [&] {
      return jev::launch_embed_norm(m, ctx->embed, tok, rd.T, ctx->layers[0].norm, x, h, s,
                                    first ? desc_host_dev : nullptr, first ? dd : nullptr,
                                    first ? up_bytes : 0);
    }));
    bool h_ready = true;  // h of this layer already written (by the gather or the previous projection)
    for (int l = 0; l < m.n_layers; ++l) {
      const jev::LayerW& w = ctx->layers[l];
      if (int rc = tap(JEV_TAP_RESID, l, x, rd.T, size_t(m.d))) return rc;
      if (!h_ready)
        HIPCHK(timed(JEV_K_RMSNORM, l, rd.T, 0, (2 * T + 1) * D * E,
                     [&] { return jev::launch_rmsnorm(m, x, w.norm, rd.T, h, s); }));
      h_ready = false;
      // last layer without read-outs: its K/V pages are all that is needed
      const bool kv_only = l + 1 == m.n_layers && rd.last_mode == LAST_NONE;
      const double NP = kv_only ? double(2 * m.hkv) * m.dh : NQKV;
      HIPCHK(timed(JEV_K_QKV, l, rd.T, 2 * T * NP * D, (T * D + NP * D + T * NP) * E, [&] {
        return jev::launch_qkv(m, w, l, h, rd.T, dd + rd.off_pos, dd + rd.off_slot, rope, q, ctx->pool, gws, s,
                               kv_only);
      }));
      if (kv_only) break;
      if (l + 1 == m.n_layers && rd.last_mode == LAST_READ_ROWS) {
        // the read-out rows alone: attention of their queries (rows of q
        // named by the compact row list) into o rows [0, R), the output
        // projection's residual written back to their rows of x
        const int32_t* rows = dd + rd.ll_off_rows;
        const double R = rd.ll_R;
        HIPCHK(timed(JEV_K_ATTN, l, rd.ll_R, 4.0 * m.dh * rd.ll_attn_pairs, 0, [&] {
          return jev::launch_attention(m, l, reinterpret_cast<const jev::AttnTile*>(dd + rd.ll_off_tiles),
                                       rd.ll_n_tiles, dd + rd.off_plist, dd + rd.ll_off_pos, q, ctx->pool, o,
                                       part_o, part_lse, rd.attn_groups, s, rows);
        }));
        if (rd.ll_n_merge > 0)
          HIPCHK(timed(JEV_K_MERGE, l, rd.ll_n_merge, 0, 0, [&] {
            return jev::launch_merge(m, reinterpret_cast<const jev::MergeItem*>(dd + rd.ll_off_merge),
                                     rd.ll_n_merge, part_o, part_lse, o, s);
          }));
        HIPCHK(timed(JEV_K_OPROJ, l, rd.ll_R, 2 * R * D * HD, (R * HD + D * HD + 2 * R * D) * E,
                     [&] { return jev::launch_oproj(m, w, o, rd.ll_R, x, gws, s, rows); }));
        break;
      }
      HIPCHK(timed(JEV_K_ATTN, l, rd.T, 4.0 * m.dh * rd.attn_pairs, 0, [&] {
        return jev::launch_attention(m, l, reinterpret_cast<const jev::AttnTile*>(dd + rd.off_tiles), rd.n_tiles,
                                     dd + rd.off_plist, dd + rd.off_pos, q, ctx->pool, o, part_o, part_lse,
                                     rd.attn_groups, s);
      }));
      if (rd.n_merge > 0)
        HIPCHK(timed(JEV_K_MERGE, l, rd.n_merge, 0, 0, [&] {
          return jev::launch_merge(m, reinterpret_cast<const jev::MergeItem*>(dd + rd.off_merge), rd.n_merge,
                                   part_o, part_lse, o, s);
        }));
      if (int rc = tap(JEV_TAP_ATTN, l, o, rd.T, size_t(m.hq) * m.dh)) return rc;
      if (rd.T <= jev::kSplitRows && l + 1 < m.n_layers && !ctx->round_invariant) {
        // split-K projection whose residual epilogue also writes the next
        // layer's normalised input (one launch fewer per layer)
        HIPCHK(timed(JEV_K_OPROJ, l, rd.T, 2 * T * D * HD, (T * HD + D * HD + 2 * T * D) * E, [&] {
          int32_t splits = 0;
          const hipError_t e = jev::launch_oproj_split(m, w, o, rd.T, gws, &splits, s);
          if (e != hipSuccess) return e;
          return jev::launch_split_res_norm(m, gws.partial, splits, rd.T, x, ctx->layers[l + 1].norm, h, s);
        }));
        h_ready = true;
      } else {
        HIPCHK(timed(JEV_K_OPROJ, l, rd.T, 2 * T * D * HD, (T * HD + D * HD + 2 * T * D) * E,
                     [&] { return jev::launch_oproj(m, w, o, rd.T, x, gws, s); }));
      }
    }
    if (int rc = tap(JEV_TAP_RESID, m.n_layers, x, rd.T, size_t(m.d))) return rc;
    if (rd.n_read > 0)
      HIPCHK(timed(JEV_K_READOUT, -1, rd.n_read, 0, 0, [&] {
        return jev::launch_readout(m, ctx->unembed, ctx->final_norm, x,
                                   reinterpret_cast<const jev::ReadoutItem*>(dd + rd.off_read), rd.n_read,
                                   dd + rd.off_labels, probs, s);
      }));
    if (timed_call) HIPCHK(hipEventRecord(ctx->round_ev[&rd - rds.data() + 1], s));
  }
  if (timed_call) ctx->n_round_ev = int32_t(rds.size()) + 1;
  HIPCHK(hipEventRecord(ctx->done_ev[half], s));
  ctx->last_done = ctx->done_ev[half];
  ctx->desc_half = half ^ 1;
  ctx->have_last = true;
  ctx->last_stream = s;
  ctx->stats.last_call_kind = ctx->call_kind;
  ctx->stats.last_prepare_ns = prepare_ns;
  ctx->stats.last_enqueue_ns = ns_since(enqueue_t0);
  return JEV_OK;
}

}  // namespace

// ===================================================================== C ABI
extern "C" {

const char* jev_last_error(void) { return g_err.c_str(); }

int jev_answers(int32_t n, const float* probs, const int64_t* label_offsets, const int32_t* kinds, double* value,
                int32_t* choice, double* confidence) {
  if (n < 0) return fail(JEV_EINVAL, "n < 0");
  if (n == 0) return JEV_OK;
  if (!probs || !label_offsets || !kinds || !value) return fail(JEV_EINVAL, "NULL probs/offsets/kinds/value");
  if (label_offsets[0] != 0) return fail(JEV_EINVAL, "label_offsets[0] != 0");
  for (int32_t i = 0; i < n; ++i) {
    const int64_t k = label_offsets[i + 1] - label_offsets[i];
    if (k < JEV_MIN_LABELS || k > JEV_MAX_LABELS)
      return fail(JEV_EINVAL, "branch " + std::to_string(i) + ": label count outside [2, 64]");
    if (kinds[i] != JEV_ANSWER_NOUL && kinds[i] != JEV_ANSWER_CHOICE && kinds[i] != JEV_ANSWER_SCORE)
      return fail(JEV_EINVAL, "branch " + std::to_string(i) + ": unknown answer kind");
    for (int64_t j = label_offsets[i]; j < label_offsets[i + 1]; ++j)
      if (!std::isfinite(probs[j]) || probs[j] < 0.f)
        return fail(JEV_EINVAL, "branch " + std::to_string(i) + ": probability not finite and >= 0");
  }
  for (int32_t i = 0; i < n; ++i) {
    const jev::Answer a = jev::answer(kinds[i], probs + label_offsets[i],
                                      int32_t(label_offsets[i + 1] - label_offsets[i]));
    value[i] = a.value;
    if (choice) choice[i] = a.choice;
    if (confidence) confidence[i] = a.confidence;
  }
  return JEV_OK;
}

size_t jev_workspace_bytes(const jev_model_desc* desc) {
  std::string why;
  if (!desc_ok(desc, &why)) return 0;
  return layout(*desc).total;
}

size_t jev_kv_pool_bytes(const jev_model_desc* desc, int32_t n_pages) {
  std::string why;
  if (!desc_ok(desc, &why) || n_pages < 0) return 0;
  return size_t(desc->n_layers) * size_t(n_pages) * desc->n_kv_heads * 2 * jev::kPage * desc->head_dim *
         elt_size(*desc);
}

int jev_create(const jev_model_desc* desc, const jev_weights* weights, void* kv_pool, int32_t n_pages,
               void* workspace, size_t workspace_bytes, jev_ctx** out) {
  std::string why;
  if (!out) return fail(JEV_EINVAL, "out is NULL");
  *out = nullptr;
  if (!desc_ok(desc, &why)) return fail(JEV_EINVAL, why);
  if (n_pages < 1 || n_pages > (1 << 26)) return fail(JEV_EINVAL, "n_pages must be in [1, 2^26]");
  std::unique_ptr<jev_ctx> c(new jev_ctx());
  jev_ctx* ctx = c.get();
  ctx->desc = *desc;
  ctx->pages.reset(n_pages);
  ctx->tree.reset(new jev::ResidentTree(&ctx->pages));
  ctx->dims = jev::ModelDims{desc->n_layers, desc->d_model, desc->n_q_heads, desc->n_kv_heads,
                             desc->head_dim, desc->vocab,  n_pages,          desc->rms_eps,
                             desc->dtype == JEV_DTYPE_BF16 ? 1 : 0};
  ctx->L = layout(*desc);
  ctx->stats.pages_total = n_pages;
  const bool dry = !weights && !kv_pool && !workspace;
  ctx->dry = dry;
  if (!dry) {
    if (!weights || !kv_pool || !workspace) return fail(JEV_EINVAL, "weights, kv_pool and workspace are all required");
    if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(JEV_EINVAL, "workspace must be 256-byte aligned");
    if (workspace_bytes < ctx->L.total)
      return fail(JEV_ENOMEM, "workspace too small: need " + std::to_string(ctx->L.total) + " bytes");
    if (!weights->embed || !weights->unembed || !weights->final_norm || !weights->attn_norm || !weights->wq ||
        !weights->wk || !weights->wv || !weights->wo)
      return fail(JEV_EINVAL, "NULL weight pointer");
    ctx->embed = weights->embed;
    ctx->unembed = weights->unembed;
    ctx->final_norm = weights->final_norm;
    for (int l = 0; l < desc->n_layers; ++l) {
      jev::LayerW w{weights->attn_norm[l], weights->wq[l], weights->wk[l], weights->wv[l], weights->wo[l]};
      if (!w.norm || !w.wq || !w.wk || !w.wv || !w.wo) return fail(JEV_EINVAL, "NULL per-layer weight pointer");
      ctx->layers.push_back(w);
    }
    ctx->pool = reinterpret_cast<char*>(kv_pool);
    ctx->ws = reinterpret_cast<char*>(workspace);
    if (int rc = device_scratch(&ctx->static_scratch)) return rc;
    HIPCHK(hipHostMalloc(reinterpret_cast<void**>(&ctx->desc_host), 2 * size_t(ctx->L.desc_ints) * sizeof(int32_t),
                         hipHostMallocDefault));
    HIPCHK(hipHostGetDevicePointer(reinterpret_cast<void**>(&ctx->desc_host_dev), ctx->desc_host, 0));
    for (hipEvent_t& e : ctx->done_ev) HIPCHK(hipEventCreateWithFlags(&e, hipEventDisableTiming));
    ctx->last_done = ctx->done_ev[0];
    // RoPE table: angle = pos * theta^(-2i/dh) in double, stored as float (cos, sin)
    const int half = desc->head_dim / 2;
    std::vector<float> rope(size_t(desc->max_positions) * half * 2);
    for (int64_t p = 0; p < desc->max_positions; ++p)
      for (int i = 0; i < half; ++i) {
        const double inv = std::pow(double(desc->rope_theta), -2.0 * i / desc->head_dim);
        const double a = double(p) * inv;
        rope[(size_t(p) * half + i) * 2] = float(std::cos(a));
        rope[(size_t(p) * half + i) * 2 + 1] = float(std::sin(a));
      }
    HIPCHK(hipMemcpy(ctx->ws + ctx->L.rope, rope.data(), rope.size() * sizeof(float), hipMemcpyHostToDevice));
    // pages never written hold zeros (a partly valid page is masked, never NaN)
    HIPCHK(hipMemset(kv_pool, 0, jev_kv_pool_bytes(desc, n_pages)));
    HIPCHK(hipDeviceSynchronize());
  }
  *out = c.release();
  return JEV_OK;
}

static void detach_sched(jev_sched* s);

int jev_destroy(jev_ctx* ctx) {
  if (!ctx) return JEV_OK;
  int rc = JEV_OK;
  // schedulers still alive lose their context (their handles stay valid until
  // jev_sched_destroy, which then only frees them)
  for (jev_sched* s : ctx->scheds) detach_sched(s);
  ctx->scheds.clear();
  if (!ctx->dry) {
    if (ctx->have_last && hipEventSynchronize(ctx->last_done) != hipSuccess) rc = fail(JEV_EHIP, "sync failed");
    if (ctx->desc_host) (void)hipHostFree(ctx->desc_host);
    for (hipEvent_t e : ctx->done_ev)
      if (e) (void)hipEventDestroy(e);
    for (auto& p : ctx->prof) {
      (void)hipEventDestroy(p.e0);
      (void)hipEventDestroy(p.e1);
    }
    for (hipEvent_t e : ctx->prof_free) (void)hipEventDestroy(e);
    for (hipEvent_t e : ctx->round_ev) (void)hipEventDestroy(e);
  }
  delete ctx;
  return rc;
}

int jev_prefill_prefix(jev_ctx* ctx, int32_t n, const jev_prefix* parents, const int32_t* tokens,
                       const int64_t* offsets, jev_prefix* out_handles, void* hip_stream) {
  if (int rc = check_alive(ctx)) return rc;
  if (int rc = check_segments(ctx, n, tokens, offsets, "prefill")) return rc;
  if (n == 0) return JEV_OK;
  if (!parents || !out_handles) return fail(JEV_EINVAL, "NULL parents/out_handles");
  begin_call(ctx, JEV_CALL_PREFILL);
  const std::set<int32_t> free_before = poison_before(ctx);
  std::vector<jev::ResidentTree::PrefillItem> items;
  for (int32_t i = 0; i < n; ++i) {
    if (!ctx->tree->has(parents[i])) return fail(JEV_EHANDLE, "unknown parent handle " + std::to_string(parents[i]));
    const int64_t len = offsets[i + 1] - offsets[i];
    if (ctx->tree->end_pos(parents[i]) + len > ctx->desc.max_positions)
      return fail(JEV_EINVAL, "prefix " + std::to_string(i) + " runs past max_positions");
    items.push_back({parents[i], tokens + offsets[i], len});
  }
  std::vector<int64_t> victims;
  {
    std::vector<int64_t> used;
    for (const auto& it : items) {
      used.push_back(it.parent);
      if (int64_t c = ctx->tree->find_child(it.parent, it.tok, it.n)) used.push_back(c);
    }
    if (int rc = find_room(ctx, path_set(*ctx->tree, used),
                           [&](const jev::ResidentTree& t, jev::PagePool& p) {
                             return t.prefill_need(items) <= p.n_free();
                           },
                           "not enough free KV pages", &victims))
      return rc;
  }
  // Simulate the allocation tree->prefill() will make after the evictions
  // (new nodes take the lowest free ids in input order; an identical resident
  // child or an earlier identical item of this call creates nothing), so that
  // descriptors are built and checked before any state changes.
  std::vector<RNode> rn;
  {
    std::set<int32_t> snap = ctx->pages.snapshot();
    release_victim_pages(ctx, victims);
    std::vector<size_t> made;  // indices of items that create a node
    for (int32_t i = 0; i < n; ++i) {
      const auto& it = items[i];
      bool exists = ctx->tree->prefill_need({it}) == 0;
      for (size_t j : made)
        if (!exists && items[j].parent == it.parent && items[j].n == it.n &&
            std::equal(it.tok, it.tok + it.n, items[j].tok))
          exists = true;
      if (exists) continue;
      made.push_back(size_t(i));
      RNode nd;
      nd.group = it.parent;
      if (it.parent != 0) nd.anc = ctx->tree->path_pages(it.parent);
      nd.tok = it.tok;
      nd.n = it.n;
      nd.start = ctx->tree->end_pos(it.parent);
      nd.pages = ctx->pages.alloc(jev::pages_for(it.n));
      rn.push_back(std::move(nd));
    }
    ctx->pages.restore(std::move(snap));
  }
  std::vector<int32_t> hb;
  std::vector<RoundDesc> rds(1);
  int64_t computed = 0;
  for (auto& nd : rn) computed += nd.n;
  if (!rn.empty() && !ctx->dry) {
    if (int rc = build_round(ctx, rn, hb, &rds[0])) return rc;
    if (int64_t(hb.size()) > ctx->L.desc_ints)
      return fail(JEV_ENOMEM, "call descriptors exceed the workspace descriptor region");
  }
  // commit the evictions and the tree change, then run (the tree allocates the
  // same lowest ids)
  for (int64_t v : victims) ctx->tree->evict(v);
  std::vector<int64_t> handles;
  std::vector<char> created;
  ctx->tree->prefill(items, &handles, &created);
  ctx->clock += 1;
  for (int32_t i = 0; i < n; ++i) {
    out_handles[i] = handles[i];
    ctx->tree->touch_path(handles[i], ctx->clock);
  }
  ctx->stats.logical_tokens = computed;
  ctx->stats.computed_tokens = computed;
  ctx->stats.cached_tokens = 0;
  ctx->stats.rounds = rn.empty() ? 0 : 1;
  ctx->stats.calls += 1;
  const hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  if (!rn.empty() && !ctx->dry) {
    if (int rc = run_rounds(ctx, rds, hb, nullptr, st, ws_scratch(ctx))) return rc;
    return poison_after(ctx, free_before, ctx->call_written, st);
  }
  return poison_after(ctx, free_before, {}, st);  // evictions only
}

namespace {

// jev_score_branches and its allocation-free variant: everything is checked
// and every descriptor built before any state changes.
int score_branches(jev_ctx* ctx, int32_t n, const jev_prefix* parents, const int32_t* tokens,
                   const int64_t* tok_offsets, const int32_t* label_ids, const int64_t* label_offsets, float* probs,
                   void* hip_stream, bool noalloc) {
  if (int rc = check_alive(ctx)) return rc;
  if (int rc = check_segments(ctx, n, tokens, tok_offsets, "branches")) return rc;
  if (n == 0) return JEV_OK;
  if (!parents) return fail(JEV_EINVAL, "NULL parents");
  if (int rc = check_labels(ctx, n, label_ids, label_offsets)) return rc;
  if (ctx->dry) return fail(JEV_ESTATE, "scoring needs a device context");
  if (!probs) return fail(JEV_EINVAL, "NULL probs");
  begin_call(ctx, JEV_CALL_BRANCHES);
  const std::set<int32_t> free_before = poison_before(ctx);
  int64_t need = 0, logical = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (!ctx->tree->has(parents[i])) return fail(JEV_EHANDLE, "unknown parent handle " + std::to_string(parents[i]));
    const int64_t len = tok_offsets[i + 1] - tok_offsets[i];
    if (ctx->tree->end_pos(parents[i]) + len > ctx->desc.max_positions)
      return fail(JEV_EINVAL, "branch " + std::to_string(i) + " runs past max_positions");
    need += jev::pages_for(len);
    logical += ctx->tree->end_pos(parents[i]) + len;
  }
  const std::vector<int64_t> used(parents, parents + n);
  std::vector<int64_t> victims;
  if (int rc = find_room(ctx, path_set(*ctx->tree, used),
                         [&](const jev::ResidentTree&, jev::PagePool& p) { return need <= p.n_free(); },
                         "not enough free KV pages", &victims))
    return rc;
  // branch pages live for this call only: allocated on the pool as it will be
  // after the evictions, then the pool is restored
  std::set<int32_t> snap = ctx->pages.snapshot();
  release_victim_pages(ctx, victims);
  std::vector<RNode> rn;
  std::map<int64_t, std::vector<jev::PageRef>> anc_cache;
  int64_t computed = 0;
  for (int32_t i = 0; i < n; ++i) {
    RNode nd;
    nd.group = parents[i];
    if (parents[i] != 0) {
      auto it = anc_cache.find(parents[i]);
      if (it == anc_cache.end()) it = anc_cache.emplace(parents[i], ctx->tree->path_pages(parents[i])).first;
      nd.anc = it->second;
    }
    nd.tok = tokens + tok_offsets[i];
    nd.n = tok_offsets[i + 1] - tok_offsets[i];
    nd.start = ctx->tree->end_pos(parents[i]);
    nd.pages = ctx->pages.alloc(jev::pages_for(nd.n));
    nd.reads.push_back(ReadSpec{i, label_ids + label_offsets[i], int32_t(label_offsets[i + 1] - label_offsets[i]),
                                label_offsets[i]});
    computed += nd.n;
    rn.push_back(std::move(nd));
  }
  ctx->pages.restore(std::move(snap));
  std::vector<int32_t> hb;
  std::vector<RoundDesc> rds(1);
  if (int rc = build_round(ctx, rn, hb, &rds[0])) return rc;
  if (int64_t(hb.size()) > ctx->L.desc_ints)
    return fail(JEV_ENOMEM, "call descriptors exceed the workspace descriptor region");
  Scratch sc = ws_scratch(ctx);
  if (noalloc)
    if (int rc = static_scratch_for(ctx, rds, &sc)) return rc;
  // commit: evictions, recency, statistics
  for (int64_t v : victims) ctx->tree->evict(v);
  ctx->clock += 1;
  for (int64_t h : used) ctx->tree->touch_path(h, ctx->clock);
  ctx->stats.logical_tokens = logical;
  ctx->stats.computed_tokens = computed;
  ctx->stats.cached_tokens = logical - computed;
  ctx->stats.rounds = 1;
  ctx->stats.calls += 1;
  const hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  if (int rc = run_rounds(ctx, rds, hb, probs, st, sc)) return rc;
  return poison_after(ctx, free_before, ctx->call_written, st);
}

}  // namespace

int jev_score_branches(jev_ctx* ctx, int32_t n, const jev_prefix* parents, const int32_t* tokens,
                       const int64_t* tok_offsets, const int32_t* label_ids, const int64_t* label_offsets,
                       float* probs, void* hip_stream) {
  return score_branches(ctx, n, parents, tokens, tok_offsets, label_ids, label_offsets, probs, hip_stream, false);
}

int jev_score_branches_noalloc(jev_ctx* ctx, int32_t n, const jev_prefix* parents, const int32_t* tokens,
                               const int64_t* tok_offsets, const int32_t* label_ids, const int64_t* label_offsets,
                               float* probs, void* hip_stream) {
  return score_branches(ctx, n, parents, tokens, tok_offsets, label_ids, label_offsets, probs, hip_stream, true);
}

// The nodes of round r of a candidate plan, as the executor takes them;
// returns their token count.  Candidate c's labels are
// label_ids[label_offsets[c] ..) and its probabilities go to probs at the same
// offsets.
static int64_t plan_round_nodes(const jev::ResidentTree& tree, const jev::Plan& plan, size_t r, const int32_t* tokens,
                         const int64_t* tok_offsets, const int32_t* label_ids, const int64_t* label_offsets,
                         std::map<int64_t, std::vector<jev::PageRef>>* anchor_pages, std::vector<RNode>* out) {
  int64_t computed = 0;
  for (int32_t idx : plan.rounds[r]) {
    const jev::PlanNode& x = plan.nodes[idx];
    RNode nd;
    const int32_t c0 = x.cand_min();
    const int64_t alen = plan.anchor_len[c0];
    // group: parent node id within the plan, or the anchor handle (negated, offset)
    nd.group = x.parent >= 0 ? int64_t(plan.nodes[x.parent].id) : -1 - x.anchor;
    if (x.anchor != 0) {
      auto it = anchor_pages->find(x.anchor);
      if (it == anchor_pages->end()) it = anchor_pages->emplace(x.anchor, tree.path_pages(x.anchor)).first;
      nd.anc = it->second;
    }
    // plan ancestors, root first
    std::vector<int32_t> chain;
    for (int32_t p = x.parent; p >= 0; p = plan.nodes[p].parent) chain.push_back(p);
    for (auto it = chain.rbegin(); it != chain.rend(); ++it) {
      const jev::PlanNode& a = plan.nodes[*it];
      const int64_t L = a.b - a.a;
      for (size_t pi = 0; pi < a.pages.size(); ++pi) {
        const int64_t v = L - int64_t(jev::kPage) * int64_t(pi);
        nd.anc.push_back(jev::PageRef{a.pages[pi], int32_t(v < jev::kPage ? v : jev::kPage)});
      }
    }
    nd.tok = tokens + tok_offsets[c0] + alen + x.a;
    nd.n = x.b - x.a;
    nd.start = alen + x.a;
    nd.pages = x.pages;
    for (int32_t c : x.readout)
      nd.reads.push_back(ReadSpec{c, label_ids + label_offsets[c], int32_t(label_offsets[c + 1] - label_offsets[c]),
                                  label_offsets[c]});
    computed += nd.n;
    out->push_back(std::move(nd));
  }
  return computed;
}

int jev_score_candidates(jev_ctx* ctx, int32_t n, const int32_t* tokens, const int64_t* tok_offsets,
                         const int32_t* label_ids, const int64_t* label_offsets, float* probs, void* hip_stream) {
  if (int rc = check_alive(ctx)) return rc;
  if (int rc = check_segments(ctx, n, tokens, tok_offsets, "candidates")) return rc;
  if (n == 0) return JEV_OK;
  if (int rc = check_labels(ctx, n, label_ids, label_offsets)) return rc;
  if (ctx->dry) return fail(JEV_ESTATE, "scoring needs a device context");
  if (!probs) return fail(JEV_EINVAL, "NULL probs");
  for (int32_t i = 0; i < n; ++i)
    if (tok_offsets[i + 1] - tok_offsets[i] > ctx->desc.max_positions)
      return fail(JEV_EINVAL, "candidate " + std::to_string(i) + " runs past max_positions");
  begin_call(ctx, JEV_CALL_CANDIDATES);
  const std::set<int32_t> free_before = poison_before(ctx);
  // the tree work (splits, evictions, the plan) on copies; the rounds and
  // their descriptors are built against the copies, which are committed only
  // once every check has passed
  jev::Plan plan;
  jev::PagePool pool;
  jev::ResidentTree tree(&pool);
  if (int rc = stage_candidates(ctx, n, tokens, tok_offsets, &pool, &tree, &plan, ctx->plan_mode)) return rc;
  std::vector<std::vector<RNode>> rounds(plan.rounds.size());
  std::map<int64_t, std::vector<jev::PageRef>> anchor_pages;
  int64_t computed = 0, logical = 0;
  for (int32_t c = 0; c < n; ++c) logical += tok_offsets[c + 1] - tok_offsets[c];
  for (size_t r = 0; r < plan.rounds.size(); ++r)
    computed += plan_round_nodes(tree, plan, r, tokens, tok_offsets, label_ids, label_offsets, &anchor_pages,
                                 &rounds[r]);
  std::vector<int32_t> hb;
  std::vector<RoundDesc> rds(rounds.size());
  for (size_t r = 0; r < rounds.size(); ++r)
    if (int rc = build_round(ctx, rounds[r], hb, &rds[r])) return rc;
  if (int64_t(hb.size()) > ctx->L.desc_ints)
    return fail(JEV_ENOMEM, "call descriptors exceed the workspace descriptor region");
  ctx->pages = pool;
  *ctx->tree = std::move(tree);
  ctx->tree->rebind(&ctx->pages);
  ctx->clock += 1;
  for (int64_t h : plan.anchors) ctx->tree->touch_path(h, ctx->clock);
  ctx->stats.logical_tokens = logical;
  ctx->stats.computed_tokens = computed;
  ctx->stats.cached_tokens = logical - computed;
  ctx->stats.rounds = int32_t(rounds.size());
  ctx->stats.calls += 1;
  if (ctx->tree->keep()) {
    // Automatic checkpoints (cache policy on): the call's nodes with children,
    // i.e. the prefixes its candidates share, stay resident as cached
    // prefixes (no reference) holding the pages the call writes, so a later
    // call over the same state reuses them.  Parents come before
    // children.  Done once nothing can fail before the rounds run.
    std::vector<int64_t> handle_of(plan.nodes.size(), 0);
    std::vector<int64_t> made;
    for (const auto& rnd : plan.rounds)
      for (int32_t idx : rnd) {
        const jev::PlanNode& x = plan.nodes[idx];
        if (x.children.empty()) continue;
        const int64_t parent = x.parent >= 0 ? handle_of[size_t(x.parent)] : x.anchor;
        const int32_t c0 = x.cand_min();
        const int64_t h = ctx->tree->adopt(parent, tokens + tok_offsets[c0] + plan.anchor_len[c0] + x.a, x.b - x.a,
                                           x.pages);
        if (h == 0) {
          ctx->dead = true;
          return fail(JEV_ESTATE, "internal: a planned page is not free");
        }
        handle_of[size_t(idx)] = h;
        ctx->tree->touch_path(h, ctx->clock);
        made.push_back(h);
      }
    for (int64_t h : made) ctx->tree->release(h);
  }
  const hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  if (int rc = run_rounds(ctx, rds, hb, probs, st, ws_scratch(ctx))) return rc;
  return poison_after(ctx, free_before, ctx->call_written, st);
}

// ----------------------------------------------------------------- scheduler
// Round-level continuous batching (see jev.h).  submit/status/result take the
// mutex and touch only the request lists; step is the single driver of the
// context.

struct jev_sched {
  jev_ctx* ctx = nullptr;
  std::mutex mu;
  struct Req {
    int64_t ticket = 0;
    std::vector<int32_t> tok, lab;
    std::vector<int64_t> off, loff;
    std::vector<char> done;
    std::vector<float> probs;  // host, in label_offsets layout
    bool started = false;      // took part in a step
  };
  std::vector<std::unique_ptr<Req>> queued;            // submitted, not yet stepped
  std::vector<std::unique_ptr<Req>> active;            // step thread only
  std::map<int64_t, std::unique_ptr<Req>> finished;    // until their result is taken
  std::set<int64_t> active_tickets;                    // under mu
  std::vector<int64_t> held;                           // resident handles the scheduler holds
  int64_t next_ticket = 1;
  int32_t n_pages = 0;  // the context's page count (fixed at creation)
  float* dprobs = nullptr;
  int64_t dprobs_cap = 0;
};

int jev_sched_create(jev_ctx* ctx, jev_sched** out) {
  if (int rc = check_alive(ctx)) return rc;
  if (!out) return fail(JEV_EINVAL, "NULL out");
  auto* s = new jev_sched();
  s->ctx = ctx;
  s->n_pages = ctx->pages.n_total();
  ctx->scheds.push_back(s);
  *out = s;
  return JEV_OK;
}

// The context of s is going away: its device buffer is freed and it forgets
// the context (the held prefixes go with the context's tree).
static void detach_sched(jev_sched* s) {
  jev_ctx* ctx = s->ctx;
  if (!ctx) return;
  if (!ctx->dry && ctx->have_last) (void)hipEventSynchronize(ctx->last_done);
  if (s->dprobs) (void)hipFree(s->dprobs);
  s->dprobs = nullptr;
  s->dprobs_cap = 0;
  s->held.clear();
  s->ctx = nullptr;
}

int jev_sched_destroy(jev_sched* s) {
  if (!s) return JEV_OK;
  jev_ctx* ctx = s->ctx;
  int rc = JEV_OK;
  if (ctx) {
    if (!ctx->dry && ctx->have_last && hipEventSynchronize(ctx->last_done) != hipSuccess)
      rc = fail(JEV_EHIP, "sync failed");
    const std::set<int32_t> free_before = poison_before(ctx);
    for (int64_t h : s->held) ctx->tree->release(h);
    if (rc == JEV_OK && !ctx->dead)
      rc = poison_after(ctx, free_before, {}, ctx->have_last ? ctx->last_stream : nullptr);
    if (s->dprobs) (void)hipFree(s->dprobs);
    ctx->scheds.erase(std::remove(ctx->scheds.begin(), ctx->scheds.end(), s), ctx->scheds.end());
  }
  delete s;
  return rc;
}

int jev_sched_submit(jev_sched* s, int32_t n, const int32_t* tokens, const int64_t* tok_offsets,
                     const int32_t* label_ids, const int64_t* label_offsets, int64_t* ticket) {
  if (!s || !ticket) return fail(JEV_EINVAL, "NULL scheduler or ticket");
  const jev_ctx* ctx = s->ctx;
  if (!ctx) return fail(JEV_ESTATE, "the scheduler's context was destroyed");
  if (n < 1) return fail(JEV_EINVAL, "a request needs at least one candidate");
  if (int rc = check_segments(ctx, n, tokens, tok_offsets, "candidates")) return rc;
  if (int rc = check_labels(ctx, n, label_ids, label_offsets)) return rc;
  for (int32_t i = 0; i < n; ++i)
    if (tok_offsets[i + 1] - tok_offsets[i] > ctx->desc.max_positions)
      return fail(JEV_EINVAL, "candidate " + std::to_string(i) + " runs past max_positions");
  {
    // a request that cannot run even alone on an empty pool would wait forever
    jev::PagePool pool(s->n_pages);
    jev::ResidentTree tree(&pool);
    jev::Plan plan;
    if (!jev::plan_candidates(tree, &pool, n, tokens, tok_offsets, &plan, jev::PlanMode::DEPTH))
      return fail(JEV_ENOMEM, "the request does not fit the page pool even alone");
  }
  auto r = std::make_unique<jev_sched::Req>();
  r->tok.assign(tokens, tokens + tok_offsets[n]);
  r->off.assign(tok_offsets, tok_offsets + n + 1);
  r->lab.assign(label_ids, label_ids + label_offsets[n]);
  r->loff.assign(label_offsets, label_offsets + n + 1);
  r->done.assign(size_t(n), 0);
  r->probs.assign(size_t(label_offsets[n]), 0.f);
  std::lock_guard<std::mutex> lk(s->mu);
  r->ticket = s->next_ticket++;
  *ticket = r->ticket;
  s->queued.push_back(std::move(r));
  return JEV_OK;
}

int jev_sched_status(jev_sched* s, int64_t ticket, int32_t* state) {
  if (!s || !state) return fail(JEV_EINVAL, "NULL scheduler or state");
  std::lock_guard<std::mutex> lk(s->mu);
  for (const auto& r : s->queued)
    if (r->ticket == ticket) return *state = JEV_SCHED_QUEUED, JEV_OK;
  if (s->active_tickets.count(ticket)) return *state = JEV_SCHED_ACTIVE, JEV_OK;
  if (s->finished.count(ticket)) return *state = JEV_SCHED_FINISHED, JEV_OK;
  return fail(JEV_EHANDLE, "unknown or collected ticket " + std::to_string(ticket));
}

int jev_sched_result(jev_sched* s, int64_t ticket, float* probs, int64_t cap) {
  if (!s) return fail(JEV_EINVAL, "NULL scheduler");
  std::lock_guard<std::mutex> lk(s->mu);
  auto it = s->finished.find(ticket);
  if (it == s->finished.end()) {
    for (const auto& r : s->queued)
      if (r->ticket == ticket) return fail(JEV_EPENDING, "request " + std::to_string(ticket) + " not finished");
    if (s->active_tickets.count(ticket)) return fail(JEV_EPENDING, "request " + std::to_string(ticket) + " not finished");
    return fail(JEV_EHANDLE, "unknown or collected ticket " + std::to_string(ticket));
  }
  if (!s->ctx) return fail(JEV_ESTATE, "the scheduler's context was destroyed");
  if (s->ctx->dry) return fail(JEV_ESTATE, "no scores on a planning-only context");
  const std::vector<float>& p = it->second->probs;
  if (!probs || cap < int64_t(p.size())) return fail(JEV_EINVAL, "probs NULL or cap below the request's label count");
  std::memcpy(probs, p.data(), p.size() * sizeof(float));
  s->finished.erase(it);
  return JEV_OK;
}

int jev_sched_step(jev_sched* s, void* hip_stream, int32_t* plan_out, int64_t plan_cap, int64_t* plan_n) {
  if (!s) return fail(JEV_EINVAL, "NULL scheduler");
  jev_ctx* ctx = s->ctx;
  if (!ctx) return fail(JEV_ESTATE, "the scheduler's context was destroyed");
  if (int rc = check_alive(ctx)) return rc;
  if (plan_n) *plan_n = 0;
  begin_call(ctx, JEV_CALL_SCHED_STEP);
  const std::set<int32_t> free_before = poison_before(ctx);
  bool ran = false;
  {
    std::lock_guard<std::mutex> lk(s->mu);
    for (auto& r : s->queued) {
      s->active_tickets.insert(r->ticket);
      s->active.push_back(std::move(r));
    }
    s->queued.clear();
  }
  // this step's candidates: unfinished ones of the included requests, in
  // order.  All active requests are included; while the plan does not fit,
  // the newest request that has not started yet waits for a later step.
  struct Ref {
    size_t req;
    int32_t cand;
  };
  std::vector<char> incl(s->active.size(), 1);
  std::vector<Ref> refs;
  std::vector<int32_t> tok, lab;
  std::vector<int64_t> off, loff;
  jev::Plan plan;
  jev::PagePool pool;
  jev::ResidentTree tree(&pool);
  for (;;) {
    refs.clear();
    tok.clear();
    lab.clear();
    off.assign(1, 0);
    loff.assign(1, 0);
    for (size_t ri = 0; ri < s->active.size(); ++ri) {
      if (!incl[ri]) continue;
      const auto& r = *s->active[ri];
      for (int32_t c = 0; c + 1 < int32_t(r.off.size()); ++c) {
        if (r.done[size_t(c)]) continue;
        refs.push_back(Ref{ri, c});
        tok.insert(tok.end(), r.tok.begin() + r.off[size_t(c)], r.tok.begin() + r.off[size_t(c) + 1]);
        off.push_back(int64_t(tok.size()));
        lab.insert(lab.end(), r.lab.begin() + r.loff[size_t(c)], r.lab.begin() + r.loff[size_t(c) + 1]);
        loff.push_back(int64_t(lab.size()));
      }
    }
    if (refs.empty()) return JEV_OK;
    const int rc = stage_candidates(ctx, int32_t(refs.size()), tok.data(), off.data(), &pool, &tree, &plan,
                                    jev::PlanMode::DEPTH);
    if (rc == JEV_OK) break;
    if (rc != JEV_ENOMEM) return rc;
    size_t drop = s->active.size();
    for (size_t ri = s->active.size(); ri-- > 0;)
      if (incl[ri] && !s->active[ri]->started) {
        drop = ri;
        break;
      }
    if (drop == s->active.size()) return rc;  // the started requests alone do not fit
    incl[drop] = 0;
  }
  if (plan_out) {
    const std::vector<int32_t> img = plan.serialize();
    if (plan_cap < int64_t(img.size())) return fail(JEV_EINVAL, "plan_out too small");
    std::copy(img.begin(), img.end(), plan_out);
    if (plan_n) *plan_n = int64_t(img.size());
  }
  // the first round, against the staged tree (anchors may be split heads)
  std::vector<RNode> rn;
  std::map<int64_t, std::vector<jev::PageRef>> anchor_pages;
  const int64_t computed =
      plan_round_nodes(tree, plan, 0, tok.data(), off.data(), lab.data(), loff.data(), &anchor_pages, &rn);
  std::vector<int32_t> hb;
  std::vector<RoundDesc> rds(1);
  if (!ctx->dry) {
    if (int rc = build_round(ctx, rn, hb, &rds[0])) return rc;
    if (int64_t(hb.size()) > ctx->L.desc_ints)
      return fail(JEV_ENOMEM, "call descriptors exceed the workspace descriptor region");
    if (s->dprobs_cap < loff.back()) {
      if (s->dprobs) HIPCHK(hipFree(s->dprobs));
      s->dprobs = nullptr;
      s->dprobs_cap = 0;
      if (hipMalloc(reinterpret_cast<void**>(&s->dprobs), size_t(loff.back()) * sizeof(float)) != hipSuccess)
        return fail(JEV_ENOMEM, "device buffer for the step's probabilities");
      s->dprobs_cap = loff.back();
    }
  }
  // commit: the staged tree and pool, then the round's nodes with children
  // become resident nodes held by the scheduler
  ctx->pages = pool;
  *ctx->tree = std::move(tree);
  ctx->tree->rebind(&ctx->pages);
  ctx->clock += 1;
  for (int64_t h : plan.anchors) ctx->tree->touch_path(h, ctx->clock);
  for (size_t ri = 0; ri < s->active.size(); ++ri)
    if (incl[ri]) s->active[ri]->started = true;
  for (int32_t idx : plan.rounds[0]) {
    const jev::PlanNode& x = plan.nodes[idx];
    if (x.children.empty()) continue;
    const int32_t c0 = x.cand_min();
    const int64_t h =
        ctx->tree->adopt(x.anchor, tok.data() + off[c0] + plan.anchor_len[c0] + x.a, x.b - x.a, x.pages);
    if (h == 0) {
      ctx->dead = true;
      return fail(JEV_ESTATE, "internal: a planned page is not free");
    }
    ctx->tree->touch_path(h, ctx->clock);
    s->held.push_back(h);
  }
  int64_t logical = 0;
  for (int32_t idx : plan.rounds[0])
    for (int32_t c : plan.nodes[idx].readout) logical += off[c + 1] - off[c];
  ctx->stats.logical_tokens = logical;
  ctx->stats.computed_tokens = computed;
  ctx->stats.cached_tokens = logical - computed;
  ctx->stats.rounds = 1;
  ctx->stats.calls += 1;
  if (!ctx->dry) {
    const hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    if (int rc = run_rounds(ctx, rds, hb, s->dprobs, st, ws_scratch(ctx))) return rc;
    ran = true;
    std::vector<float> hp(size_t(loff.back()));
    HIPCHK(hipMemcpyAsync(hp.data(), s->dprobs, hp.size() * sizeof(float), hipMemcpyDeviceToHost, st));
    HIPCHK(hipStreamSynchronize(st));
    for (int32_t idx : plan.rounds[0])
      for (int32_t c : plan.nodes[idx].readout) {
        auto& r = *s->active[refs[size_t(c)].req];
        const int32_t rc_ = refs[size_t(c)].cand;
        std::copy(hp.begin() + loff[c], hp.begin() + loff[c + 1], r.probs.begin() + r.loff[size_t(rc_)]);
      }
  }
  for (int32_t idx : plan.rounds[0])
    for (int32_t c : plan.nodes[idx].readout) s->active[refs[size_t(c)].req]->done[size_t(refs[size_t(c)].cand)] = 1;
  {
    std::vector<std::unique_ptr<jev_sched::Req>> still;
    std::lock_guard<std::mutex> lk(s->mu);
    for (auto& r : s->active) {
      bool all = true;
      for (char d : r->done) all = all && d;
      if (all) {
        s->active_tickets.erase(r->ticket);
        s->finished.emplace(r->ticket, std::move(r));
      } else {
        still.push_back(std::move(r));
      }
    }
    s->active = std::move(still);
  }
  // release held nodes that no unfinished candidate of a started request
  // passes through (a waiting request does not pin them: it might never fit
  // beside them)
  std::set<int64_t> needed;
  for (const auto& r : s->active)
    for (int32_t c = 0; r->started && c + 1 < int32_t(r->off.size()); ++c) {
      if (r->done[size_t(c)]) continue;
      int64_t h, m;
      ctx->tree->match(r->tok.data() + r->off[size_t(c)], r->off[size_t(c) + 1] - r->off[size_t(c)], &h, &m);
      for (; h != 0 && !needed.count(h); h = ctx->tree->node(h).parent) needed.insert(h);
    }
  std::vector<int64_t> keep;
  for (int64_t h : s->held) {
    if (needed.count(h))
      keep.push_back(h);
    else
      ctx->tree->release(h);
  }
  s->held = std::move(keep);
  return poison_after(ctx, free_before, ran ? ctx->call_written : std::vector<int32_t>{},
                      reinterpret_cast<hipStream_t>(hip_stream));
}

int jev_set_plan_mode(jev_ctx* ctx, int32_t mode) {
  if (!ctx) return fail(JEV_EINVAL, "ctx is NULL");
  if (mode != JEV_PLAN_DEPTH && mode != JEV_PLAN_CANDIDATE_FIRST) return fail(JEV_EINVAL, "unknown plan mode");
  ctx->plan_mode = mode == JEV_PLAN_DEPTH ? jev::PlanMode::DEPTH : jev::PlanMode::CANDIDATE_FIRST;
  return JEV_OK;
}

int jev_set_cache_policy(jev_ctx* ctx, int32_t policy) {
  if (!ctx) return fail(JEV_EINVAL, "ctx is NULL");
  if (policy != JEV_CACHE_RELEASE && policy != JEV_CACHE_LRU) return fail(JEV_EINVAL, "unknown cache policy");
  ctx->tree->set_keep(policy == JEV_CACHE_LRU);
  if (policy == JEV_CACHE_RELEASE)
    while (ctx->tree->evict_one({}) != 0) {
    }
  return JEV_OK;
}

int jev_free_pages(jev_ctx* ctx, int32_t n, const jev_prefix* handles) {
  if (!ctx) return fail(JEV_EINVAL, "ctx is NULL");
  if (n < 0 || (n > 0 && !handles)) return fail(JEV_EINVAL, "bad handle array");
  // validate first: every handle must hold enough caller references
  std::map<int64_t, int64_t> count;
  for (int32_t i = 0; i < n; ++i) {
    if (handles[i] == 0 || !ctx->tree->has(handles[i]))
      return fail(JEV_EHANDLE, "unknown handle " + std::to_string(handles[i]));
    count[handles[i]] += 1;
  }
  for (auto& kv : count)
    if (ctx->tree->node(kv.first).refs < kv.second) return fail(JEV_EHANDLE, "handle released more times than held");
  const std::set<int32_t> free_before = poison_before(ctx);
  ctx->clock += 1;
  for (int32_t i = 0; i < n; ++i) {
    ctx->tree->touch_path(handles[i], ctx->clock);
    ctx->tree->release(handles[i]);
  }
  // freed pages are poisoned after the work already queued that may read them
  if (ctx->dead) return JEV_OK;
  return poison_after(ctx, free_before, {}, ctx->have_last ? ctx->last_stream : nullptr);
}

int jev_plan(jev_ctx* ctx, int32_t n, const int32_t* tokens, const int64_t* tok_offsets, int32_t* out,
             int64_t cap, int64_t* out_len) {
  if (!ctx || !out_len) return fail(JEV_EINVAL, "NULL ctx/out_len");
  if (int rc = check_segments(ctx, n, tokens, tok_offsets, "candidates")) return rc;
  jev::Plan plan;
  if (n > 0) {
    // what jev_score_candidates would do (splits and evictions included), on copies
    jev::PagePool pool;
    jev::ResidentTree tree(&pool);
    if (int rc = stage_candidates(ctx, n, tokens, tok_offsets, &pool, &tree, &plan, ctx->plan_mode)) return rc;
  }
  std::vector<int32_t> s = n > 0 ? plan.serialize() : std::vector<int32_t>{0, 0};
  *out_len = int64_t(s.size());
  if (!out) return JEV_OK;
  if (cap < int64_t(s.size())) return fail(JEV_EINVAL, "output buffer too small");
  std::copy(s.begin(), s.end(), out);
  return JEV_OK;
}

int jev_page_table(jev_ctx* ctx, jev_prefix h, int32_t* page_ids, int32_t* valid, int32_t cap, int32_t* n) {
  if (!ctx || !n) return fail(JEV_EINVAL, "NULL ctx/n");
  if (h == 0 || !ctx->tree->has(h)) return fail(JEV_EHANDLE, "unknown handle");
  std::vector<jev::PageRef> p = ctx->tree->path_pages(h);
  *n = int32_t(p.size());
  if (cap < int32_t(p.size())) return fail(JEV_EINVAL, "output buffer too small");
  for (size_t i = 0; i < p.size(); ++i) {
    if (page_ids) page_ids[i] = p[i].page;
    if (valid) valid[i] = p[i].valid;
  }
  return JEV_OK;
}

int jev_match(jev_ctx* ctx, const int32_t* tokens, int64_t n, jev_prefix* handle, int64_t* matched) {
  if (!ctx || !handle || !matched || (n > 0 && !tokens) || n < 0) return fail(JEV_EINVAL, "bad arguments");
  int64_t h, m;
  ctx->tree->match(tokens, n, &h, &m);
  *handle = h;
  *matched = m;
  return JEV_OK;
}

int jev_stats(jev_ctx* ctx, jev_stats_t* out) {
  if (!ctx || !out) return fail(JEV_EINVAL, "NULL ctx/out");
  ctx->stats.pages_total = ctx->pages.n_total();
  ctx->stats.pages_in_use = ctx->pages.n_total() - ctx->pages.n_free();
  ctx->stats.resident_prefixes = ctx->tree->size();
  ctx->stats.cached_prefixes = ctx->tree->cached_count();
  ctx->stats.cached_pages = ctx->tree->cached_pages();
  ctx->stats.evictions = ctx->tree->evictions();
  ctx->stats.debug_flags = ctx->debug;
  ctx->stats.last_prefill_ms = -1.0;
  ctx->stats.last_branch_ms = -1.0;
  if (ctx->n_round_ev > 1 && !ctx->dead) {
    HIPCHK(hipEventSynchronize(ctx->round_ev[size_t(ctx->n_round_ev - 1)]));
    double pre = 0.0, br = 0.0;
    for (int32_t r = 0; r + 1 < ctx->n_round_ev; ++r) {
      float ms = 0.f;
      HIPCHK(hipEventElapsedTime(&ms, ctx->round_ev[size_t(r)], ctx->round_ev[size_t(r) + 1]));
      (ctx->round_reads[size_t(r)] ? br : pre) += ms;
    }
    ctx->stats.last_prefill_ms = pre;
    ctx->stats.last_branch_ms = br;
  }
  *out = ctx->stats;
  return JEV_OK;
}

int jev_set_round_invariant(jev_ctx* ctx, int32_t on) {
  if (!ctx) return fail(JEV_EINVAL, "ctx is NULL");
  if (on != 0 && on != 1) return fail(JEV_EINVAL, "on must be 0 or 1");
  ctx->round_invariant = on != 0;
  return JEV_OK;
}

int jev_set_gemm_variant(int32_t large, int32_t splits, int32_t bn) {
  if (large < 0 || large > 3) return fail(JEV_EINVAL, "large must be 0..3");
  if (splits < 0 || splits > jev::kMaxSplits) return fail(JEV_EINVAL, "splits must be 0..8");
  if (bn != 0 && bn != 128 && bn != 160) return fail(JEV_EINVAL, "bn must be 0, 128 or 160");
  // 0 selects the loader-wave kernel (the dispatcher's kind 4)
  jev::g_gemm_tuning = jev::GemmTuning{splits, bn, large};
  return JEV_OK;
}

int jev_set_debug(jev_ctx* ctx, uint32_t flags) {
  if (!ctx) return fail(JEV_EINVAL, "ctx is NULL");
  if (flags & ~uint32_t(JEV_DEBUG_POISON_FREED_PAGES | JEV_DEBUG_TIME_CALLS | JEV_DEBUG_FULL_LAST_LAYER))
    return fail(JEV_EINVAL, "unknown debug flag");
  ctx->debug = flags;
  if (!(flags & JEV_DEBUG_TIME_CALLS)) ctx->n_round_ev = 0;
  return JEV_OK;
}

int jev_limits(jev_ctx* ctx, jev_limits_t* out) {
  if (!ctx || !out) return fail(JEV_EINVAL, "NULL ctx/out");
  jev_limits_t l{};
  l.page_tokens = jev::kPage;
  l.min_labels = JEV_MIN_LABELS;
  l.max_labels = JEV_MAX_LABELS;
  l.max_positions = ctx->desc.max_positions;
  l.max_round_tokens = ctx->desc.max_round_tokens;
  l.n_pages = ctx->pages.n_total();
  l.split_k_rows = ctx->round_invariant ? 0 : jev::kSplitRows;
  l.max_tile_pages = jev::kMaxTilePages;
  l.noalloc_scratch_bytes = int64_t(kNoAllocScratchBytes);
  l.noalloc_partial_rows = ctx->dry ? 0 : noalloc_rows(ctx);
  l.workspace_partial_rows = ctx->dry ? 0 : ctx->L.part_rows;
  *out = l;
  return JEV_OK;
}

int jev_debug_tap(jev_ctx* ctx, int32_t what, int32_t layer, void* dst, int64_t cap_rows) {
  if (!ctx) return fail(JEV_EINVAL, "NULL ctx");
  if (!dst) {
    ctx->taps.clear();
    return JEV_OK;
  }
  const int32_t max_layer = what == JEV_TAP_RESID ? ctx->desc.n_layers : ctx->desc.n_layers - 1;
  if ((what != JEV_TAP_ATTN && what != JEV_TAP_RESID) || layer < 0 || layer > max_layer || cap_rows < 1)
    return fail(JEV_EINVAL, "bad tap");
  if (ctx->taps.size() >= 16) return fail(JEV_ENOMEM, "too many taps");
  ctx->taps.push_back({what, layer, dst, cap_rows});
  return JEV_OK;
}

int jev_profile(jev_ctx* ctx, uint32_t kind_mask) { return jev_profile_rows(ctx, kind_mask, 0); }

int jev_profile_rows(jev_ctx* ctx, uint32_t kind_mask, int64_t rows) {
  if (!ctx) return fail(JEV_EINVAL, "NULL ctx");
  if (rows < 0) return fail(JEV_EINVAL, "rows < 0");
  if (ctx->dry) return fail(JEV_ESTATE, "profiling needs a device context");
  if (kind_mask >> JEV_K_COUNT) return fail(JEV_EINVAL, "unknown kernel kind");
  if (kind_mask == 0) {
    if (ctx->have_last) HIPCHK(hipEventSynchronize(ctx->last_done));
    for (auto& p : ctx->prof) {
      ctx->prof_free.push_back(p.e0);
      ctx->prof_free.push_back(p.e1);
    }
    ctx->prof.clear();
  }
  ctx->prof_mask = kind_mask;
  ctx->prof_rows = rows;
  return JEV_OK;
}

int jev_profile_read(jev_ctx* ctx, jev_launch_record* out, int64_t cap, int64_t* n) {
  if (!ctx || !n || cap < 0) return fail(JEV_EINVAL, "bad arguments");
  *n = int64_t(ctx->prof.size());
  const int64_t k = std::min<int64_t>(cap, *n);
  for (int64_t i = 0; i < k; ++i) {
    auto& p = ctx->prof[size_t(i)];
    HIPCHK(hipEventSynchronize(p.e1));
    HIPCHK(hipEventElapsedTime(&p.rec.ms, p.e0, p.e1));
    if (out) out[i] = p.rec;
  }
  return JEV_OK;
}

}  // extern "C"
