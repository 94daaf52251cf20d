// Host-callable launchers of the gfx950 kernels and the descriptor formats the
// host engine fills in.  All pointers are device pointers.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

namespace jev {

// One attention work item: query rows of `n_tok` consecutive round tokens
// starting at `t0` (each token contributes Hq/Hkv rows, one per query head of
// the KV head) against a key list of `n_pages` pages at `page_off` in the
// page-list array (pairs page id, valid slots).  causal: key slot s of list
// page i sits at position kv_pos0 + 16*i + s and is visible to a query at
// position p iff that is <= p; otherwise every valid key is visible.
// out_mode 0: normalised output written straight to the attention output;
// 1: normalised output and log2-sum-exp written to partial slot `part_slot`,
// rows (part_slot*Hkv + kv_head)*128 + token_in_tile*G + head_in_group.
struct AttnTile {
  int32_t t0, n_tok, page_off, n_pages, causal, kv_pos0, out_mode, part_slot;
};

// Merge of the partial states of one round token: n_own parts over its own
// node's pages (slots own_slot0 + c, token own_ti of those tiles; more than one
// when a long causal tile is split into page chunks) and n_anc prefix chunks
// (slots anc_slot0 + c, token anc_ti of those tiles).
constexpr int kMaxOwnParts = 2;
constexpr int kMaxAncParts = 8;
struct MergeItem {
  int32_t t, own_slot0, own_ti, n_own, anc_slot0, anc_ti, n_anc, pad;
};

// Readout of one candidate: final norm of round row `row`, logits at
// labels[label_off .. label_off+k), softmax written to probs[out_off ..].
struct ReadoutItem {
  int32_t row, label_off, k, out_off;
};

struct ModelDims {
  int32_t n_layers, d, hq, hkv, dh, vocab, n_pages;
  float eps;
  int32_t dtype;  // 0 f32, 1 bf16
};

struct LayerW {
  const void* norm;
  const void* wq;
  const void* wk;
  const void* wv;
  const void* wo;
};

// Longest page list of one attention tile (its page ids are staged in LDS);
// the host keeps max_positions within it.
constexpr int kMaxTilePages = 4096;

// Scratch of the projection GEMMs with at most 256 rows: one fp32 [256][N]
// partial tile per K split (up to kMaxSplits), overwritten by every launch.
constexpr int kMaxSplits = 8;
// GEMMs with at most this many rows split K over workgroups (branch scoring).
constexpr int kSplitRows = 256;
struct GemmWs {
  float* partial;
  size_t partial_elems;
  // rounds of at most kSplitRows rows too project without a K split, with the
  // large rounds' K order (round-invariant numerics)
  bool no_split = false;
};

// Timing of the next launcher call (profiling): its first kernel records
// `start` when it begins and its kernels record `stop` when they end (the last
// one leaves the final value), carried by the dispatches themselves
// (hipExtLaunchKernel), without separate event packets between kernels.
struct LaunchTiming {
  hipEvent_t start;
  hipEvent_t stop;
};
extern thread_local LaunchTiming g_launch_timing;

#define JEV_LAUNCH(KERNEL, GRID, BLOCK, SHMEM, STREAM, ...)                                                  \
  do {                                                                                                       \
    hipEvent_t e0_ = ::jev::g_launch_timing.start;                                                           \
    ::jev::g_launch_timing.start = nullptr;                                                                  \
    hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, e0_, ::jev::g_launch_timing.stop, 0u, __VA_ARGS__); \
  } while (0)

struct GemmTuning {
  int splits;  // split-K count of the skinny GEMM (0 = automatic)
  int bn;      // column tile of the large GEMM (0 = automatic)
  int large;   // large bf16 GEMM kernel: 0 = automatic (4), 1 = register staging, 2/3 = direct loads, 2/3
               // stages, 4 = direct loads by loader waves
};
extern GemmTuning g_gemm_tuning;

// h = RMSNorm(x) * g, stored
hipError_t launch_rmsnorm(const ModelDims& m, const void* x, const void* g, int32_t T, void* h,
                          hipStream_t s);
// q/k/v projections of h with RoPE at pos[t]; q -> qbuf [T][Hq][dh]; k, v -> the
// layer's pages at kvslot[t] = page*16 + slot.  rope: float2 [pos][dh/2].
// kv_only: k and v alone (q is not written), each element summed in the
// order of the full projection.
hipError_t launch_qkv(const ModelDims& m, const LayerW& w, int32_t layer, const void* h, int32_t T,
                      const int32_t* pos, const int32_t* kvslot, const float* rope, void* qbuf,
                      void* pool, const GemmWs& ws, hipStream_t s, bool kv_only = false);
// x = E[tok], then h = RMSNorm(x) * g (the first layer's norm), with the same
// arithmetic as launch_rmsnorm on the gathered rows.  With up_bytes > 0 (a
// multiple of 16) the kernel also copies up_bytes from up_src (device-visible
// pinned host memory) to up_dst, for the kernels launched after it.
hipError_t launch_embed_norm(const ModelDims& m, const void* embed, const int32_t* tok, int32_t T, const void* g,
                             void* x, void* h, hipStream_t s, const void* up_src = nullptr, void* up_dst = nullptr,
                             int64_t up_bytes = 0);
// Residual projection of a round of at most kSplitRows rows without its
// epilogue: the split-K partial tiles go to ws.partial (slice y at
// y * 256 * d), *splits receives their count.  launch_split_res_norm adds them.
hipError_t launch_oproj_split(const ModelDims& m, const LayerW& w, const void* o, int32_t T, const GemmWs& ws,
                              int32_t* splits, hipStream_t s);
// x += sum of the split partial tiles (slice order), then h = RMSNorm(x) * g:
// the residual epilogue of the projection fused with the next layer's norm,
// bitwise equal to the two separate kernels.
hipError_t launch_split_res_norm(const ModelDims& m, const float* partial, int32_t splits, int32_t T, void* x,
                                 const void* g, void* h, hipStream_t s);
// attention tiles (grid n_tiles x Hkv); groups = wave groups per workgroup (1
// or 2: two split every tile's steps in halves, for rounds with long tiles);
// with qrows, query row t of the tiles reads row qrows[t] of qbuf
hipError_t launch_attention(const ModelDims& m, int32_t layer, const AttnTile* tiles, int32_t n_tiles,
                            const int32_t* page_list, const int32_t* tok_pos, const void* qbuf,
                            const void* pool, void* o, float* part_o, float* part_lse, int32_t groups,
                            hipStream_t s, const int32_t* qrows = nullptr);
hipError_t launch_merge(const ModelDims& m, const MergeItem* items, int32_t n_items, const float* part_o,
                        const float* part_lse, void* o, hipStream_t s);
// x += o Wo^T (stored); with x_rows, row r of o updates x row x_rows[r]
hipError_t launch_oproj(const ModelDims& m, const LayerW& w, const void* o, int32_t T, void* x,
                        const GemmWs& ws, hipStream_t s, const int32_t* x_rows = nullptr);
// Debug: fills KV pages [first, first + count) of every layer with the bytes
// 0x7F (finite, near the dtype's maximum).
hipError_t launch_poison_pages(const ModelDims& m, void* pool, int32_t first, int32_t count, hipStream_t s);
hipError_t launch_readout(const ModelDims& m, const void* unembed, const void* final_norm, const void* x,
                          const ReadoutItem* items, int32_t n_items, const int32_t* labels, float* probs,
                          hipStream_t s);

}  // namespace jev
