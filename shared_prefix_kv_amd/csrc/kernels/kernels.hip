// gfx950 kernels of the shared-prefix scoring path (the projection GEMMs are
// in gemm.hip).
//
//  embed+norm x[t] = E[token t], h = RMSNorm(x) * g of the first layer
//  rmsnorm    h = x / sqrt(mean x^2 + eps) * g  (fp32 math, stored)
//  attention  paged attention of packed query rows (token x query head of one
//             KV head) against a page list; causal over a node's own pages,
//             unmasked over a shared prefix's pages (read once for all rows of
//             the sibling group); online softmax in fp32; writes the output or
//             a normalised partial state plus its log2-sum-exp
//  merge      log-sum-exp merge of the partial states of a token
//  readout    final norm of a candidate's last row, logits at its label ids
//             only, max-subtracted softmax over the labels
//
// The scoring rule (last position only, label ids only, stable softmax over
// the labels) is the jdon.com openjev-sglang article's "prefill-only" section;
// reading only the labels' logits is exact because the full-vocabulary
// log-normaliser cancels in the label softmax.
#include <float.h>

#include <algorithm>
#include <cmath>

#include "common.hpp"
#include "launch.hpp"

namespace jev {
namespace dev {

constexpr float kNegInf = -INFINITY;

// block-wide sum over 256 threads
__device__ __forceinline__ float block_sum256(float v, float* scratch) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  float r = scratch[0] + scratch[1] + scratch[2] + scratch[3];
  __syncthreads();
  return r;
}

template <typename T>
__device__ __forceinline__ void load16(const T* p, float* out);
template <>
__device__ __forceinline__ void load16<bf16s>(const bf16s* p, float* out) {
  u32x4 u = *reinterpret_cast<const u32x4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
// the elements of one 16-byte unit already loaded, as fp32
template <typename T>
__device__ __forceinline__ void unpack16(const u32x4& u, float* out);
template <>
__device__ __forceinline__ void unpack16<bf16s>(const u32x4& u, float* out) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
template <>
__device__ __forceinline__ void unpack16<float>(const u32x4& u, float* out) {
  out[0] = __uint_as_float(u.x);
  out[1] = __uint_as_float(u.y);
  out[2] = __uint_as_float(u.z);
  out[3] = __uint_as_float(u.w);
}
template <>
__device__ __forceinline__ void load16<float>(const float* p, float* out) {
  float4 u = *reinterpret_cast<const float4*>(p);
  out[0] = u.x;
  out[1] = u.y;
  out[2] = u.z;
  out[3] = u.w;
}

// ------------------------------------------------------------------ rmsnorm
// One block per row; d <= 256 * 8 * (16 / sizeof(T)) / 8 handled by the loop.
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const T* __restrict__ x, const T* __restrict__ g, int d,
                                                      float eps, T* __restrict__ h) {
  constexpr int CH = 16 / sizeof(T);
  __shared__ float scratch[4];
  const T* xr = x + (size_t)blockIdx.x * d;
  T* hr = h + (size_t)blockIdx.x * d;
  constexpr int MAXV = 4;  // chunks per thread held in registers (d <= 256*CH*4)
  float v[MAXV][CH], gg[MAXV][CH];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < MAXV; ++j) {
    const int i = (threadIdx.x + 256 * j) * CH;
    if (i < d) {
      load16<T>(xr + i, v[j]);
      load16<T>(g + i, gg[j]);  // loaded with x, used after the reduction
#pragma unroll
      for (int e = 0; e < CH; ++e) ss += v[j][e] * v[j][e];
    }
  }
  ss = block_sum256(ss, scratch);
  const float r = 1.0f / sqrtf(ss / float(d) + eps);
#pragma unroll
  for (int j = 0; j < MAXV; ++j) {
    const int i = (threadIdx.x + 256 * j) * CH;
    if (i < d) {
#pragma unroll
      for (int e = 0; e < CH; ++e) hr[i + e] = from_f32<T>(v[j][e] * r * gg[j][e]);
    }
  }
}

// Embedding gather fused with layer 0's norm: ROWS tokens per block, each
// row x = E[tok] and h = RMSNorm(x) * g with rmsnorm_kernel's element and
// reduction order (bitwise those of the two kernels).  The block's token ids
// are read by one load of its first wave: when they sit in pinned host memory
// (the first round of a call) every read is a bus transaction, so ROWS = 4
// takes a quarter of them; all rows' embedding loads are in flight together.
//
// With up_units > 0 the workgroups also copy up_units 16-byte units from
// up_src (the call's descriptors in pinned host memory, which tok then points
// into) to up_dst in device memory, for the kernels that follow: consecutive
// threads copy consecutive units (grid-stride), so a wave reads 1 KiB of
// contiguous host memory.
template <typename T, int ROWS>
__global__ __launch_bounds__(256) void embed_norm_kernel(const T* __restrict__ E, const int32_t* __restrict__ tok,
                                                         int n_tok, int d, const T* __restrict__ g, float eps,
                                                         T* __restrict__ x, T* __restrict__ h,
                                                         const u32x4* __restrict__ up_src, u32x4* __restrict__ up_dst,
                                                         int up_units) {
  constexpr int CH = 16 / sizeof(T);
  constexpr int MAXV = 4;
  __shared__ float scratch[4];
  __shared__ int32_t stok[ROWS];
  for (int u = (int)blockIdx.x * 256 + (int)threadIdx.x; u < up_units; u += (int)gridDim.x * 256)
    up_dst[u] = up_src[u];
  const int r0 = (int)blockIdx.x * ROWS;
  const int nr = min(ROWS, n_tok - r0);
  int tk[ROWS];
  if constexpr (ROWS > 1) {
    if (threadIdx.x < (unsigned)nr) stok[threadIdx.x] = tok[r0 + threadIdx.x];
    __syncthreads();
    // rows past the last token repeat it (loaded, never stored)
#pragma unroll
    for (int rr = 0; rr < ROWS; ++rr) tk[rr] = stok[min(rr, nr - 1)];
  } else {
    tk[0] = tok[r0];  // one uniform load, no barrier
  }
  // the embedding rows first, then the norm weights, with no branch between
  u32x4 raw[ROWS][MAXV];
  float gg[MAXV][CH];
#pragma unroll
  for (int j = 0; j < MAXV; ++j) {
    const int i = (threadIdx.x + 256 * j) * CH;
    if (i < d) {
#pragma unroll
      for (int rr = 0; rr < ROWS; ++rr) raw[rr][j] = *reinterpret_cast<const u32x4*>(E + (size_t)tk[rr] * d + i);
      load16<T>(g + i, gg[j]);
    }
  }
#pragma unroll
  for (int rr = 0; rr < ROWS; ++rr) {
    if (rr >= nr) break;
    T* xr = x + (size_t)(r0 + rr) * d;
    T* hr = h + (size_t)(r0 + rr) * d;
    float v[MAXV][CH];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < MAXV; ++j) {
      const int i = (threadIdx.x + 256 * j) * CH;
      if (i < d) {
        *reinterpret_cast<u32x4*>(xr + i) = raw[rr][j];
        unpack16<T>(raw[rr][j], v[j]);
#pragma unroll
        for (int e = 0; e < CH; ++e) ss += v[j][e] * v[j][e];
      }
    }
    ss = block_sum256(ss, scratch);
    const float r = 1.0f / sqrtf(ss / float(d) + eps);
#pragma unroll
    for (int j = 0; j < MAXV; ++j) {
      const int i = (threadIdx.x + 256 * j) * CH;
      if (i < d) {
#pragma unroll
        for (int e = 0; e < CH; ++e) hr[i + e] = from_f32<T>(v[j][e] * r * gg[j][e]);
      }
    }
  }
}

// Residual epilogue of a split-K projection fused with the next layer's norm:
// one block per row.  x = x + (p_0 + p_1 + ... + p_{S-1}) summed in slice
// order and rounded to T (as split_epilogue's residual epilogue does), then h
// = RMSNorm(x) * g with the rows's elements, squares and block sum in
// rmsnorm_kernel's order: both outputs are bitwise those of the two kernels.
// MAXV = 16-byte chunks per thread that the row needs (d <= 256 * CH * MAXV).
template <typename T, int MAXV>
__global__ __launch_bounds__(256) void split_res_norm_kernel(const float* __restrict__ part, int splits, int d,
                                                             T* __restrict__ x, const T* __restrict__ g, float eps,
                                                             T* __restrict__ h) {
  constexpr int CH = 16 / sizeof(T);
  __shared__ float scratch[4];
  const size_t slice = (size_t)256 * d;
  T* xr = x + (size_t)blockIdx.x * d;
  const float* pr = part + (size_t)blockIdx.x * d;
  T* hr = h + (size_t)blockIdx.x * d;
  float v[MAXV][CH], gg[MAXV][CH];
  float ss = 0.f;
  // every slice of every chunk is loaded before the first sum (the slice
  // count is at most kMaxSplits; slices past it are not read)
  u32x4 raw_x[MAXV];
  float4 sp[MAXV][kMaxSplits][CH / 4];
#pragma unroll
  for (int j = 0; j < MAXV; ++j) {
    const int i = (threadIdx.x + 256 * j) * CH;
    if (i < d) {
      raw_x[j] = *reinterpret_cast<const u32x4*>(xr + i);
      load16<T>(g + i, gg[j]);
#pragma unroll
      for (int y = 0; y < kMaxSplits; ++y)
        if (y < splits)
#pragma unroll
          for (int q = 0; q < CH / 4; ++q) sp[j][y][q] = reinterpret_cast<const float4*>(pr + y * slice + i)[q];
    }
  }
#pragma unroll
  for (int j = 0; j < MAXV; ++j) {
    const int i = (threadIdx.x + 256 * j) * CH;
    if (i < d) {
      float xs[CH], acc[CH];
      unpack16<T>(raw_x[j], xs);
#pragma unroll
      for (int q = 0; q < CH / 4; ++q) {
        acc[4 * q] = sp[j][0][q].x;
        acc[4 * q + 1] = sp[j][0][q].y;
        acc[4 * q + 2] = sp[j][0][q].z;
        acc[4 * q + 3] = sp[j][0][q].w;
      }
      // slice order, as the separate residual epilogue sums them
#pragma unroll
      for (int y = 1; y < kMaxSplits; ++y)
        if (y < splits)
#pragma unroll
          for (int q = 0; q < CH / 4; ++q) {
            acc[4 * q] += sp[j][y][q].x;
            acc[4 * q + 1] += sp[j][y][q].y;
            acc[4 * q + 2] += sp[j][y][q].z;
            acc[4 * q + 3] += sp[j][y][q].w;
          }
#pragma unroll
      for (int e = 0; e < CH; ++e) {
        const T r = from_f32<T>(xs[e] + acc[e]);
        xr[i + e] = r;
        v[j][e] = to_f32(r);
        ss += v[j][e] * v[j][e];
      }
    }
  }
  ss = block_sum256(ss, scratch);
  const float r = 1.0f / sqrtf(ss / float(d) + eps);
#pragma unroll
  for (int j = 0; j < MAXV; ++j) {
    const int i = (threadIdx.x + 256 * j) * CH;
    if (i < d) {
#pragma unroll
      for (int e = 0; e < CH; ++e) hr[i + e] = from_f32<T>(v[j][e] * r * gg[j][e]);
    }
  }
}

// ------------------------------------------------------------------ attention
// A wave group = 4 waves = 128 query rows (tokens_per_tile x G heads of one KV
// head); wave w owns rows [32w, 32w+32).  Per step two pages (32 keys) of K and
// V go through LDS.  A workgroup has one group, or two that take the two
// halves of the tile's steps and merge their softmax states at the end (the
// chain of a long causal tile halves; the CU holds the same eight waves).  S^T = K Q^T (keys as MFMA rows, query rows as columns) keeps a
// query row's softmax statistics in one lane column, so that O^T = V^T P^T
// rescales per lane with no cross-lane traffic besides the two half-waves.
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag frag_zero();
template <>
__device__ __forceinline__ bf16x8 frag_zero<bf16s>() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.0f;
  return z;
}
template <>
__device__ __forceinline__ float frag_zero<float>() { return 0.f; }

// Key order of the bf16 score product.  The score MFMA's output register r
// of lane half hh holds row 8 (r / 4) + 4 hh + r % 4 of its A operand; lane c
// loads K row key_of_row(c) there, so that register r holds key
// 16 (r / 8) + 8 hh + r % 8: the 8 probabilities a lane feeds to one P.V MFMA
// (keys 16 tt + 8 hh .. + 7) are then 8 consecutive keys of one page, 16
// contiguous bytes of its V^T row.
__device__ __forceinline__ int key_of_row(int c) {
  return 16 * (c >> 4) + 8 * ((c >> 2) & 1) + 4 * ((c >> 3) & 1) + (c & 3);
}
// LDS V^T tile [DH][32 keys] for bf16: four 16-byte units per 64-byte row
// (keys 8u .. 8u+7 in unit u), XOR-swizzled by (d >> 2) & 3, which puts the
// 16 rows of a 16-lane read in 16 different bank groups.
__device__ __forceinline__ int vq_unit(int d, int unit) { return d * 4 + (unit ^ ((d >> 2) & 3)); }
// f32 (8 quads of 4 keys per 32-key row): plain 16-byte units swizzled by d.
__device__ __forceinline__ int v_off(int d, int key) {
  const int u = (key >> 2) ^ (d & 7);
  return d * 32 + u * 4 + (key & 3);
}

// Lazy rescaling: a row's running maximum m is only moved when a new score
// exceeds it by more than 2^RESCALE_SLACK (log2 units); until then
// probabilities exp2(s - m) may exceed 1 (by at most 2^8) and the output and
// normaliser keep accumulating on the same scale.  The result is the same
// softmax; only the rounding order changes.
constexpr float RESCALE_SLACK = 8.0f;


template <typename T, int DH, int GROUPS>
__global__ __launch_bounds__(256 * GROUPS) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_kernel(const AttnTile* __restrict__ tiles,
                                                   const int32_t* __restrict__ plist,
                                                   const int32_t* __restrict__ tok_pos, const T* __restrict__ q,
                                                   const T* __restrict__ pool, T* __restrict__ o,
                                                   float* __restrict__ part_o, float* __restrict__ part_lse,
                                                   int hq, int hkv, size_t layer_base, float scale_log2,
                                                   const int32_t* __restrict__ qrows) {
  using MF = Mfma<T>;
  using frag = typename MF::frag;
  constexpr int KL = MF::KL, KSTEP = MF::KSTEP;
  constexpr int NKS = DH / KSTEP;
  constexpr int CH = 16 / sizeof(T);
  constexpr int KCH = DH / CH;            // 16-byte chunks per K row
  constexpr int PAGE_ELEMS = 16 * DH;
  constexpr int PAGE_CHUNKS = PAGE_ELEMS / CH;
  constexpr int VCPR = 16 / CH;           // 16-byte chunks per V^T row of a page
  constexpr int NDB = DH / 32;
  static_assert(PAGE_CHUNKS == 256, "two pages per step = 512 chunks = 2 per thread");
  static_assert(GROUPS == 1 || GROUPS == 2, "one or two wave groups");
  // Per wave group: K and V double buffers.  Then the tile's page list, page
  // id * 32 + valid keys (read once per workgroup).  With two groups the
  // buffers are reused after the loop for group 1's state (NDB * 16 + 2
  // floats per thread).
  constexpr int KV_BYTES = 2 * 32 * DH * (int)sizeof(T);
  constexpr int XCH_BYTES = GROUPS > 1 ? (DH / 32 * 16 + 2) * 256 * 4 : 0;
  constexpr int MAIN_BYTES = GROUPS * 2 * KV_BYTES + kMaxTilePages * 4;
  __shared__ __attribute__((aligned(16))) char lds[MAIN_BYTES > XCH_BYTES ? MAIN_BYTES : XCH_BYTES];
  int32_t* const sP = reinterpret_cast<int32_t*>(lds + GROUPS * 2 * KV_BYTES);
  // one workgroup per (tile, KV head); the KV head is the fast index, so that
  // neighbouring workgroups read the same pages (whose KV heads are adjacent)
  const int kvh = blockIdx.x % hkv;
  const AttnTile tile = tiles[blockIdx.x / hkv];
  for (int i = threadIdx.x; i < tile.n_pages; i += blockDim.x)
    sP[i] = plist[2 * (tile.page_off + i)] * 32 + plist[2 * (tile.page_off + i) + 1];
  const int G = hq / hkv;
  // wave group: with two, group g takes the g-th half of the tile's steps
  const int grp = GROUPS > 1 ? __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 8) : 0;
  T (*const sK)[32 * DH] = reinterpret_cast<T (*)[32 * DH]>(lds + grp * 2 * KV_BYTES);
  T (*const sV)[DH * 32] = reinterpret_cast<T (*)[DH * 32]>(lds + grp * 2 * KV_BYTES + KV_BYTES);
  const int tid = threadIdx.x & 255, lane = tid & 63, wave = tid >> 6, c = lane & 31, hh = lane >> 5;
  // Barrier of the step pipeline: the workgroup barrier (with two groups every
  // wave of both groups meets it; their halves are offset, see the loop).
  auto step_sync = [&]() __attribute__((always_inline)) { __syncthreads(); };
  const int row = wave * 32 + c;
  const int ti = row / G, hg = row % G;
  const bool row_ok = ti < tile.n_tok;
  const int t = tile.t0 + (row_ok ? ti : 0);
  const int qhead = kvh * G + hg;
  const int qpos = tok_pos[t];
  // smallest query position of the wave: keys up to it are visible to every row
  int qmin = qpos;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) qmin = min(qmin, __shfl_xor(qmin, off, 64));

  frag qf[NKS];
  {
    // query row t of the launch is row qrows[t] of q (qrows null: row t)
    const T* qrow = q + ((size_t)(qrows ? qrows[t] : t) * hq + qhead) * DH;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = row_ok ? MF::load(qrow + ks * KSTEP + KL * hh) : frag_zero<T>();
  }

  const T* kvbase = pool + layer_base + (size_t)kvh * 2 * PAGE_ELEMS;
  // steps of two pages: this group's first global step s0 and the loop count
  // nst (the same for both groups, so that their barriers pair up; a group's
  // steps past the tile's end have every key masked)
  const int nst_all = (tile.n_pages + 1) >> 1;
  const int nst_own = (nst_all + GROUPS - 1) / GROUPS;
  const int s0 = grp * nst_own;
  // pages of this group's steps (the rest of its steps are fully masked)
  const int page_end = min(tile.n_pages, 2 * (s0 + nst_own));
  // two groups: an even count, so that the ping-pong loop body (two steps)
  // has no conditional half; the extra step, if any, is fully masked
  const int nst = GROUPS > 1 ? (nst_own + 1) & ~1 : nst_own;

  // loop-invariant LDS offsets
  int koff[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const int e = ks * KSTEP + KL * hh;
    const int kr = KL == 8 ? key_of_row(c) : c;  // the K row this lane feeds
    koff[ks] = kr * DH + (((e / CH) ^ (kr & (KCH - 1))) * CH) + e % CH;
  }
  const int st_krow = tid / KCH, st_kch = tid % KCH;
  const int st_koff = st_krow * DH + ((st_kch ^ (st_krow & (KCH - 1))) * CH);  // + 16*DH*i for page i
  const int st_d = tid / VCPR, st_half = tid % VCPR;

  // K and V of a step (two pages) are staged separately: at step st the loop
  // computes S for step st+1 from LDS K buffer (st+1)&1 while it applies the
  // softmax of step st and PV with V buffer st&1; meanwhile K of step st+2 goes
  // into K buffer st&1 (last read for S of step st, one barrier ago) and V of
  // step st+1 into V buffer (st+1)&1 (last read at step st-1).
  // Global loads are unconditional (page index clamped to the tile's last
  // page; keys of pages past the end are masked by their zero valid count),
  // so the number of loads in flight is static and each LDS store waits only
  // for the loads of its own step, issued one step earlier. The staging
  // registers alternate between two sets from step to step (the loop is
  // unrolled by two), so no register copy waits for loads still in flight.
  u32x4 rkA[2], rvA[2], rkB[2], rvB[2];
  // A window of 64 page-list entries, one per lane (entries pw_base + lane),
  // read by readlane: a step needs entries 2st .. 2st+7 (global step st), so
  // the window is moved every 16 steps and page ids cost no memory access in
  // between.  Page indexes are clamped to the tile's last page, and so is the
  // window's base.
  int pw = 0, pw_base = 0;
  auto page_entry = [&](int lp) -> int {
    return __builtin_amdgcn_readlane(pw, min(lp, tile.n_pages - 1) - pw_base);
  };
  // page byte offsets as one unsigned 32 x 32 -> 64-bit product (a page id is
  // below 2^26 and a page's K+V for all KV heads is hkv * 2 * PAGE_ELEMS
  // elements, far below 4 GiB)
  const char* kvbytes = reinterpret_cast<const char*>(kvbase);
  const uint32_t page_bytes = (uint32_t)hkv * (uint32_t)(2 * PAGE_ELEMS * sizeof(T));
  auto page_ptr = [&](int lp) -> const T* {
    const uint32_t pg = (uint32_t)page_entry(lp) >> 5;
    return reinterpret_cast<const T*>(kvbytes + (uint64_t)pg * page_bytes);
  };
  // K or V of this group's step st (global step s0 + st)
  auto gload_k = [&](int st, u32x4* dst) {
#pragma unroll
    for (int i = 0; i < 2; ++i) dst[i] = reinterpret_cast<const u32x4*>(page_ptr(2 * (s0 + st) + i))[tid];
  };
  auto gload_v = [&](int st, u32x4* dst) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      dst[i] = reinterpret_cast<const u32x4*>(page_ptr(2 * (s0 + st) + i) + PAGE_ELEMS)[tid];
  };
  auto sstore_k = [&](int buf, const u32x4* rk) {
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<u32x4*>(&sK[buf][st_koff + 16 * DH * i]) = rk[i];
  };
  auto sstore_v = [&](int buf, const u32x4* rv) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (CH == 8) {
        // page i holds keys 16i..16i+15; this chunk is keys 16i + 8 st_half ..
        // + 7 of V^T row st_d: unit 2i + st_half
        reinterpret_cast<u32x4*>(&sV[buf][0])[vq_unit(st_d, 2 * i + st_half)] = rv[i];
      } else {
        *reinterpret_cast<u32x4*>(&sV[buf][v_off(st_d, 16 * i + st_half * CH)]) = rv[i];
      }
    }
  };
  auto qk = [&](int buf) {
    f32x16 S;
#pragma unroll
    for (int r = 0; r < 16; ++r) S[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) S = MF::mma(MF::load(&sK[buf][koff[ks]]), qf[ks], S);
    return S;
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;
  float mrun = kNegInf, lrun = 0.f;

  __syncthreads();  // page list
  pw_base = min(2 * s0, tile.n_pages - 1);
  pw = sP[min(pw_base + lane, tile.n_pages - 1)];
  if (nst > 0) {
    // K and V of step 0 and K of step 1 in flight together (one load latency)
    gload_k(0, rkA);
    gload_v(0, rvA);
    gload_k(1, rkB);
    sstore_k(0, rkA);
    sstore_v(0, rvA);
    sstore_k(1, rkB);
    // staged for the first step's stores: K of step 2, V of step 1
    gload_k(2, rkA);
    gload_v(1, rvA);
  }
  step_sync();
  f32x16 SA, SB;
  if (nst > 0) SA = qk(0);
  // step 0 stores K of step 2 into K buffer 0: every wave has to be done
  // reading K of step 0 from it first (once per tile)
  if (GROUPS > 1 || nst > 2) step_sync();

  // ---- pieces of a step (st = this group's step) ----
  // page-list window: moved every 16 steps
  auto window = [&](const int st) __attribute__((always_inline)) {
    if (st > 0 && (st & 15) == 0) {
      pw_base = min(2 * (s0 + st), tile.n_pages - 1);
      pw = sP[min(pw_base + lane, tile.n_pages - 1)];
    }
  };
  // First half of the softmax of step st's scores S (masked in place): the
  // mask where needed (partial pages, keys past the wave's first query), the
  // running maximum with its lazy rescale of the output and the sum; returns
  // the offset that the exponentials subtract.
  auto softmax_a = [&](const int st, f32x16& S) __attribute__((always_inline)) -> float {
    const int lp0 = 2 * (s0 + st);
    const int v0 = (lp0 < page_end) ? (page_entry(lp0) & 31) : 0;
    const int v1 = (lp0 + 1 < page_end) ? (page_entry(lp0 + 1) & 31) : 0;
    const bool mask = (v0 < 16) || (v1 < 16) || (tile.causal && tile.kv_pos0 + 16 * lp0 + 31 > qmin);
    if (mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = KL == 8 ? 16 * (r >> 3) + 8 * hh + (r & 7) : 8 * (r >> 2) + 4 * hh + (r & 3);
        const int pi = key >> 4, slot = key & 15;
        const bool ok = slot < (pi ? v1 : v0) && (!tile.causal || tile.kv_pos0 + 16 * (lp0 + pi) + slot <= qpos);
        S[r] = ok ? S[r] : kNegInf;
      }
    }
    float mloc = S[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mloc = fmaxf(mloc, S[r]);
    mloc = xor32_max(mloc) * scale_log2;
    if (__any(mloc > mrun + RESCALE_SLACK)) {
      // each row moves its own maximum only when it exceeds the slack itself
      // (alpha = 1 exactly otherwise), so a row's rounding never depends on
      // the other rows of its wave
      const float mnew = (mloc > mrun + RESCALE_SLACK) ? mloc : mrun;
      const float alpha = (mnew == kNegInf) ? 1.f : exp2f(mrun - mnew);
      lrun *= alpha;
#pragma unroll
      for (int b = 0; b < NDB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
      mrun = mnew;
    }
    return (mrun == kNegInf) ? 0.f : -mrun;
  };
  // Second half: the probabilities, their sum, and (bf16) P = P_hi + P_lo,
  // both bf16 (P_hi the upper 16 bits of the fp32 value, P_lo its exact
  // remainder rounded to nearest), so that the PV product sees P to ~16
  // significant bits, not the 8 of one bf16 rounding (that rounding alone
  // moved label probabilities several times further than any change of
  // summation order does).
  auto softmax_b = [&](const f32x16& S, const float nm, frag* pb, frag* pl) __attribute__((always_inline)) {
    float p[16];
    float lsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = __builtin_amdgcn_exp2f(fmaf(S[r], scale_log2, nm));
      lsum += p[r];
    }
    lsum = xor32_sum(lsum);
    lrun += lsum;
#pragma unroll
    for (int tt = 0; tt < 16 / KL; ++tt) {
      if constexpr (KL == 8) {
#pragma unroll
        for (int sidx = 0; sidx < 8; ++sidx) {
          const uint32_t u = __float_as_uint(p[8 * tt + sidx]);
          pb[tt][sidx] = __builtin_bit_cast(__bf16, uint16_t(u >> 16));
          pl[tt][sidx] = (__bf16)(p[8 * tt + sidx] - __uint_as_float(u & 0xFFFF0000u));
        }
      } else {
        pb[tt] = p[tt];
      }
    }
  };
  // O^T += V^T P^T from V buffer buf; MFMA tt covers keys 16tt + 8hh + i,
  // i < 8 (bf16), or key 8 (tt / 4) + 4 hh + tt % 4 (f32)
  auto pv = [&](const int buf, const frag* pb, const frag* pl) __attribute__((always_inline)) {
#pragma unroll
    for (int tt = 0; tt < 16 / KL; ++tt) {
      frag va[NDB];
#pragma unroll
      for (int b = 0; b < NDB; ++b) {
        const int d = 32 * b + c;
        if constexpr (KL == 8) {
          // keys 16tt + 8hh .. 16tt + 8hh + 7 (page tt): unit 2tt + hh
          va[b] = __builtin_bit_cast(bf16x8, reinterpret_cast<const u32x4*>(&sV[buf][0])[vq_unit(d, 2 * tt + hh)]);
        } else {
          const int key = 8 * (tt >> 2) + 4 * hh + (tt & 3);
          va[b] = MF::load(&sV[buf][v_off(d, key)]);
        }
        oacc[b] = MF::mma(va[b], pb[tt], oacc[b]);
      }
      if constexpr (KL == 8) {
#pragma unroll
        for (int b = 0; b < NDB; ++b) oacc[b] = MF::mma(va[b], pl[tt], oacc[b]);
      }
    }
  };

  if constexpr (GROUPS == 1) {
    // One step: stores K of step st+2 and V of step st+1 from (kst, vst), loads
    // K of step st+3 and V of step st+2 into (kld, vld), turns S_in (scores of
    // step st) into probabilities and leaves the scores of step st+1 in S_out.
    auto step = [&](const int st, const u32x4* kst, const u32x4* vst, u32x4* kld, u32x4* vld, f32x16& S_in,
                    f32x16& S_out) __attribute__((always_inline)) {
      const int buf = st & 1;
      window(st);
      // loads for the next step's stores
      gload_k(st + 3, kld);
      gload_v(st + 2, vld);
      const float nm = softmax_a(st, S_in);
      // Branch-free from here: the S MFMAs of the next step (a dependent chain)
      // are interleaved with this step's exponentials, so that one wave per
      // SIMD keeps the MFMA and VALU pipes busy together. On the last step the
      // product reads stale LDS and is never used.
      S_out = qk(buf ^ 1);
      frag pb[16 / KL], pl[16 / KL];
      softmax_b(S_in, nm, pb, pl);
      pv(buf, pb, pl);
      if constexpr (KL == 8) {
        // Order of the branch-free block: 2 K-fragment reads ahead; per S MFMA
        // ~10 VALU (exponentials, row sums, the P_hi / P_lo split) and the next
        // K read, plus, over the last four, the V reads of the first PV block;
        // then the PV MFMAs (hi then lo per 16 keys) with the V reads of the
        // second block spread over the first half.
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int i = 0; i < NKS; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);
          if (i + 2 < NKS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          if (i >= NKS - NDB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < 4 * NDB; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (i < 2 * NDB && (i & 1) == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        }
      }
      if (st + 2 < nst) sstore_k(buf, kst);
      if (st + 1 < nst) sstore_v(buf ^ 1, vst);
      step_sync();
    };
    for (int st = 0; st < nst; st += 2) {
      step(st, rkA, rvA, rkB, rvB, SA, SB);
      if (st + 1 < nst) step(st + 1, rkB, rvB, rkA, rvA, SB, SA);
    }
  } else {
    // Two groups in ping-pong: a step is split into a softmax half (VALU: the
    // mask, maximum, exponentials, sum and P split of step st, then the LDS
    // stores of K of step st+2 and V of step st+1) and a matrix half (MFMA:
    // the scores of step st+1 and O += V P of step st, with the global loads
    // of K of step st+3 and V of step st+2).  Group 1 runs one half behind
    // group 0, and every half ends at the workgroup barrier, so that on each
    // SIMD one wave issues MFMAs while the other works the VALU.  Both groups
    // run the same number of halves and barriers.
    frag pb[16 / KL], pl[16 / KL];
    // The first fragments of the next MFMA half (K of step st+1 and the first
    // V block of step st, stored two halves earlier; the softmax half writes
    // the other buffers) are read at the end of the softmax half, so the MFMA
    // half starts without an LDS latency: 2.5% on the causal prefill, bitwise
    // unchanged.
    constexpr int PF_K = 2;
    frag kf_pf[PF_K], v0_pf[NDB];
    auto half_softmax = [&](const int st, f32x16& S_in, const u32x4* kst, const u32x4* vst)
                            __attribute__((always_inline)) {
      const int buf = st & 1;
      window(st);
      const float nm = softmax_a(st, S_in);
      softmax_b(S_in, nm, pb, pl);
      if (st + 2 < nst) sstore_k(buf, kst);
      if (st + 1 < nst) sstore_v(buf ^ 1, vst);
      if constexpr (KL == 8) {
#pragma unroll
        for (int ks = 0; ks < PF_K; ++ks) kf_pf[ks] = MF::load(&sK[buf ^ 1][koff[ks]]);
#pragma unroll
        for (int b = 0; b < NDB; ++b)
          v0_pf[b] = __builtin_bit_cast(bf16x8, reinterpret_cast<const u32x4*>(&sV[buf][0])[vq_unit(32 * b + c, hh)]);
      }
    };
    auto half_mfma = [&](const int st, f32x16& S_out, u32x4* kld, u32x4* vld) __attribute__((always_inline)) {
      const int buf = st & 1;
      gload_k(st + 3, kld);
      gload_v(st + 2, vld);
      // keep the loads here, two halves ahead of the stores that use them
      // (the compiler would otherwise sink them next to the stores)
      asm volatile("" ::: "memory");
      // on the last step the score product reads stale LDS and is never used
      if constexpr (KL == 8) {
        // every fragment read first; then the dependent score chain of step
        // st+1 alternates with the independent O += V P_hi / V P_lo MFMAs of
        // step st (per output block the same order as pv(): hi then lo for
        // keys 0-15, then for keys 16-31)
        frag kf[NKS], v0[NDB], v1[NDB];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) kf[ks] = ks < PF_K ? kf_pf[ks] : MF::load(&sK[buf ^ 1][koff[ks]]);
#pragma unroll
        for (int b = 0; b < NDB; ++b) {
          v0[b] = v0_pf[b];
          v1[b] = __builtin_bit_cast(bf16x8, reinterpret_cast<const u32x4*>(&sV[buf][0])[vq_unit(32 * b + c, 2 + hh)]);
        }
        // every read issued before the first MFMA, and the MFMAs in the
        // source order below (the scheduler would otherwise move the score
        // chain last and the second V reads next to their MFMAs)
        __builtin_amdgcn_sched_barrier(0);
        f32x16 S;
#pragma unroll
        for (int r = 0; r < 16; ++r) S[r] = 0.f;
#pragma unroll
        for (int i = 0; i < 2 * NDB; ++i) {
          oacc[i % NDB] = MF::mma(v0[i % NDB], i < NDB ? pb[0] : pl[0], oacc[i % NDB]);
          if (i < NKS) S = MF::mma(kf[i], qf[i], S);
          // an opaque use of the running score keeps each score MFMA next to
          // its output-block MFMA (without it the chain is sunk to its end)
          asm volatile("" : "+v"(S));
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 2 * NDB; i < NKS; ++i) S = MF::mma(kf[i], qf[i], S);
#pragma unroll
        for (int i = 0; i < 2 * NDB; ++i)
          oacc[i % NDB] = MF::mma(v1[i % NDB], i < NDB ? pb[1] : pl[1], oacc[i % NDB]);
        S_out = S;
      } else {
        S_out = qk(buf ^ 1);
        pv(buf, pb, pl);
      }
    };
    // the halves are kept apart for the scheduler as well: nothing moves
    // across a half's barrier (MFMAs would otherwise drift into the softmax
    // half, which the partner group needs for its own MFMAs)
    auto half_sync = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    };
    if (grp == 1) half_sync();
    for (int st = 0; st < nst; st += 2) {
      half_softmax(st, SA, rkA, rvA);
      half_sync();
      half_mfma(st, SB, rkB, rvB);
      half_sync();
      half_softmax(st + 1, SB, rkB, rvB);
      half_sync();
      half_mfma(st + 1, SA, rkA, rvA);
      half_sync();
    }
    if (grp == 0) half_sync();
  }

  if constexpr (GROUPS > 1) {
    // group 1 leaves its running maximum, sum and unnormalised output in LDS
    // (element k of thread tid at k * 256 + tid); group 0 rescales both to
    // the larger maximum and adds them (the softmax over the union of the
    // two key ranges)
    float* const xo = reinterpret_cast<float*>(lds);
    constexpr int NX = NDB * 16;
    __syncthreads();  // both groups done with their buffers (the groups sync separately in the loop)
    if (grp == 1) {
#pragma unroll
      for (int b = 0; b < NDB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[(b * 16 + r) * 256 + tid] = oacc[b][r];
      xo[NX * 256 + tid] = mrun;
      xo[(NX + 1) * 256 + tid] = lrun;
    }
    __syncthreads();
    if (grp == 1) return;
    const float m1 = xo[NX * 256 + tid], l1 = xo[(NX + 1) * 256 + tid];
    const float mn = fmaxf(mrun, m1);
    const float a0 = (mrun == kNegInf) ? 0.f : exp2f(mrun - mn);
    const float a1 = (m1 == kNegInf) ? 0.f : exp2f(m1 - mn);
    lrun = lrun * a0 + l1 * a1;
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[b][r] = oacc[b][r] * a0 + xo[(b * 16 + r) * 256 + tid] * a1;
    mrun = mn;
  }

  if (!row_ok) return;
  const float inv = lrun > 0.f ? 1.0f / lrun : 0.f;
  if (tile.out_mode == 0) {
    T* orow = o + ((size_t)t * hq + qhead) * DH;
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) orow[32 * b + 8 * (r >> 2) + 4 * hh + (r & 3)] = from_f32<T>(oacc[b][r] * inv);
  } else {
    const size_t prow = ((size_t)tile.part_slot * hkv + kvh) * 128 + row;
    float* orow = part_o + prow * DH;
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float4 v = make_float4(oacc[b][4 * j] * inv, oacc[b][4 * j + 1] * inv, oacc[b][4 * j + 2] * inv,
                               oacc[b][4 * j + 3] * inv);
        *reinterpret_cast<float4*>(orow + 32 * b + 8 * j + 4 * hh) = v;
      }
    if (hh == 0) part_lse[prow] = lrun > 0.f ? mrun + log2f(lrun) : kNegInf;
  }
}

// ------------------------------------------------------------------ merge
// At most kMaxOwnParts own parts + kMaxAncParts prefix chunks per token (the
// host never plans more).
constexpr int MAX_PARTS = kMaxOwnParts + kMaxAncParts;

template <typename T, int DH>
__global__ __launch_bounds__(256) void merge_kernel(const MergeItem* __restrict__ items,
                                                    const float* __restrict__ part_o,
                                                    const float* __restrict__ part_lse, T* __restrict__ o, int hq,
                                                    int hkv) {
  // one workgroup per (token, KV head): the G query heads of the group
  const MergeItem it = items[blockIdx.x / hkv];
  const int kvh = blockIdx.x % hkv;
  const int G = hq / hkv;
  const int np = it.n_own + it.n_anc;
  for (int e = threadIdx.x; e < G * DH / 4; e += blockDim.x) {
    const int hg = e / (DH / 4), d4 = (e % (DH / 4)) * 4;
    const int head = kvh * G + hg;
    size_t rows[MAX_PARTS];
    float L[MAX_PARTS];
#pragma unroll
    for (int p = 0; p < MAX_PARTS; ++p) {
      rows[p] = p < it.n_own ? ((size_t)(it.own_slot0 + p) * hkv + kvh) * 128 + it.own_ti * G + hg
                             : ((size_t)(it.anc_slot0 + p - it.n_own) * hkv + kvh) * 128 + it.anc_ti * G + hg;
      L[p] = p < np ? part_lse[rows[p]] : kNegInf;
    }
    float4 v[MAX_PARTS];
#pragma unroll
    for (int p = 0; p < MAX_PARTS; ++p)
      v[p] = p < np ? *reinterpret_cast<const float4*>(part_o + rows[p] * DH + d4) : make_float4(0.f, 0.f, 0.f, 0.f);
    float M = L[0];
#pragma unroll
    for (int p = 1; p < MAX_PARTS; ++p) M = fmaxf(M, L[p]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float ws = 0.f;
#pragma unroll
    for (int p = 0; p < MAX_PARTS; ++p) {
      const float w = p < np ? exp2f(L[p] - M) : 0.f;
      acc.x += w * v[p].x;
      acc.y += w * v[p].y;
      acc.z += w * v[p].z;
      acc.w += w * v[p].w;
      ws += w;
    }
    const float inv = 1.0f / ws;
    T* orow = o + ((size_t)it.t * hq + head) * DH + d4;
    orow[0] = from_f32<T>(acc.x * inv);
    orow[1] = from_f32<T>(acc.y * inv);
    orow[2] = from_f32<T>(acc.z * inv);
    orow[3] = from_f32<T>(acc.w * inv);
  }
}

// ------------------------------------------------------------------ readout
template <typename T>
__global__ __launch_bounds__(256) void readout_kernel(const T* __restrict__ U, const T* __restrict__ g,
                                                      const T* __restrict__ x, const ReadoutItem* __restrict__ items,
                                                      const int32_t* __restrict__ labels, float* __restrict__ probs,
                                                      int d, float eps) {
  constexpr int CH = 16 / sizeof(T);
  extern __shared__ float sh[];  // d floats of normed hidden, then 64 logits
  __shared__ float scratch[4];
  float* hn = sh;
  float* logit = sh + d;
  const ReadoutItem it = items[blockIdx.x];
  const T* xr = x + (size_t)it.row * d;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // loads issued together (one memory latency, not one per step): the row,
  // the norm weights and the first unembedding row of each wave (label k =
  // wave), held in registers while the norm is computed
  constexpr int MAXU = 16;  // 16-byte units per lane of a row: d <= 1024 * CH, the norm kernels' limit
  u32x4 u0[MAXU];
  if (wave < it.k) {
    const T* ur = U + (size_t)labels[it.label_off + wave] * d;
#pragma unroll
    for (int j = 0; j < MAXU; ++j) {
      const int i = (lane + 64 * j) * CH;
      if (i < d) u0[j] = *reinterpret_cast<const u32x4*>(ur + i);
    }
  }
  float ss = 0.f;
  for (int i = tid * CH; i < d; i += 256 * CH) {
    float v[CH];
    load16<T>(xr + i, v);
#pragma unroll
    for (int e = 0; e < CH; ++e) {
      ss += v[e] * v[e];
      hn[i + e] = v[e];
    }
  }
  ss = block_sum256(ss, scratch);
  const float r = 1.0f / sqrtf(ss / float(d) + eps);
  for (int i = tid * CH; i < d; i += 256 * CH) {
    float gg[CH];
    load16<T>(g + i, gg);
#pragma unroll
    for (int e = 0; e < CH; ++e) hn[i + e] = to_f32(from_f32<T>(hn[i + e] * r * gg[e]));
  }
  __syncthreads();
  for (int k = wave; k < it.k; k += 4) {
    const T* ur = U + (size_t)labels[it.label_off + k] * d;
    float z = 0.f;
#pragma unroll
    for (int j = 0; j < MAXU; ++j) {
      const int i = (lane + 64 * j) * CH;
      if (i < d) {
        float u[CH];
        if (k == wave)
          unpack16<T>(u0[j], u);
        else
          load16<T>(ur + i, u);
#pragma unroll
        for (int e = 0; e < CH; ++e) z += hn[i + e] * u[e];
      }
    }
    z = wave_sum(z);
    if (lane == 0) logit[k] = z;
  }
  __syncthreads();
  if (wave == 0) {
    const float z = lane < it.k ? logit[lane] : kNegInf;
    const float mx = wave_max(z);
    const float e = lane < it.k ? expf(z - mx) : 0.f;
    const float s = wave_sum(e);
    if (lane < it.k) probs[it.out_off + lane] = e / s;
  }
}

// ------------------------------------------------------------------ page poison
// Debug fill of a run of `count` KV pages starting at page `first`, in every
// layer: each 16-byte unit of their K and V blocks gets the bytes 0x7F.
__global__ __launch_bounds__(256) void poison_pages_kernel(u32x4* __restrict__ pool, size_t layer_units,
                                                           size_t page_units, int32_t first, int32_t count,
                                                           int32_t n_layers) {
  const size_t run = page_units * (size_t)count;
  const size_t total = run * (size_t)n_layers;
  const u32x4 v = {0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu};
  for (size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += (size_t)gridDim.x * blockDim.x) {
    const size_t layer = u / run, within = u % run;
    pool[layer * layer_units + (size_t)first * page_units + within] = v;
  }
}

}  // namespace dev

thread_local LaunchTiming g_launch_timing{nullptr, nullptr};

// ------------------------------------------------------------------ launchers
using dev::bf16s;

#define JEV_DISPATCH_T(m, ...)      \
  if ((m).dtype == 1) {             \
    using T = bf16s;                \
    __VA_ARGS__                     \
  } else {                          \
    using T = float;                \
    __VA_ARGS__                     \
  }

hipError_t launch_rmsnorm(const ModelDims& m, const void* x, const void* g, int32_t T_, void* h, hipStream_t s) {
  if (T_ <= 0) return hipSuccess;
  JEV_DISPATCH_T(m, {
    JEV_LAUNCH(dev::rmsnorm_kernel<T>, dim3(T_), dim3(256), 0, s, reinterpret_cast<const T*>(x),
                       reinterpret_cast<const T*>(g), m.d, m.eps, reinterpret_cast<T*>(h));
  })
  return hipGetLastError();
}

hipError_t launch_embed_norm(const ModelDims& m, const void* embed, const int32_t* tok, int32_t T_, const void* g,
                             void* x, void* h, hipStream_t s, const void* up_src, void* up_dst, int64_t up_bytes) {
  if (T_ <= 0) return hipSuccess;
  if (up_bytes < 0 || up_bytes % 16 || up_bytes / 16 > INT32_MAX || (up_bytes > 0 && (!up_src || !up_dst)))
    return hipErrorInvalidValue;
  // four rows per block where that still leaves a few blocks per CU
  JEV_DISPATCH_T(m, {
    if (T_ >= 1024)
      JEV_LAUNCH((dev::embed_norm_kernel<T, 4>), dim3((T_ + 3) / 4), dim3(256), 0, s,
                 reinterpret_cast<const T*>(embed), tok, T_, m.d, reinterpret_cast<const T*>(g), m.eps,
                 reinterpret_cast<T*>(x), reinterpret_cast<T*>(h), reinterpret_cast<const dev::u32x4*>(up_src),
                 reinterpret_cast<dev::u32x4*>(up_dst), int(up_bytes / 16));
    else
      JEV_LAUNCH((dev::embed_norm_kernel<T, 1>), dim3(T_), dim3(256), 0, s, reinterpret_cast<const T*>(embed), tok,
                 T_, m.d, reinterpret_cast<const T*>(g), m.eps, reinterpret_cast<T*>(x), reinterpret_cast<T*>(h),
                 reinterpret_cast<const dev::u32x4*>(up_src), reinterpret_cast<dev::u32x4*>(up_dst),
                 int(up_bytes / 16));
  })
  return hipGetLastError();
}

hipError_t launch_split_res_norm(const ModelDims& m, const float* partial, int32_t splits, int32_t T_, void* x,
                                 const void* g, void* h, hipStream_t s) {
  if (T_ <= 0) return hipSuccess;
  if (T_ > kSplitRows || splits < 1 || splits > kMaxSplits) return hipErrorInvalidValue;
  // the slice loads of all chunks of a row are held in registers together:
  // as many chunks as the row has
  JEV_DISPATCH_T(m, {
    constexpr int ROW_CHUNK = 256 * 16 / (int)sizeof(T);
    const int nv = (m.d + ROW_CHUNK - 1) / ROW_CHUNK;
    if (nv <= 1)
      JEV_LAUNCH((dev::split_res_norm_kernel<T, 1>), dim3(T_), dim3(256), 0, s, partial, splits, m.d,
                 reinterpret_cast<T*>(x), reinterpret_cast<const T*>(g), m.eps, reinterpret_cast<T*>(h));
    else if (nv == 2)
      JEV_LAUNCH((dev::split_res_norm_kernel<T, 2>), dim3(T_), dim3(256), 0, s, partial, splits, m.d,
                 reinterpret_cast<T*>(x), reinterpret_cast<const T*>(g), m.eps, reinterpret_cast<T*>(h));
    else
      JEV_LAUNCH((dev::split_res_norm_kernel<T, 4>), dim3(T_), dim3(256), 0, s, partial, splits, m.d,
                 reinterpret_cast<T*>(x), reinterpret_cast<const T*>(g), m.eps, reinterpret_cast<T*>(h));
  })
  return hipGetLastError();
}

hipError_t launch_attention(const ModelDims& m, int32_t layer, const AttnTile* tiles, int32_t n_tiles,
                            const int32_t* page_list, const int32_t* tok_pos, const void* qbuf, const void* pool,
                            void* o, float* part_o, float* part_lse, int32_t groups, hipStream_t s,
                            const int32_t* qrows) {
  if (n_tiles <= 0) return hipSuccess;
  if (groups != 1 && groups != 2) return hipErrorInvalidValue;
  const size_t layer_base = (size_t)layer * m.n_pages * m.hkv * 2 * 16 * m.dh;
  const float scale_log2 = float(1.4426950408889634 / std::sqrt((double)m.dh));
  dim3 grid(n_tiles * m.hkv);
  const dim3 block(256 * groups);
#define JEV_ATTN(T_, DH_, G_)                                                                              \
  JEV_LAUNCH((dev::attn_kernel<T_, DH_, G_>), grid, block, 0, s, tiles, page_list, tok_pos,                 \
             reinterpret_cast<const T_*>(qbuf), reinterpret_cast<const T_*>(pool), reinterpret_cast<T_*>(o), \
             part_o, part_lse, m.hq, m.hkv, layer_base, scale_log2, qrows)
  if (m.dtype == 1 && m.dh == 128) {
    if (groups == 2)
      JEV_ATTN(bf16s, 128, 2);
    else
      JEV_ATTN(bf16s, 128, 1);
  } else if (m.dtype == 0 && m.dh == 64) {
    if (groups == 2)
      JEV_ATTN(float, 64, 2);
    else
      JEV_ATTN(float, 64, 1);
  } else {
    return hipErrorInvalidValue;
  }
#undef JEV_ATTN
  return hipGetLastError();
}

hipError_t launch_merge(const ModelDims& m, const MergeItem* items, int32_t n_items, const float* part_o,
                        const float* part_lse, void* o, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  if (m.dtype == 1 && m.dh == 128) {
    JEV_LAUNCH((dev::merge_kernel<bf16s, 128>), dim3(n_items * m.hkv), dim3(256), 0, s, items, part_o, part_lse,
                       reinterpret_cast<bf16s*>(o), m.hq, m.hkv);
  } else if (m.dtype == 0 && m.dh == 64) {
    JEV_LAUNCH((dev::merge_kernel<float, 64>), dim3(n_items * m.hkv), dim3(256), 0, s, items, part_o, part_lse,
                       reinterpret_cast<float*>(o), m.hq, m.hkv);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_poison_pages(const ModelDims& m, void* pool, int32_t first, int32_t count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  if (first < 0 || count > m.n_pages - first) return hipErrorInvalidValue;
  const size_t elt = m.dtype == 1 ? 2 : 4;
  const size_t page_bytes = (size_t)m.hkv * 2 * 16 * m.dh * elt;  // a multiple of 16 (dh >= 64)
  const size_t page_units = page_bytes / 16;
  const size_t total = page_units * (size_t)count * (size_t)m.n_layers;
  const unsigned blocks = (unsigned)std::min<size_t>((total + 255) / 256, 65536);
  JEV_LAUNCH(dev::poison_pages_kernel, dim3(blocks), dim3(256), 0, s, reinterpret_cast<dev::u32x4*>(pool),
             page_units * (size_t)m.n_pages, page_units, first, count, m.n_layers);
  return hipGetLastError();
}

hipError_t launch_readout(const ModelDims& m, const void* unembed, const void* final_norm, const void* x,
                          const ReadoutItem* items, int32_t n_items, const int32_t* labels, float* probs,
                          hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  const size_t shmem = (size_t)(m.d + 64) * sizeof(float);
  JEV_DISPATCH_T(m, {
    JEV_LAUNCH(dev::readout_kernel<T>, dim3(n_items), dim3(256), shmem, s,
                       reinterpret_cast<const T*>(unembed), reinterpret_cast<const T*>(final_norm),
                       reinterpret_cast<const T*>(x), items, labels, probs, m.d, m.eps);
  })
  return hipGetLastError();
}

}  // namespace jev
