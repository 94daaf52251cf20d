// Projection GEMMs of the scoring path on gfx950 MFMA (fp32 accumulation).
//
//   C[M, N] = A[M, K] . B[N, K]^T   (A = activations, B rows = weight rows)
//
// Two shapes occur.  Prefix prefill: M = prefix tokens (thousands), compute
// bound.  Branch scoring: M = suffix tokens of all branches (a few hundred),
// bound by streaming the weights once.
//
// Tiles of 256 rows x BN columns; BN = 160 where it makes the tile count fit
// the 256 CUs (QKV at 2,000 rows: 8 x 32 tiles), else 128.  Up to 256 rows
// (branch scoring) K is split over several workgroups per column tile so that
// the weights stream from every CU.  Full-K bf16 tiles run gemm_pc_kernel:
// gemm_dl_kernel's four MFMA waves (operands loaded straight into LDS, three
// stages deep) with the loads issued by four loader waves.  The split-K tiles
// and float32 run gemm_kernel (register-staged loads, eight waves).
//
// Epilogues run on an fp32 tile staged in LDS (full K) or in the fp32 scratch
// (split K), so their element mapping is independent of the MFMA layout:
//  * QKV: columns are ordered so that every tile holds whole rotate-half pairs
//    (first elements, then their partners, then V columns); RoPE at the
//    token's logical position, then q -> round buffer, k and v -> the token's
//    KV page (V transposed within the page);
//  * RES: x = x + acc (the residual add of the output projection).
#include <algorithm>
#include <cmath>

#include "common.hpp"
#include "launch.hpp"

namespace jev {
namespace dev {

// --------------------------------------------------------------- column map
struct ColMap {
  const void* wq;
  const void* wk;
  const void* wv;
  int hq, hkv, dh;
  int n_pairs;  // (hq + hkv) * dh / 2 rotate-half pairs (0: identity map)
};

enum { COL_FIRST = 0, COL_SECOND = 1, COL_V = 2 };

struct ColInfo {
  int kind;
  int pair;  // FIRST/SECOND
  int vcol;  // V
};

// Column j of tile t (tile width BN) in the pair-ordered QKV layout.
__device__ __forceinline__ ColInfo qkv_col(const ColMap& cm, int BN, int t, int j) {
  const int half = BN >> 1;
  const int np_t = max(0, min(half, cm.n_pairs - half * t));
  const int pairs_before = min(cm.n_pairs, half * t);
  ColInfo ci;
  if (j < np_t) {
    ci.kind = COL_FIRST;
    ci.pair = half * t + j;
    ci.vcol = 0;
  } else if (j < 2 * np_t) {
    ci.kind = COL_SECOND;
    ci.pair = half * t + j - np_t;
    ci.vcol = 0;
  } else {
    ci.kind = COL_V;
    ci.pair = 0;
    ci.vcol = BN * t - 2 * pairs_before + (j - 2 * np_t);
  }
  return ci;
}

template <typename T>
__device__ __forceinline__ const T* weight_row(const ColMap& cm, int BN, int n, int K) {
  if (cm.n_pairs == 0) return reinterpret_cast<const T*>(cm.wq) + (size_t)n * K;
  const ColInfo ci = qkv_col(cm, BN, n / BN, n % BN);
  if (ci.kind == COL_V) return reinterpret_cast<const T*>(cm.wv) + (size_t)ci.vcol * K;
  const int h2 = cm.dh >> 1;
  const int head = ci.pair / h2, i = ci.pair % h2;
  const int f = i + (ci.kind == COL_SECOND ? h2 : 0);
  if (head < cm.hq) return reinterpret_cast<const T*>(cm.wq) + ((size_t)head * cm.dh + f) * K;
  return reinterpret_cast<const T*>(cm.wk) + ((size_t)(head - cm.hq) * cm.dh + f) * K;
}

struct QkvOut {
  const int32_t* pos;
  const int32_t* kvslot;
  const float2* rope;
  void* qbuf;
  void* pool;        // this layer's pages
  int hq, hkv, dh;
};

struct ResOut {
  void* x;
  int ld;
  const int32_t* rows;  // row r of the product updates x row rows[r] (null: row r)
};

enum { EPI_QKV = 0, EPI_RES = 1 };

// Eight consecutive stored elements <-> fp32 (16 bytes of bf16, 32 of fp32).
// The address is aligned to the eight elements.
template <typename T>
__device__ __forceinline__ void load8(const T* src, float v[8]);
template <>
__device__ __forceinline__ void load8<bf16s>(const bf16s* src, float v[8]) {
  const u32x4 u = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(u[i] << 16);
    v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* src, float v[8]) {
  const float4 a = reinterpret_cast<const float4*>(src)[0], b = reinterpret_cast<const float4*>(src)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <typename T>
__device__ __forceinline__ void store8(T* dst, const float v[8]);
template <>
__device__ __forceinline__ void store8<bf16s>(bf16s* dst, const float v[8]) {
  u32x4 u;
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = uint32_t(from_f32<bf16s>(v[2 * i]).bits) | (uint32_t(from_f32<bf16s>(v[2 * i + 1]).bits) << 16);
  *reinterpret_cast<u32x4*>(dst) = u;
}
template <>
__device__ __forceinline__ void store8<float>(float* dst, const float v[8]) {
  reinterpret_cast<float4*>(dst)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(dst)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// What the epilogue of a tile reads besides the tile, for a thread's first
// unit of each kind (for tiles of at most 16 rows every thread has at most one
// unit of each kind): loaded before the tile exists, so that those loads and
// the tile's own overlap.  The same index rules as tile_epilogue.
struct EpiPre {
  float xv[8];        // RES: the row's x elements
  int pos;            // QKV pairs: the row's position
  int sl;             // QKV pairs: the row's KV slot (key heads)
  float4 cs01, cs23;  // QKV pairs: (cos, sin) of its four pairs
  int slv[8];         // QKV V columns: the KV slots of the unit's 8 rows
};

// first part: loads that depend on nothing.  Every thread loads (rows and
// units clamped into the tile, so every address is valid), which keeps the
// code free of branches and lets the second part wait for these loads alone.
template <typename T, int EPI>
__device__ __forceinline__ void epilogue_preload(int rows, int m0, int M, int nt, int BN, const ColMap& cm,
                                                 const QkvOut& qo, const ResOut& ro, int tid, int nthreads,
                                                 EpiPre* pre) {
  rows = min(rows, M - m0);
  if constexpr (EPI == EPI_RES) {
    const int cpr = BN / 8;
    const int r = min(tid / cpr, rows - 1);
    const int xr = ro.rows ? ro.rows[m0 + r] : m0 + r;
    load8<T>(reinterpret_cast<const T*>(ro.x) + (size_t)xr * ro.ld + (size_t)nt * BN + 8 * (tid % cpr), pre->xv);
  } else {
    const int half = BN >> 1;
    const int np_t = max(0, min(half, cm.n_pairs - half * nt));
    if (np_t > 0) {
      const int r = min(tid / (np_t >> 2), rows - 1);
      pre->pos = qo.pos[m0 + r];
      pre->sl = qo.kvslot[m0 + r];
    }
    const int nv = BN - 2 * np_t;
    if (nv > 0) {
      const int r = min((tid / nv) * 8, rows - 1);
#pragma unroll
      for (int q = 0; q < 8; ++q) pre->slv[q] = qo.kvslot[m0 + min(r + q, rows - 1)];
    }
  }
}

// second part: the rotation table rows at the positions of the first part
template <int EPI>
__device__ __forceinline__ void epilogue_preload_rope(int nt, int BN, const ColMap& cm, const QkvOut& qo, int tid,
                                                      EpiPre* pre) {
  if constexpr (EPI == EPI_QKV) {
    const int h2 = cm.dh >> 1;
    const int half = BN >> 1;
    const int np_t = max(0, min(half, cm.n_pairs - half * nt));
    const int pairs_before = min(cm.n_pairs, half * nt);
    if (np_t > 0) {
      const int i0 = (pairs_before + 4 * (tid % (np_t >> 2))) % h2;
      const float4* rp = reinterpret_cast<const float4*>(qo.rope + (size_t)pre->pos * h2 + i0);
      pre->cs01 = rp[0];
      pre->cs23 = rp[1];
    }
  }
}

// Epilogue over an fp32 tile: rows [0, rows) are output rows m0.., columns
// [0, BN) are column tile nt; element (r, j) at tile[r * ld + j] (LDS or
// global).  Work is cut into vector units so that every thread issues 16-byte
// loads and stores:
//  * RES: 8 columns of one row, x += tile;
//  * QKV, rotate-half pairs: 4 consecutive pairs (i, i + dh/2) of one row and
//    head, rotated at the row's position and written as 8 adjacent elements
//    (pair i at 2i, 2i+1) of q or of the row's K page slot;
//  * QKV, V columns: one column over 8 rows; when the rows' KV slots are 8
//    consecutive, 8-aligned slots of one page (the usual case) they are one
//    16-byte run of the transposed V block, else single stores.
template <typename T, int EPI, bool PRE = false>
__device__ __forceinline__ void tile_epilogue(const float* tile, int ld, int rows, int m0, int M, int nt, int BN,
                                              const ColMap& cm, const QkvOut& qo, const ResOut& ro, int tid,
                                              int nthreads, const EpiPre* pre = nullptr) {
  rows = min(rows, M - m0);
  if constexpr (EPI == EPI_RES) {
    const int cpr = BN / 8;
    const int rstep = nthreads / cpr;
    const int c8 = tid % cpr;
    for (int r = tid / cpr; r < rows && tid < rstep * cpr; r += rstep) {
      const int xr = ro.rows ? ro.rows[m0 + r] : m0 + r;
      T* xp = reinterpret_cast<T*>(ro.x) + (size_t)xr * ro.ld + (size_t)nt * BN + 8 * c8;
      const float* tp = tile + (size_t)r * ld + 8 * c8;
      float v[8];
      if (PRE && r == tid / cpr) {
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = pre->xv[q];
      } else {
        load8<T>(xp, v);
      }
      const float4 t0 = reinterpret_cast<const float4*>(tp)[0], t1 = reinterpret_cast<const float4*>(tp)[1];
      v[0] += t0.x; v[1] += t0.y; v[2] += t0.z; v[3] += t0.w;
      v[4] += t1.x; v[5] += t1.y; v[6] += t1.z; v[7] += t1.w;
      store8<T>(xp, v);
    }
  } else {
    const int h2 = cm.dh >> 1;
    const int half = BN >> 1;
    const int np_t = max(0, min(half, cm.n_pairs - half * nt));
    const int pairs_before = min(cm.n_pairs, half * nt);
    const size_t pe = (size_t)16 * qo.dh;
    T* __restrict__ qbuf = reinterpret_cast<T*>(qo.qbuf);
    T* __restrict__ pool = reinterpret_cast<T*>(qo.pool);
    if (np_t > 0) {
      const int g4 = np_t >> 2;  // units of 4 pairs per row
      const int rstep = nthreads / g4;
      const int g = tid % g4;
      const int p0 = pairs_before + 4 * g;  // global pair index of the unit
      const int head = p0 / h2, i0 = p0 % h2;
      for (int r = tid / g4; r < rows && tid < rstep * g4; r += rstep) {
        const int m = m0 + r;
        const float* tp = tile + (size_t)r * ld + 4 * g;
        const float4 a0 = *reinterpret_cast<const float4*>(tp);
        const float4 a1 = *reinterpret_cast<const float4*>(tp + np_t);
        const bool first = PRE && r == tid / g4;
        float4 cs01, cs23;  // (cos, sin) of pairs i0 .. i0+3
        if (first) {
          cs01 = pre->cs01;
          cs23 = pre->cs23;
        } else {
          const float4* rp = reinterpret_cast<const float4*>(qo.rope + (size_t)qo.pos[m] * h2 + i0);
          cs01 = rp[0];
          cs23 = rp[1];
        }
        float v[8];
        v[0] = a0.x * cs01.x - a1.x * cs01.y; v[1] = a1.x * cs01.x + a0.x * cs01.y;
        v[2] = a0.y * cs01.z - a1.y * cs01.w; v[3] = a1.y * cs01.z + a0.y * cs01.w;
        v[4] = a0.z * cs23.x - a1.z * cs23.y; v[5] = a1.z * cs23.x + a0.z * cs23.y;
        v[6] = a0.w * cs23.z - a1.w * cs23.w; v[7] = a1.w * cs23.z + a0.w * cs23.w;
        // q and k store each rotate-half pair (i, i + dh/2) adjacently, at
        // 2i and 2i+1: both sides of every q.k product use the same order
        T* dst;
        if (head < cm.hq) {
          dst = qbuf + ((size_t)m * qo.hq + head) * qo.dh + 2 * i0;
        } else {
          const int sl = first ? pre->sl : qo.kvslot[m];
          dst = pool + ((size_t)(sl >> 4) * qo.hkv + (head - cm.hq)) * 2 * pe + (size_t)(sl & 15) * qo.dh + 2 * i0;
        }
        store8<T>(dst, v);
      }
    }
    const int nv = BN - 2 * np_t;  // V columns of this tile
    if (nv > 0) {
      const int vcol0 = BN * nt - 2 * pairs_before;
      const int rstep = (nthreads / nv) * 8;
      const int j = tid % nv;
      const int vcol = vcol0 + j, head = vcol / qo.dh, f = vcol % qo.dh;
      T* vb_head = pool + (size_t)head * 2 * pe + pe + (size_t)f * 16;
      for (int r = (tid / nv) * 8; r < rows && tid < (nthreads / nv) * nv; r += rstep) {
        const float* tp = tile + (size_t)r * ld + 2 * np_t + j;
        const int n = min(8, rows - r);
        int sl[8];
        float v[8];
        const bool first = PRE && r == (tid / nv) * 8;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          sl[q] = first ? pre->slv[q] : qo.kvslot[m0 + r + min(q, n - 1)];
          v[q] = tp[(size_t)min(q, n - 1) * ld];
        }
        bool run = n == 8 && (sl[0] & 7) == 0;
#pragma unroll
        for (int q = 1; q < 8; ++q) run = run && sl[q] == sl[0] + q;
        if (run) {
          store8<T>(vb_head + (size_t)(sl[0] >> 4) * qo.hkv * 2 * pe + (sl[0] & 15), v);
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q)
            if (q < n) vb_head[(size_t)(sl[q] >> 4) * qo.hkv * 2 * pe + (sl[q] & 15)] = from_f32<T>(v[q]);
        }
      }
    }
  }
}

// Workgroup -> tile mapping.  Consecutive workgroup ids go to the 8 XCDs in
// turn, and each XCD has its own L2; tiles are therefore enumerated in groups of
// up to 4 row tiles (column-major inside a group) and the tile list is cut into
// 8 contiguous parts, part x running on XCD x, so that an XCD's workgroups share
// A row tiles and B column tiles in its L2.
__device__ __forceinline__ void xcd_tile(int b, int n_blocks, int m_tiles, int* mt, int* nt) {
  const int n_tiles_n = n_blocks / m_tiles;
  int t = b;
  if (n_blocks % 8 == 0) t = (b % 8) * (n_blocks / 8) + b / 8;
  const int gm = min(4, m_tiles);
  const int group = t / (gm * n_tiles_n);
  const int first_m = group * gm;
  const int rows_in_group = min(gm, m_tiles - first_m);
  const int within = t - group * gm * n_tiles_n;
  *mt = first_m + within % rows_in_group;
  *nt = within / rows_in_group;
}

// --------------------------------------------------------------- main kernel
// Block = 4 waves over a 256-row x BN-column tile; wave w owns rows
// [64w, 64w+64) and all BN columns (2 x BN/32 MFMA 32x32 blocks).  Both
// operands are staged through LDS: global loads are fully coalesced (8 lanes
// per 128-byte row segment), held in registers two K stages ahead and written
// to a double-buffered LDS stage whose rows are padded to 144 bytes, so that
// the 16 rows touched by one 16-lane fragment read (or one 16-lane write) fall
// in different bank groups; the stores of the next stage are spread between
// the MFMAs of the current one.  One barrier per 128-byte K stage.  With SPLIT,
// blockIdx.y selects a slice of K and the fp32 partial tile is stored to its
// own [256][N] scratch slice; split_epilogue (next launch) sums the slices and
// runs the epilogue.
//
// BM_ = 64 (split K only): the same K slices, stages, k-steps and MFMA shape
// on a 64-row tile, for rounds of at most 64 rows; every output element is
// summed in the same order as on the 256-row tile, so the partial slices are
// bitwise those of the 256-row kernel.
template <typename T, int BN, int EPI, bool SPLIT, int WM, int WN, int BM_ = 256>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(WM * WN / 4, WM * WN / 4))) void gemm_kernel(const T* __restrict__ A, int M, int K, int N, ColMap cm,
                                                   QkvOut qo, ResOut ro, float* __restrict__ scratch) {
  using MF = Mfma<T>;
  using frag = typename MF::frag;
  constexpr int BM = BM_;
  static_assert(BM == 256 || SPLIT, "row tiles below 256 rows are split-K only");
  constexpr int CH = 16 / sizeof(T);   // elements per 16-byte chunk
  constexpr int BK = 8 * CH;           // 128 bytes of K per stage
  constexpr int KS = BK / MF::KSTEP;   // MFMA k-steps per stage
  constexpr int NTH = WM * WN * 64;
  constexpr int NRB = BM / WM / 32;    // row blocks per wave
  constexpr int TN = BN / WN / 32;     // column blocks per wave
  constexpr int RPL = NTH / 8;         // rows per staging load (8 lanes per 128-byte row)
  constexpr int LA = BM / RPL;         // A chunks per thread per stage
  constexpr int LB = (BN + RPL - 1) / RPL;  // B chunks per thread per stage (the last may idle)
  constexpr int NST = LA + LB;         // LDS stores per thread per stage
  constexpr bool B_FULL = BN % RPL == 0;  // every thread's B rows are inside the tile (lrow < RPL)
  constexpr int RS = 9;                // LDS row stride, 16-byte units
  constexpr int STAGE = (BM + BN) * RS;
  constexpr int LDS_MAIN = 2 * STAGE;
  constexpr int LDS_EPI = 128 * (BN + 4) / 4;
  constexpr int LDS_UNITS = LDS_MAIN > LDS_EPI ? LDS_MAIN : LDS_EPI;
  static_assert(BM % (WM * 32) == 0 && BN % (WN * 32) == 0 && BM % RPL == 0 && KS % 2 == 0, "tile");
  __shared__ __attribute__((aligned(16))) u32x4 smem[LDS_UNITS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 31, hh = lane >> 5;
  const int rowA0 = (BM / WM) * (wave / WN), colB0 = (BN / WN) * (wave % WN);
  int mt, nt;
  if (SPLIT) {
    mt = 0;
    nt = blockIdx.x;
  } else {
    xcd_tile(blockIdx.x, gridDim.x, (M + BM - 1) / BM, &mt, &nt);
  }
  const int m0 = mt * BM, n0 = nt * BN;
  const int lrow = tid >> 3, lch = tid & 7;
  const int KTall = K / BK;
  const int kt0 = SPLIT ? (KTall * (int)blockIdx.y) / (int)gridDim.y : 0;
  const int KT = SPLIT ? (KTall * ((int)blockIdx.y + 1)) / (int)gridDim.y - kt0 : KTall;

  const u32x4* ap[LA];
#pragma unroll
  for (int i = 0; i < LA; ++i)
    ap[i] = reinterpret_cast<const u32x4*>(A + (size_t)min(m0 + lrow + RPL * i, M - 1) * K + (size_t)kt0 * BK) + lch;
  const u32x4* bp[LB];
#pragma unroll
  for (int i = 0; i < LB; ++i)
    bp[i] = reinterpret_cast<const u32x4*>(weight_row<T>(cm, BN, n0 + min(lrow + RPL * i, BN - 1), K) +
                                           (size_t)kt0 * BK) + lch;

  f32x16 acc[NRB][TN];
#pragma unroll
  for (int i = 0; i < NRB; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  u32x4 ra0[LA], rb0[LB], ra1[LA], rb1[LB];
#define G_LOAD(RA, RB, KT_)                                                                 \
  do {                                                                                      \
    const int kk_ = min((KT_), KT - 1) * 8;                                                 \
    _Pragma("unroll") for (int i = 0; i < LA; ++i) RA[i] = ap[i][kk_];                      \
    _Pragma("unroll") for (int i = 0; i < LB; ++i) RB[i] = bp[i][kk_];                      \
  } while (0)
#define G_STORE(RA, RB, BUF)                                                                \
  do {                                                                                      \
    u32x4* sA_ = smem + (BUF) * STAGE;                                                      \
    u32x4* sB_ = sA_ + BM * RS;                                                             \
    _Pragma("unroll") for (int i = 0; i < LA; ++i) sA_[(lrow + RPL * i) * RS + lch] = RA[i]; \
    _Pragma("unroll") for (int i = 0; i < LB; ++i) if (B_FULL || lrow + RPL * i < BN) sB_[(lrow + RPL * i) * RS + lch] = RB[i]; \
  } while (0)
  // One stage of compute on LDS buffer BUF, with the next stage's staged
  // registers (RA, RB) written into the other buffer during it (W_ = 1).
  // Fragments of k-step s+1 are read into the other fragment set before the
  // MFMAs of k-step s; inside each k-step's region the scheduling groups put
  // one LDS read or write between consecutive MFMAs, so LDS traffic overlaps
  // MFMA execution instead of following it.
#define G_FRAGS(FA, FB, S_)                                                                      \
  do {                                                                                           \
    const int k_ = (S_) * MF::KSTEP + MF::KL * hh;                                               \
    _Pragma("unroll") for (int i = 0; i < NRB; ++i) FA[i] =                                      \
        MF::load(reinterpret_cast<const T*>(&sA_[(rowA0 + 32 * i + c) * RS + k_ / CH]) + k_ % CH); \
    _Pragma("unroll") for (int j = 0; j < TN; ++j) FB[j] =                                       \
        MF::load(reinterpret_cast<const T*>(&sB_[(colB0 + 32 * j + c) * RS + k_ / CH]) + k_ % CH); \
  } while (0)
#define G_MMA(FA, FB)                                                                            \
  do {                                                                                           \
    _Pragma("unroll") for (int i = 0; i < NRB; ++i) _Pragma("unroll") for (int j = 0; j < TN; ++j) \
        acc[i][j] = MF::mma(FA[i], FB[j], acc[i][j]);                                            \
  } while (0)
#define G_WRITES(RA, RB, S_)                                                                     \
  do {                                                                                           \
    _Pragma("unroll") for (int q = (S_) * NST / KS; q < ((S_) + 1) * NST / KS; ++q) {            \
      if (q < LA) wA_[(lrow + RPL * q) * RS + lch] = RA[q < LA ? q : 0];                         \
      else if (B_FULL || lrow + RPL * (q - LA) < BN) wB_[(lrow + RPL * (q - LA)) * RS + lch] = RB[q < LA ? 0 : q - LA]; \
    }                                                                                            \
  } while (0)
#define G_GROUPS(NR_, NW_)                                                                       \
  do {                                                                                           \
    _Pragma("unroll") for (int m_ = 0; m_ < NRB * TN; ++m_) {                                    \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                         \
      if (m_ < (NR_)) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                         \
      if (m_ < (NW_)) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);                         \
    }                                                                                            \
  } while (0)
#define G_PHASE(BUF, RA, RB, W_)                                                                 \
  do {                                                                                           \
    const u32x4* sA_ = smem + (BUF) * STAGE;                                                     \
    const u32x4* sB_ = sA_ + BM * RS;                                                            \
    u32x4* wA_ = smem + ((BUF) ^ 1) * STAGE;                                                     \
    u32x4* wB_ = wA_ + BM * RS;                                                                  \
    (void)wA_;                                                                                   \
    (void)wB_;                                                                                   \
    frag fa0[NRB], fb0[TN], fa1[NRB], fb1[TN];                                                   \
    G_FRAGS(fa0, fb0, 0);                                                                        \
    __builtin_amdgcn_sched_barrier(0);                                                           \
    _Pragma("unroll") for (int s = 0; s < KS; s += 2) {                                          \
      if (s + 1 < KS) G_FRAGS(fa1, fb1, s + 1);                                                  \
      G_MMA(fa0, fb0);                                                                           \
      if (W_) G_WRITES(RA, RB, s);                                                               \
      G_GROUPS(s + 1 < KS ? NRB + TN : 0, (W_) ? ((s + 1) * NST / KS - s * NST / KS) : 0);      \
      __builtin_amdgcn_sched_barrier(0);                                                         \
      if (s + 1 < KS) {                                                                          \
        if (s + 2 < KS) G_FRAGS(fa0, fb0, s + 2);                                                \
        G_MMA(fa1, fb1);                                                                         \
        if (W_) G_WRITES(RA, RB, s + 1);                                                         \
        G_GROUPS(s + 2 < KS ? NRB + TN : 0, (W_) ? ((s + 2) * NST / KS - (s + 1) * NST / KS) : 0); \
        __builtin_amdgcn_sched_barrier(0);                                                       \
      }                                                                                          \
    }                                                                                            \
  } while (0)

  // Split K: the stage barrier sits before the MFMAs of the stage's last
  // k-step; after it each wave reads the first fragments of the next stage
  // while those MFMAs run, so the MFMA pipe does not drain at every stage
  // boundary (with ~10 stages per slice, a drained pipe per stage cost about
  // a third of the loop).  All LDS writes of the next stage and all reads of
  // this stage are issued before the barrier.
#define G_PHASE_SPLIT(BUF, RA, RB)                                                               \
  do {                                                                                           \
    const u32x4* sA_ = smem + (BUF) * STAGE;                                                     \
    const u32x4* sB_ = sA_ + BM * RS;                                                            \
    u32x4* wA_ = smem + ((BUF) ^ 1) * STAGE;                                                     \
    u32x4* wB_ = wA_ + BM * RS;                                                                  \
    _Pragma("unroll") for (int s = 0; s < KS; s += 2) {                                          \
      G_FRAGS(fa1, fb1, s + 1);                                                                  \
      G_MMA(fa0, fb0);                                                                           \
      G_WRITES(RA, RB, s);                                                                       \
      G_GROUPS(NRB + TN, (s + 1) * NST / KS - s * NST / KS);                                     \
      __builtin_amdgcn_sched_barrier(0);                                                         \
      if (s + 2 < KS) {                                                                          \
        G_FRAGS(fa0, fb0, s + 2);                                                                \
        G_MMA(fa1, fb1);                                                                         \
        G_WRITES(RA, RB, s + 1);                                                                 \
        G_GROUPS(NRB + TN, (s + 2) * NST / KS - (s + 1) * NST / KS);                             \
        __builtin_amdgcn_sched_barrier(0);                                                       \
      } else {                                                                                   \
        G_WRITES(RA, RB, s + 1);                                                                 \
        __syncthreads();                                                                         \
        {                                                                                        \
          const u32x4* sA_ = smem + ((BUF) ^ 1) * STAGE;                                         \
          const u32x4* sB_ = sA_ + BM * RS;                                                      \
          G_FRAGS(fa0, fb0, 0);                                                                  \
        }                                                                                        \
        G_MMA(fa1, fb1);                                                                         \
        G_GROUPS(NRB + TN, 0);                                                                   \
        __builtin_amdgcn_sched_barrier(0);                                                       \
      }                                                                                          \
    }                                                                                            \
  } while (0)

  G_LOAD(ra0, rb0, 0);
  G_LOAD(ra1, rb1, 1);
  G_STORE(ra0, rb0, 0);
  __syncthreads();
  if constexpr (SPLIT) {
    frag fa0[NRB], fb0[TN], fa1[NRB], fb1[TN];
    {
      const u32x4* sA_ = smem;
      const u32x4* sB_ = sA_ + BM * RS;
      G_FRAGS(fa0, fb0, 0);
    }
    // the last stage's writes store a clamped copy of it into a buffer that
    // no stage reads, and its post-barrier reads fetch unused values
    int kt = 0;
    for (; kt + 1 < KT; kt += 2) {
      G_LOAD(ra0, rb0, kt + 2);
      __builtin_amdgcn_sched_barrier(0);
      G_PHASE_SPLIT(0, ra1, rb1);
      G_LOAD(ra1, rb1, kt + 3);
      __builtin_amdgcn_sched_barrier(0);
      G_PHASE_SPLIT(1, ra0, rb0);
    }
    if (kt < KT) G_PHASE_SPLIT(0, ra1, rb1);
  } else {
    int kt = 0;
    // two stages per trip keep the register sets static
    for (; kt + 1 < KT; kt += 2) {
      G_LOAD(ra0, rb0, kt + 2);
      __builtin_amdgcn_sched_barrier(0);
      G_PHASE(0, ra1, rb1, 1);
      __syncthreads();
      G_LOAD(ra1, rb1, kt + 3);
      __builtin_amdgcn_sched_barrier(0);
      G_PHASE(1, ra0, rb0, 1);
      __syncthreads();
    }
    if (kt < KT) G_PHASE(0, ra1, rb1, 0);
  }
#undef G_LOAD
#undef G_STORE
#undef G_PHASE
#undef G_PHASE_SPLIT
#undef G_FRAGS
#undef G_MMA
#undef G_WRITES
#undef G_GROUPS

  if constexpr (SPLIT) {
    float* part = scratch + (size_t)blockIdx.y * kSplitRows * N;
#pragma unroll
    for (int i = 0; i < NRB; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = rowA0 + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (m < M) part[(size_t)m * N + n0 + colB0 + 32 * j + c] = acc[i][j][r];
        }
  } else {
    float* stile = reinterpret_cast<float*>(smem);
    constexpr int LD = BN + 4;
    __syncthreads();
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (rowA0 / 128 == half) {
#pragma unroll
        for (int i = 0; i < NRB; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = rowA0 % 128 + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
              stile[row * LD + colB0 + 32 * j + c] = acc[i][j][r];
            }
      }
      __syncthreads();
      if (m0 + 128 * half < M)
        tile_epilogue<T, EPI>(stile, LD, 128, m0 + 128 * half, M, nt, BN, cm, qo, ro, tid, NTH);
      __syncthreads();
    }
  }
}

// --------------------------------------------------- large GEMM, direct loads
// LDS unit of 16-byte chunk j of stage row R in the direct-load layout: rows of
// 8 units (128 bytes, unpadded), chunk slots XOR-swizzled by (R / 2) mod 8, so
// that the 16 lanes of a fragment read (16 consecutive rows, one chunk) fall in
// 16 distinct bank groups.
__device__ __forceinline__ int dl_unit(int R, int j) { return R * 8 + (j ^ ((R >> 1) & 7)); }

// Waits until at most N vector memory operations of this wave are outstanding
// and all of its LDS operations are done, then joins the workgroup barrier.
// The direct loads below are vector memory operations that write LDS, so after
// the barrier every wave's loads up to that point have landed.
template <int N>
__device__ __forceinline__ void vm_lds_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Scheduling groups of one k-step region: NMF MFMAs, with the region's NRD LDS
// fragment reads two per MFMA from the first one on (the next region starts
// by waiting for all of them), then NV direct loads spread over the MFMAs after
// those.  (A direct load writes LDS, so the scheduler keeps it after LDS reads
// that precede it in program order: the reads are issued first.)
template <int NMF, int NRD, int NV, int M_ = 0>
__device__ __forceinline__ void dl_groups() {
  if constexpr (M_ < NMF) {
    constexpr int RS = (NRD + 1) / 2;  // MFMAs that take reads
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int r = M_ < RS ? (2 * M_ + 2 <= NRD ? 2 : NRD - 2 * M_) : 0;
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
    constexpr int NT = NMF - RS > 0 ? NMF - RS : 1;  // MFMAs that take loads
    constexpr int q = M_ - (NMF - NT);
    constexpr int v = q < 0 ? 0 : (NV * (q + 1)) / NT - (NV * q) / NT;
    if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x020, v, 0);
    dl_groups<NMF, NRD, NV, M_ + 1>();
  }
}

// Large bf16 GEMM (prefill projections): one 256 x BN tile per workgroup of
// four waves, one wave per SIMD; wave w owns rows [64w, 64w+64) and all BN
// columns (2 x BN/32 MFMA 32x32 blocks, accumulators in the unified register
// file).  Both operands go from global memory straight into LDS
// (global_load_lds, 16 bytes per lane: each instruction fills 8 stage rows of
// 128 bytes, lane l writing slot l of that 1 KB and loading the chunk that the
// swizzle puts there), NSTG stages deep: the loads of stage k + NSTG - 1 are
// issued, between the MFMAs, when stage k starts, into the buffer of stage
// k - 1.  Near the end they reload the last stage into that buffer, which no
// later stage reads, so every wait count is static and the loop body has no
// branch (a branch would make the compiler wait for all LDS reads where its
// paths join).  One barrier per 64-wide K
// stage, placed before the MFMAs of the stage's last k-step: after it the wave
// reads the first fragments of the next stage, and those 10 MFMAs cover the
// read latency, so the MFMA pipe does not drain at stage boundaries.  Same
// tile order and epilogue as gemm_kernel; every output accumulates over K in
// the same order, so the results are bitwise those of gemm_kernel.  (With K
// split over workgroups the loop is ~10 stages long, and this kernel measured
// slower than gemm_kernel there: the split-K GEMMs keep gemm_kernel.)
template <int BN, int EPI, int NSTG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_dl_kernel(
    const bf16s* __restrict__ A, int M, int K, int N, ColMap cm, QkvOut qo, ResOut ro) {
  using T = bf16s;
  using MF = Mfma<T>;
  using frag = typename MF::frag;
  constexpr int BM = 256, NW = 4, NTH = 256;
  constexpr int CH = 8;                    // bf16 per 16-byte chunk
  constexpr int BK = 64;                   // K per stage (128 bytes)
  constexpr int KS = BK / MF::KSTEP;       // 4 k-steps per stage
  constexpr int NRB = 2, TN = BN / 32;
  constexpr int NL = (BM + BN) / 8;        // 1 KB loads per stage
  constexpr int LPW = NL / NW;             // loads per wave per stage
  constexpr int STAGE = (BM + BN) * 8;     // 16-byte units
  constexpr int LDS_MAIN = NSTG * STAGE;
  constexpr int LDS_EPI = 128 * (BN + 4) / 4;
  constexpr int LDS_UNITS = LDS_MAIN > LDS_EPI ? LDS_MAIN : LDS_EPI;
  constexpr int VM_AHEAD = (NSTG - 2) * LPW;  // loads allowed in flight at a stage barrier
  static_assert(KS == 4 && BN % 32 == 0 && NL % NW == 0 && (NSTG == 2 || NSTG == 3), "tile");
  static_assert(LDS_UNITS * 16 <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) u32x4 smem[LDS_UNITS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & 3;
  const int c = lane & 31, hh = lane >> 5;
  const int rowA0 = 64 * wave;
  int mt, nt;
  xcd_tile(blockIdx.x, gridDim.x, (M + BM - 1) / BM, &mt, &nt);
  const int m0 = mt * BM, n0 = nt * BN;
  const int KT = K / BK;

  // this wave's loads: load i fills stage rows 8 li .. 8 li + 7, li = wave + NW i
  const T* src[LPW];
  {
    const int lr = lane >> 3, lp = lane & 7;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int li = wave + NW * i;
      const int R = 8 * li + lr;
      const int j = lp ^ ((R >> 1) & 7);
      src[i] = (R < BM ? A + (size_t)min(m0 + R, M - 1) * K : weight_row<T>(cm, BN, n0 + R - BM, K)) + j * CH;
    }
  }
  // loads [I0, I1) of stage min(kt, KT - 1) into LDS buffer buf
  auto issue = [&](int kt, int buf, int I0, int I1) __attribute__((always_inline)) {
    const size_t koff = (size_t)min(kt, KT - 1) * BK;
    u32x4* dst = smem + buf * STAGE + 64 * wave;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      if (i < I0 || i >= I1) continue;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src[i] + koff),
                                       (__attribute__((address_space(3))) void*)(dst + 64 * NW * i), 16, 0, 0);
    }
  };

  f32x16 acc[NRB][TN];
#pragma unroll
  for (int i = 0; i < NRB; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto frags = [&](const u32x4* st, int s, frag* fa, frag* fb) __attribute__((always_inline)) {
    const int j = 2 * s + hh;  // chunk of this lane's 8 k elements
#pragma unroll
    for (int i = 0; i < NRB; ++i) fa[i] = MF::load(&st[dl_unit(rowA0 + 32 * i + c, j)]);
#pragma unroll
    for (int t = 0; t < TN; ++t) fb[t] = MF::load(&st[dl_unit(BM + 32 * t + c, j)]);
  };
  auto mma = [&](const frag* fa, const frag* fb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NRB; ++i)
#pragma unroll
      for (int t = 0; t < TN; ++t) acc[i][t] = MF::mma(fa[i], fb[t], acc[i][t]);
  };
  // loads of a stage, spread over the three k-step regions before the barrier
  constexpr int P1 = (LPW + 2) / 3, P2 = P1 + (LPW - P1 + 1) / 2;

#pragma unroll
  for (int p = 0; p < NSTG - 1; ++p) issue(p, p, 0, LPW);
  vm_lds_barrier<VM_AHEAD>();  // stage 0 landed
  frag fa0[NRB], fb0[TN], fa1[NRB], fb1[TN];
  frags(smem, 0, fa0, fb0);
  int buf = 0, ibuf = NSTG - 1;  // buffers of stage kt and of stage kt + NSTG - 1
  for (int kt = 0; kt < KT; ++kt) {
    const u32x4* st = smem + buf * STAGE;
    // loads of stage kt + NSTG - 1 go into the buffer of stage kt - 1, which
    // every wave finished reading before the barrier that ended that stage
    frags(st, 1, fa1, fb1);
    issue(kt + NSTG - 1, ibuf, 0, P1);
    mma(fa0, fb0);
    dl_groups<NRB * TN, NRB + TN, P1>();
    __builtin_amdgcn_sched_barrier(0);
    frags(st, 2, fa0, fb0);
    issue(kt + NSTG - 1, ibuf, P1, P2);
    mma(fa1, fb1);
    dl_groups<NRB * TN, NRB + TN, P2 - P1>();
    __builtin_amdgcn_sched_barrier(0);
    frags(st, 3, fa1, fb1);
    issue(kt + NSTG - 1, ibuf, P2, LPW);
    mma(fa0, fb0);
    dl_groups<NRB * TN, NRB + TN, LPW - P2>();
    __builtin_amdgcn_sched_barrier(0);
    // stage kt + 1 landed (the loads of stage kt + 2 may still be in flight);
    // on the last stage the reads below fetch unused values
    vm_lds_barrier<VM_AHEAD>();
    buf = buf + 1 == NSTG ? 0 : buf + 1;
    ibuf = ibuf + 1 == NSTG ? 0 : ibuf + 1;
    frags(smem + buf * STAGE, 0, fa0, fb0);
    mma(fa1, fb1);
    dl_groups<NRB * TN, NRB + TN, 0>();
    __builtin_amdgcn_sched_barrier(0);
  }

  float* stile = reinterpret_cast<float*>(smem);
  constexpr int LD = BN + 4;
  vm_lds_barrier<0>();  // every load and read of the main loop done
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (rowA0 / 128 == half) {
#pragma unroll
      for (int i = 0; i < NRB; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = rowA0 % 128 + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
            stile[row * LD + 32 * t + c] = acc[i][t][r];
          }
    }
    __syncthreads();
    if (m0 + 128 * half < M) tile_epilogue<T, EPI>(stile, LD, 128, m0 + 128 * half, M, nt, BN, cm, qo, ro, tid, NTH);
    __syncthreads();
  }
}

// gemm_dl_kernel with the direct loads moved to four loader waves (one per
// SIMD, next to its MFMA wave; two waves per SIMD, 226 registers each): the
// MFMA waves only read fragments and multiply, and no longer wait on memory
// counters; a loader wave issues its share of stage k + 2 when stage k
// starts, then waits for stage k + 1 and joins the stage barrier.  Same
// tile, LDS layout, k order and epilogue (run by all eight waves): results
// are bitwise those of gemm_dl_kernel.  Measured 4% faster on the QKV GEMM
// at 2,000 rows (81 vs 84.4 us in the bench).  BM = 128 (MFMA waves of 32
// rows) makes twice the tiles for narrow products; every output element still
// accumulates its K in the same order, so the values do not depend on BM.
template <int BM, int BN, int EPI>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_pc_kernel(
    const bf16s* __restrict__ A, int M, int K, int N, ColMap cm, QkvOut qo, ResOut ro) {
  using T = bf16s;
  using MF = Mfma<T>;
  using frag = typename MF::frag;
  constexpr int NW = 4, NTH = 512;
  constexpr int CH = 8, BK = 64, KS = BK / MF::KSTEP;
  constexpr int NSTG = 3;
  constexpr int NRB = BM / 128, TN = BN / 32;
  constexpr int NL = (BM + BN) / 8;
  constexpr int LPW = NL / NW;             // loads per loader wave per stage
  constexpr int STAGE = (BM + BN) * 8;
  constexpr int LDS_MAIN = NSTG * STAGE;
  constexpr int LDS_EPI = 128 * (BN + 4) / 4;
  constexpr int LDS_UNITS = LDS_MAIN > LDS_EPI ? LDS_MAIN : LDS_EPI;
  static_assert(KS == 4 && BN % 32 == 0 && NL % NW == 0 && (BM == 128 || BM == 256), "tile");
  static_assert(LDS_UNITS * 16 <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) u32x4 smem[LDS_UNITS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & 7;
  const int w4 = wave & 3;
  const int c = lane & 31, hh = lane >> 5;
  const int rowA0 = (BM / 4) * w4;
  int mt, nt;
  xcd_tile(blockIdx.x, gridDim.x, (M + BM - 1) / BM, &mt, &nt);
  const int m0 = mt * BM, n0 = nt * BN;
  const int KT = K / BK;

  f32x16 acc[NRB][TN];
  if (wave >= NW) {
    // loader wave w4: load i fills stage rows 8 li .. 8 li + 7, li = w4 + NW i
    const T* src[LPW];
    {
      const int lr = lane >> 3, lp = lane & 7;
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int R = 8 * (w4 + NW * i) + lr;
        const int j = lp ^ ((R >> 1) & 7);
        src[i] = (R < BM ? A + (size_t)min(m0 + R, M - 1) * K : weight_row<T>(cm, BN, n0 + R - BM, K)) + j * CH;
      }
    }
    auto issue = [&](int kt, int buf) __attribute__((always_inline)) {
      const size_t koff = (size_t)min(kt, KT - 1) * BK;
      u32x4* dst = smem + buf * STAGE + 64 * w4;
#pragma unroll
      for (int i = 0; i < LPW; ++i)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src[i] + koff),
                                         (__attribute__((address_space(3))) void*)(dst + 64 * NW * i), 16, 0, 0);
    };
    issue(0, 0);
    issue(1, 1);
    vm_lds_barrier<LPW>();  // stage 0 landed
    int ibuf = NSTG - 1;
    for (int kt = 0; kt < KT; ++kt) {
      // stage kt + 2 into the buffer of stage kt - 1, which every MFMA wave
      // finished reading before the last barrier
      issue(kt + NSTG - 1, ibuf);
      vm_lds_barrier<LPW>();  // stage kt + 1 landed
      ibuf = ibuf + 1 == NSTG ? 0 : ibuf + 1;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NRB; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    auto frags = [&](const u32x4* st, int s, frag* fa, frag* fb) __attribute__((always_inline)) {
      const int j = 2 * s + hh;
#pragma unroll
      for (int i = 0; i < NRB; ++i) fa[i] = MF::load(&st[dl_unit(rowA0 + 32 * i + c, j)]);
#pragma unroll
      for (int t = 0; t < TN; ++t) fb[t] = MF::load(&st[dl_unit(BM + 32 * t + c, j)]);
    };
    auto mma = [&](const frag* fa, const frag* fb) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < NRB; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t) acc[i][t] = MF::mma(fa[i], fb[t], acc[i][t]);
    };
    vm_lds_barrier<0>();  // stage 0 landed
    frag fa0[NRB], fb0[TN], fa1[NRB], fb1[TN];
    frags(smem, 0, fa0, fb0);
    int buf = 0;
    for (int kt = 0; kt < KT; ++kt) {
      const u32x4* st = smem + buf * STAGE;
      frags(st, 1, fa1, fb1);
      mma(fa0, fb0);
      dl_groups<NRB * TN, NRB + TN, 0>();
      __builtin_amdgcn_sched_barrier(0);
      frags(st, 2, fa0, fb0);
      mma(fa1, fb1);
      dl_groups<NRB * TN, NRB + TN, 0>();
      __builtin_amdgcn_sched_barrier(0);
      frags(st, 3, fa1, fb1);
      mma(fa0, fb0);
      dl_groups<NRB * TN, NRB + TN, 0>();
      __builtin_amdgcn_sched_barrier(0);
      vm_lds_barrier<0>();  // stage kt + 1 landed; stage kt fully read
      buf = buf + 1 == NSTG ? 0 : buf + 1;
      frags(smem + buf * STAGE, 0, fa0, fb0);
      mma(fa1, fb1);
      dl_groups<NRB * TN, NRB + TN, 0>();
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  float* stile = reinterpret_cast<float*>(smem);
  constexpr int LD = BN + 4;
  vm_lds_barrier<0>();  // every load and read of the main loop done
#pragma unroll
  for (int half = 0; half < BM / 128; ++half) {
    if (wave < NW && rowA0 / 128 == half) {
#pragma unroll
      for (int i = 0; i < NRB; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = rowA0 % 128 + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
            stile[row * LD + 32 * t + c] = acc[i][t][r];
          }
    }
    __syncthreads();
    if (m0 + 128 * half < M) tile_epilogue<T, EPI>(stile, LD, 128, m0 + 128 * half, M, nt, BN, cm, qo, ro, tid, NTH);
    __syncthreads();
  }
}

// Epilogue of a split-K GEMM: block (column tile of 128, 16 rows) sums the
// `splits` partial slices in slice order into an LDS tile (all of a thread's
// slice loads in flight at once), then runs the epilogue on it.
template <typename T, int EPI>
__global__ __launch_bounds__(256) void split_epilogue(const float* __restrict__ scratch, int splits, int M, int N,
                                                      ColMap cm, QkvOut qo, ResOut ro) {
  constexpr int BN = 128, RB = 16, LD = BN + 4;
  constexpr int PER = RB * (BN / 4) / 256;  // float4 units per thread
  __shared__ __attribute__((aligned(16))) float stile[RB * LD];
  const int nt = blockIdx.x, r0 = blockIdx.y * RB;
  const int rows = min(RB, M - r0);
  const float* tile = scratch + (size_t)r0 * N + nt * BN;
  const size_t slice = (size_t)256 * N;
  const int tid = threadIdx.x;
  // the epilogue's own loads (positions, slots, residual rows), then every
  // slice of both units, then the rotation rows: one memory latency for all
  EpiPre pre;
  epilogue_preload<T, EPI>(rows, r0, M, nt, BN, cm, qo, ro, tid, 256, &pre);
  // unconditional loads (slice and row clamped: slices past the count reload
  // the last one, rows past the tile its last row) keep the code branch-free
  float4 w[PER][kMaxSplits];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int e = tid + 256 * k, r = min(e / (BN / 4), rows - 1), q4 = e % (BN / 4);
#pragma unroll
    for (int y = 0; y < kMaxSplits; ++y)
      w[k][y] = *reinterpret_cast<const float4*>(tile + min(y, splits - 1) * slice + (size_t)r * N + 4 * q4);
  }
  epilogue_preload_rope<EPI>(nt, BN, cm, qo, tid, &pre);
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int e = tid + 256 * k, r = e / (BN / 4), q4 = e % (BN / 4);
    if (r < rows) {
      float4 v = w[k][0];
#pragma unroll
      for (int y = 1; y < kMaxSplits; ++y)
        if (y < splits) {
          v.x += w[k][y].x; v.y += w[k][y].y; v.z += w[k][y].z; v.w += w[k][y].w;
        }
      *reinterpret_cast<float4*>(&stile[r * LD + 4 * q4]) = v;
    }
  }
  __syncthreads();
  tile_epilogue<T, EPI, true>(stile, LD, rows, r0, M, nt, BN, cm, qo, ro, tid, 256, &pre);
}

}  // namespace dev

// --------------------------------------------------------------- launchers
using dev::bf16s;

// Tile and split choices (overridable for tuning sweeps; 0 = automatic).
GemmTuning g_gemm_tuning{};

namespace {

// K splits of a split-K GEMM with `tiles` column tiles: tiles x splits fill
// the CUs at most once, at most 6 (measured at 240 rows: more splits cost more
// in partial-slice traffic than the extra CUs bring), and every split keeps
// >= 2 K stages.
int split_count(int tiles, int K, int elt_bytes) {
  const int KT = K / (8 * (16 / elt_bytes));
  int S = g_gemm_tuning.splits > 0 ? g_gemm_tuning.splits : std::min(6, std::max(1, 256 / tiles));
  return std::max(1, std::min({S, kMaxSplits, KT / 2 > 0 ? KT / 2 : 1}));
}

template <typename T, int EPI>
hipError_t gemm_dispatch(const ModelDims& m, const GemmWs& ws, const void* A, int M, int K, int N,
                         const dev::ColMap& cm, const dev::QkvOut& qo, const dev::ResOut& ro, hipStream_t s) {
  const T* a = reinterpret_cast<const T*>(A);
  if (M <= kSplitRows && !ws.no_split) {
    // split K so that the column tiles times the splits fill the CUs once
    constexpr int BN = 128;
    if (N % BN) return hipErrorInvalidValue;
    const int tiles = N / BN;
    const int S = split_count(tiles, K, int(sizeof(T)));
    if ((size_t)S * 256 * N > ws.partial_elems) return hipErrorInvalidValue;
    if (M <= 64)
      JEV_LAUNCH((dev::gemm_kernel<T, BN, EPI, true, 1, 4, 64>), dim3(tiles, S), dim3(256), 0, s, a, M, K, N, cm,
                 qo, ro, ws.partial);
    else
      JEV_LAUNCH((dev::gemm_kernel<T, BN, EPI, true, 4, 2>), dim3(tiles, S), dim3(512), 0, s, a, M, K, N, cm,
                 qo, ro, ws.partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    JEV_LAUNCH((dev::split_epilogue<T, EPI>), dim3(tiles, (M + 15) / 16), dim3(256), 0, s, ws.partial, S, M,
                       N, cm, qo, ro);
    return hipGetLastError();
  }
  const int mt = (M + 255) / 256;
  if constexpr (sizeof(T) == 2) {
    // narrow products (the K/V projection alone): 256-row tiles would leave
    // most CUs idle; 128-row tiles, and 64 columns if that is still too few
    const int t128 = mt * (N / 128);
    if (N % 128 == 0 && t128 < 192 && K % 64 == 0 && g_gemm_tuning.large == 0) {
      const int mt2 = (M + 127) / 128;
      dim3 grid2;
      if (mt2 * (N / 128) >= 192 || N % 64) {
        grid2 = dim3(mt2 * (N / 128));
        JEV_LAUNCH((dev::gemm_pc_kernel<128, 128, EPI>), grid2, dim3(512), 0, s, a, M, K, N, cm, qo, ro);
      } else {
        grid2 = dim3(mt2 * (N / 64));
        JEV_LAUNCH((dev::gemm_pc_kernel<128, 64, EPI>), grid2, dim3(512), 0, s, a, M, K, N, cm, qo, ro);
      }
      return hipGetLastError();
    }
  }
  // tile width: 160 when it divides N and fills the CUs better than 128
  int bn = 128;
  if (N % 160 == 0) {
    const double t128 = double(mt) * (N / 128), t160 = double(mt) * (N / 160);
    const double e128 = t128 / (std::ceil(t128 / 256.0) * 256.0), e160 = t160 / (std::ceil(t160 / 256.0) * 256.0);
    if (e160 > e128 + 1e-9) bn = 160;
  }
  if (g_gemm_tuning.bn == 128 || g_gemm_tuning.bn == 160) bn = g_gemm_tuning.bn;
  if (N % bn) return hipErrorInvalidValue;
  dim3 grid((N / bn) * mt);
  if constexpr (sizeof(T) == 2) {
    // bf16, operands loaded straight into LDS: 4 (default) loader and MFMA
    // waves, 3 / 2 MFMA waves that load, three / two stages deep
    const int kind = g_gemm_tuning.large == 0 ? 4 : g_gemm_tuning.large;
    if (kind == 4 && K % 64 == 0) {
      if (bn == 160)
        JEV_LAUNCH((dev::gemm_pc_kernel<256, 160, EPI>), grid, dim3(512), 0, s, a, M, K, N, cm, qo, ro);
      else
        JEV_LAUNCH((dev::gemm_pc_kernel<256, 128, EPI>), grid, dim3(512), 0, s, a, M, K, N, cm, qo, ro);
      return hipGetLastError();
    }
    if (kind >= 2 && K % 64 == 0) {
      if (bn == 160 && kind == 2)
        JEV_LAUNCH((dev::gemm_dl_kernel<160, EPI, 2>), grid, dim3(256), 0, s, a, M, K, N, cm, qo, ro);
      else if (bn == 160)
        JEV_LAUNCH((dev::gemm_dl_kernel<160, EPI, 3>), grid, dim3(256), 0, s, a, M, K, N, cm, qo, ro);
      else if (kind == 2)
        JEV_LAUNCH((dev::gemm_dl_kernel<128, EPI, 2>), grid, dim3(256), 0, s, a, M, K, N, cm, qo, ro);
      else
        JEV_LAUNCH((dev::gemm_dl_kernel<128, EPI, 3>), grid, dim3(256), 0, s, a, M, K, N, cm, qo, ro);
      return hipGetLastError();
    }
  }
  // eight waves (two per SIMD): 8 x 1 over a 160-wide tile, 4 x 2 over 128
  if (bn == 160)
    JEV_LAUNCH((dev::gemm_kernel<T, 160, EPI, false, 8, 1>), grid, dim3(512), 0, s, a, M, K, N, cm, qo, ro,
                       nullptr);
  else
    JEV_LAUNCH((dev::gemm_kernel<T, 128, EPI, false, 4, 2>), grid, dim3(512), 0, s, a, M, K, N, cm, qo, ro,
                       nullptr);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qkv(const ModelDims& m, const LayerW& w, int32_t layer, const void* h, int32_t T_,
                      const int32_t* pos, const int32_t* kvslot, const float* rope, void* qbuf, void* pool,
                      const GemmWs& ws, hipStream_t s, bool kv_only) {
  if (T_ <= 0) return hipSuccess;
  // K/V only: the same column layout without the query heads (no q written)
  const int hq = kv_only ? 0 : m.hq;
  const int N = (hq + 2 * m.hkv) * m.dh;
  dev::ColMap cm{w.wq, w.wk, w.wv, hq, m.hkv, m.dh, (hq + m.hkv) * m.dh / 2};
  const size_t elt = m.dtype == 1 ? 2 : 4;
  dev::QkvOut qo{pos, kvslot, reinterpret_cast<const float2*>(rope), qbuf,
                 reinterpret_cast<char*>(pool) + (size_t)layer * m.n_pages * m.hkv * 2 * 16 * m.dh * elt,
                 m.hq, m.hkv, m.dh};
  dev::ResOut ro{nullptr, 0};
  if (m.dtype == 1) return gemm_dispatch<bf16s, dev::EPI_QKV>(m, ws, h, T_, m.d, N, cm, qo, ro, s);
  return gemm_dispatch<float, dev::EPI_QKV>(m, ws, h, T_, m.d, N, cm, qo, ro, s);
}

hipError_t launch_oproj_split(const ModelDims& m, const LayerW& w, const void* o, int32_t T_, const GemmWs& ws,
                              int32_t* splits, hipStream_t s) {
  if (T_ <= 0 || T_ > kSplitRows) return hipErrorInvalidValue;
  dev::ColMap cm{w.wo, nullptr, nullptr, 0, 0, m.dh, 0};
  const int K = m.hq * m.dh, N = m.d;
  constexpr int BN = 128;
  if (N % BN) return hipErrorInvalidValue;
  const int tiles = N / BN;
  const int S = split_count(tiles, K, m.dtype == 1 ? 2 : 4);
  if ((size_t)S * 256 * N > ws.partial_elems) return hipErrorInvalidValue;
  *splits = S;
  if (m.dtype == 1 && T_ <= 64)
    JEV_LAUNCH((dev::gemm_kernel<bf16s, BN, dev::EPI_RES, true, 1, 4, 64>), dim3(tiles, S), dim3(256), 0, s,
               reinterpret_cast<const bf16s*>(o), T_, K, N, cm, dev::QkvOut{}, dev::ResOut{}, ws.partial);
  else if (m.dtype == 1)
    JEV_LAUNCH((dev::gemm_kernel<bf16s, BN, dev::EPI_RES, true, 4, 2>), dim3(tiles, S), dim3(512), 0, s,
               reinterpret_cast<const bf16s*>(o), T_, K, N, cm, dev::QkvOut{}, dev::ResOut{}, ws.partial);
  else if (T_ <= 64)
    JEV_LAUNCH((dev::gemm_kernel<float, BN, dev::EPI_RES, true, 1, 4, 64>), dim3(tiles, S), dim3(256), 0, s,
               reinterpret_cast<const float*>(o), T_, K, N, cm, dev::QkvOut{}, dev::ResOut{}, ws.partial);
  else
    JEV_LAUNCH((dev::gemm_kernel<float, BN, dev::EPI_RES, true, 4, 2>), dim3(tiles, S), dim3(512), 0, s,
               reinterpret_cast<const float*>(o), T_, K, N, cm, dev::QkvOut{}, dev::ResOut{}, ws.partial);
  return hipGetLastError();
}

hipError_t launch_oproj(const ModelDims& m, const LayerW& w, const void* o, int32_t T_, void* x, const GemmWs& ws,
                        hipStream_t s, const int32_t* x_rows) {
  if (T_ <= 0) return hipSuccess;
  dev::ColMap cm{w.wo, nullptr, nullptr, 0, 0, m.dh, 0};
  dev::QkvOut qo{};
  dev::ResOut ro{x, m.d, x_rows};
  if (m.dtype == 1) return gemm_dispatch<bf16s, dev::EPI_RES>(m, ws, o, T_, m.hq * m.dh, m.d, cm, qo, ro, s);
  return gemm_dispatch<float, dev::EPI_RES>(m, ws, o, T_, m.hq * m.dh, m.d, cm, qo, ro, s);
}

}  // namespace jev
