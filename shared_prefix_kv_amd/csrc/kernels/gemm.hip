// Projection GEMMs of the scoring path on gfx950 MFMA (fp32 accumulation).
//
//   C[M, N] = A[M, K] . B[N, K]^T   (A = activations, B rows = weight rows)
//
// Two shapes occur.  Prefix prefill: M = prefix tokens (thousands), compute
// bound.  Branch scoring: M = suffix tokens of all branches (a few hundred),
// bound by streaming the weights once.
//
// One kernel, gemm_v3 (below): 256-row x BN-column tiles, 4 waves of 64 rows;
// BN = 160 where it makes the tile count fit the 256 CUs (QKV at 2,000 rows:
// 8 x 32 tiles), else 128.  Up to 256 rows (branch scoring) it splits K over
// ~4 workgroups per column tile so that the weights stream from every CU.
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
};

enum { EPI_QKV = 0, EPI_RES = 1 };

// Writes one rotate-half pair (or one V element) of row m.
template <typename T>
__device__ __forceinline__ void qkv_store_pair(const QkvOut& qo, const ColMap& cm, int m, int pair, float a0,
                                               float a1) {
  const int h2 = qo.dh >> 1;
  const int head = pair / h2, i = pair % h2;
  const float2 cs = qo.rope[(size_t)qo.pos[m] * h2 + i];
  const float o0 = a0 * cs.x - a1 * cs.y;
  const float o1 = a1 * cs.x + a0 * cs.y;
  if (head < cm.hq) {
    T* q = reinterpret_cast<T*>(qo.qbuf) + ((size_t)m * qo.hq + head) * qo.dh;
    q[i] = from_f32<T>(o0);
    q[i + h2] = from_f32<T>(o1);
  } else {
    const int sl = qo.kvslot[m];
    const size_t pe = (size_t)16 * qo.dh;
    T* kb = reinterpret_cast<T*>(qo.pool) + ((size_t)(sl >> 4) * qo.hkv + (head - cm.hq)) * 2 * pe +
            (size_t)(sl & 15) * qo.dh;
    kb[i] = from_f32<T>(o0);
    kb[i + h2] = from_f32<T>(o1);
  }
}

template <typename T>
__device__ __forceinline__ void qkv_store_v(const QkvOut& qo, int m, int vcol, float a) {
  const int sl = qo.kvslot[m];
  const size_t pe = (size_t)16 * qo.dh;
  const int head = vcol / qo.dh, f = vcol % qo.dh;
  T* vb = reinterpret_cast<T*>(qo.pool) + ((size_t)(sl >> 4) * qo.hkv + head) * 2 * pe + pe;
  vb[(size_t)f * 16 + (sl & 15)] = from_f32<T>(a);
}

// Two adjacent stored elements (address aligned to their pair).
template <typename T>
__device__ __forceinline__ void store_pair(T* dst, float x, float y);
template <>
__device__ __forceinline__ void store_pair<bf16s>(bf16s* dst, float x, float y) {
  *reinterpret_cast<uint32_t*>(dst) = uint32_t(from_f32<bf16s>(x).bits) | (uint32_t(from_f32<bf16s>(y).bits) << 16);
}
template <>
__device__ __forceinline__ void store_pair<float>(float* dst, float x, float y) {
  *reinterpret_cast<float2*>(dst) = make_float2(x, y);
}

// Epilogue over an fp32 tile: rows [0, rows) of tile_row0.., columns [0, BN) of
// column tile nt; element (r, j) at tile[r * ld + j].
template <typename T, int EPI>
__device__ __forceinline__ void tile_epilogue(const float* tile, int ld, int rows, int m0, int M, int nt, int BN,
                                              const ColMap& cm, const QkvOut& qo, const ResOut& ro, int tid,
                                              int nthreads) {
  if constexpr (EPI == EPI_RES) {
    constexpr int CH = 16 / sizeof(T);
    const int cpr = BN / CH;  // 16-byte chunks per row
    for (int e = tid; e < rows * cpr; e += nthreads) {
      const int r = e / cpr, c = (e % cpr) * CH;
      const int m = m0 + r;
      if (m >= M) continue;
      T* xp = reinterpret_cast<T*>(ro.x) + (size_t)m * ro.ld + (size_t)nt * BN + c;
      float xv[CH];
#pragma unroll
      for (int i = 0; i < CH; ++i) xv[i] = to_f32(xp[i]) + tile[r * ld + c + i];
#pragma unroll
      for (int i = 0; i < CH; ++i) xp[i] = from_f32<T>(xv[i]);
    }
  } else {
    // QKV: per-row (position, KV slot) and per-column (kind, pair or V
    // column) data are staged in LDS once per tile; the element loop is
    // unrolled so that the RoPE table loads of 8 elements are in flight
    // together.
    __shared__ int s_pos[256], s_slot[256], s_col[256];
    const int32_t* __restrict__ pos = qo.pos;
    const int32_t* __restrict__ kvslot = qo.kvslot;
    const float2* __restrict__ rope = qo.rope;
    T* __restrict__ qbuf = reinterpret_cast<T*>(qo.qbuf);
    T* __restrict__ pool = reinterpret_cast<T*>(qo.pool);
    const int h2 = cm.dh >> 1;
    const int np_t = max(0, min(BN >> 1, cm.n_pairs - (BN >> 1) * nt));
    for (int r = tid; r < rows; r += nthreads) {
      const int m = min(m0 + r, M - 1);
      s_pos[r] = pos[m];
      s_slot[r] = kvslot[m];
    }
    for (int j = tid; j < BN; j += nthreads) {
      const ColInfo ci = qkv_col(cm, BN, nt, j);
      // bits 0-1 kind, 2-13 head, 14-27 index within the head (pair index i
      // for q/k, feature f for v)
      int head, idx;
      if (ci.kind == COL_V) {
        head = ci.vcol / qo.dh;
        idx = ci.vcol % qo.dh;
      } else {
        head = ci.pair / h2;
        idx = ci.pair % h2;
      }
      s_col[j] = ci.kind | (head << 2) | (idx << 14);
    }
    __syncthreads();
    const size_t pe = (size_t)16 * qo.dh;
    const int valid_rows = min(rows, M - m0);
    // active columns: the np_t pair heads, then the V columns (partners are
    // handled with their pair)
    const int n_act = BN - np_t;
    const int total = valid_rows * n_act;
#pragma unroll 8
    for (int e = tid; e < total; e += nthreads) {
      const int r = e / n_act, a = e - (e / n_act) * n_act;
      const int j = a < np_t ? a : a + np_t;
      const int cc = s_col[j];
      const int kind = cc & 3, head = (cc >> 2) & 4095, idx = cc >> 14;
      const int m = m0 + r;
      if (kind == COL_FIRST) {
        const float2 cs = rope[(size_t)s_pos[r] * h2 + idx];
        const float a0 = tile[r * ld + j], a1 = tile[r * ld + j + np_t];
        // q and k store each rotate-half pair (i, i + dh/2) adjacently, at
        // 2i and 2i+1: both sides of every q.k product use the same order
        T* dst;
        if (head < cm.hq) {
          dst = qbuf + ((size_t)m * qo.hq + head) * qo.dh + 2 * idx;
        } else {
          const int sl = s_slot[r];
          dst = pool + ((size_t)(sl >> 4) * qo.hkv + (head - cm.hq)) * 2 * pe + (size_t)(sl & 15) * qo.dh + 2 * idx;
        }
        store_pair<T>(dst, a0 * cs.x - a1 * cs.y, a1 * cs.x + a0 * cs.y);
      } else if (kind == COL_V) {
        const int sl = s_slot[r];
        pool[((size_t)(sl >> 4) * qo.hkv + head) * 2 * pe + pe + (size_t)idx * 16 + (sl & 15)] =
            from_f32<T>(tile[r * ld + j]);
      }
    }
    __syncthreads();
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
// Block = 4 waves; wave w owns rows [64w, 64w+64) of a 256-row tile and all BN
// columns.  A rows are private to a wave, so A fragments go straight from
// global memory into MFMA-layout registers (one stage ahead); B rows are shared
// by the 4 waves and go through LDS (rows padded to 144 bytes so the 16 rows of
// one 16-lane fragment read fall in 16 different bank groups), register-staged
// two stages ahead.  With SPLIT, blockIdx.y selects a slice of K and partial sums
// are added (agent-scope fp32 atomics) into an fp32 [M][N] scratch tile;
// split_epilogue (next launch) runs the epilogue on the sums over all CUs and
// clears the scratch for the next use.
template <typename T, int BN, int EPI, bool SPLIT>
__global__ __launch_bounds__(256) void gemm_v3(const T* __restrict__ A, int M, int K, int N, ColMap cm, QkvOut qo,
                                               ResOut ro, float* __restrict__ scratch) {
  using MF = Mfma<T>;
  using frag = typename MF::frag;
  constexpr int BM = 256;
  constexpr int CH = 16 / sizeof(T);   // elements per 16-byte chunk
  constexpr int BK = 8 * CH;           // 128 bytes of K per stage
  constexpr int KS = BK / MF::KSTEP;   // MFMA k-steps per stage
  constexpr int TN = BN / 32;
  constexpr int LB = BN * 8 / 256;     // B chunks per thread per stage
  constexpr int LDS_B = 2 * BN * 9;                 // in 16-byte units
  constexpr int LDS_EPI = SPLIT ? 0 : 128 * (BN + 4) / 4;
  constexpr int LDS_UNITS = LDS_B > LDS_EPI ? LDS_B : LDS_EPI;
  static_assert((BN * 8) % 256 == 0, "tile");
  __shared__ __attribute__((aligned(16))) u32x4 smem[LDS_UNITS];
  u32x4* sB[2] = {smem, smem + BN * 9};

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_tiles_n = N / BN;
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

  const T* ap[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    ap[i] = A + (size_t)min(m0 + wave * 64 + 32 * i + (lane & 31), M - 1) * K + MF::KL * (lane >> 5) + (size_t)kt0 * BK;
  const u32x4* bp[LB];
#pragma unroll
  for (int i = 0; i < LB; ++i)
    bp[i] = reinterpret_cast<const u32x4*>(weight_row<T>(cm, BN, n0 + lrow + 32 * i, K) + (size_t)kt0 * BK) + lch;
  (void)n_tiles_n;

  f32x16 acc[2][TN];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  frag a0[2][KS], a1[2][KS];
  u32x4 rb0[LB], rb1[LB];
#define V3_ALOAD(AA, KT_)                                                              \
  do {                                                                                 \
    const int kk_ = min((KT_), KT - 1) * BK;                                           \
    _Pragma("unroll") for (int i = 0; i < 2; ++i) _Pragma("unroll") for (int s = 0; s < KS; ++s) \
        AA[i][s] = MF::load(ap[i] + kk_ + s * MF::KSTEP);                              \
  } while (0)
#define V3_BLOAD(RB, KT_)                                                              \
  do {                                                                                 \
    const int kk_ = min((KT_), KT - 1) * 8;                                            \
    _Pragma("unroll") for (int i = 0; i < LB; ++i) RB[i] = bp[i][kk_];                 \
  } while (0)
#define V3_BSTORE(RB, BUF)                                                             \
  do {                                                                                 \
    _Pragma("unroll") for (int i = 0; i < LB; ++i) sB[BUF][(lrow + 32 * i) * 9 + lch] = RB[i]; \
  } while (0)
#define V3_COMPUTE(AA, BUF)                                                                          \
  do {                                                                                               \
    _Pragma("unroll") for (int s = 0; s < KS; ++s) {                                                 \
      const int k_ = s * MF::KSTEP + MF::KL * (lane >> 5);                                           \
      frag b_[TN];                                                                                   \
      _Pragma("unroll") for (int j = 0; j < TN; ++j) b_[j] =                                         \
          MF::load(reinterpret_cast<const T*>(&sB[BUF][(32 * j + (lane & 31)) * 9 + k_ / CH]) + k_ % CH); \
      _Pragma("unroll") for (int i = 0; i < 2; ++i) _Pragma("unroll") for (int j = 0; j < TN; ++j) acc[i][j] = \
          MF::mma(AA[i][s], b_[j], acc[i][j]);                                                       \
    }                                                                                                \
  } while (0)

  V3_ALOAD(a0, 0);
  V3_BLOAD(rb0, 0);
  V3_BLOAD(rb1, 1);
  V3_BSTORE(rb0, 0);
  __syncthreads();
  int kt = 0;
  // two stages per trip keep the register sets static; scheduling barriers keep
  // the prefetch loads ahead of the MFMA block
  for (; kt + 1 < KT; kt += 2) {
    V3_ALOAD(a1, kt + 1);
    V3_BLOAD(rb0, kt + 2);
    __builtin_amdgcn_sched_barrier(0);
    V3_COMPUTE(a0, 0);
    __builtin_amdgcn_sched_barrier(0);
    V3_BSTORE(rb1, 1);
    __syncthreads();
    V3_ALOAD(a0, kt + 2);
    V3_BLOAD(rb1, kt + 3);
    __builtin_amdgcn_sched_barrier(0);
    V3_COMPUTE(a1, 1);
    __builtin_amdgcn_sched_barrier(0);
    V3_BSTORE(rb0, 0);
    __syncthreads();
  }
  if (kt < KT) V3_COMPUTE(a0, 0);
#undef V3_ALOAD
#undef V3_BLOAD
#undef V3_BSTORE
#undef V3_COMPUTE

  const int c = lane & 31, hh = lane >> 5;
  if constexpr (SPLIT) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = wave * 64 + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (m < M)
            __hip_atomic_fetch_add(scratch + (size_t)m * N + n0 + 32 * j + c, acc[i][j][r], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
  } else {
    float* stile = reinterpret_cast<float*>(smem);
    constexpr int LD = BN + 4;
    __syncthreads();
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if ((wave >> 1) == half) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = (wave & 1) * 64 + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
              stile[row * LD + 32 * j + c] = acc[i][j][r];
            }
      }
      __syncthreads();
      tile_epilogue<T, EPI>(stile, LD, 128, m0 + 128 * half, M, nt, BN, cm, qo, ro, tid, 256);
      __syncthreads();
    }
  }
}

// Epilogue of a split-K GEMM: block (column tile of 128, 16 rows).
template <typename T, int EPI>
__global__ __launch_bounds__(256) void split_epilogue(float* __restrict__ scratch, int M, int N, ColMap cm, QkvOut qo,
                                                      ResOut ro) {
  constexpr int BN = 128, RB = 16;
  const int nt = blockIdx.x, r0 = blockIdx.y * RB;
  const int rows = min(RB, M - r0);
  float* tile = scratch + (size_t)r0 * N + nt * BN;
  tile_epilogue<T, EPI>(tile, N, rows, r0, M, nt, BN, cm, qo, ro, threadIdx.x, 256);
  __syncthreads();
  for (int e = threadIdx.x; e < rows * (BN / 4); e += 256) {
    const int r = e / (BN / 4), q4 = e % (BN / 4);
    *reinterpret_cast<float4*>(tile + (size_t)r * N + 4 * q4) = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

}  // namespace dev

// --------------------------------------------------------------- launchers
using dev::bf16s;

// Tile and split choices (overridable for tuning sweeps; 0 = automatic).
GemmTuning g_gemm_tuning{};

namespace {

template <typename T, int EPI>
hipError_t gemm_dispatch(const ModelDims& m, const GemmWs& ws, const void* A, int M, int K, int N,
                         const dev::ColMap& cm, const dev::QkvOut& qo, const dev::ResOut& ro, hipStream_t s) {
  const T* a = reinterpret_cast<const T*>(A);
  if (M <= 256) {
    // split-K over ~4 workgroups per 128-column tile
    constexpr int BN = 128;
    if (N % BN) return hipErrorInvalidValue;
    const int tiles = N / BN;
    const int KT = K / (8 * (16 / int(sizeof(T))));
    int S = g_gemm_tuning.splits > 0 ? g_gemm_tuning.splits : std::max(1, 512 / tiles);
    S = std::max(1, std::min({S, 8, KT / 2 > 0 ? KT / 2 : 1}));
    if ((size_t)256 * N > ws.partial_elems) return hipErrorInvalidValue;
    hipLaunchKernelGGL((dev::gemm_v3<T, BN, EPI, true>), dim3(tiles, S), dim3(256), 0, s, a, M, K, N, cm, qo, ro,
                       ws.partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dev::split_epilogue<T, EPI>), dim3(tiles, (M + 15) / 16), dim3(256), 0, s, ws.partial, M, N,
                       cm, qo, ro);
    return hipGetLastError();
  }
  const int mt = (M + 255) / 256;
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
  if (bn == 160)
    hipLaunchKernelGGL((dev::gemm_v3<T, 160, EPI, false>), grid, dim3(256), 0, s, a, M, K, N, cm, qo, ro, nullptr);
  else
    hipLaunchKernelGGL((dev::gemm_v3<T, 128, EPI, false>), grid, dim3(256), 0, s, a, M, K, N, cm, qo, ro, nullptr);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qkv(const ModelDims& m, const LayerW& w, int32_t layer, const void* h, int32_t T_,
                      const int32_t* pos, const int32_t* kvslot, const float* rope, void* qbuf, void* pool,
                      const GemmWs& ws, hipStream_t s) {
  if (T_ <= 0) return hipSuccess;
  const int N = (m.hq + 2 * m.hkv) * m.dh;
  dev::ColMap cm{w.wq, w.wk, w.wv, m.hq, m.hkv, m.dh, (m.hq + m.hkv) * m.dh / 2};
  const size_t elt = m.dtype == 1 ? 2 : 4;
  dev::QkvOut qo{pos, kvslot, reinterpret_cast<const float2*>(rope), qbuf,
                 reinterpret_cast<char*>(pool) + (size_t)layer * m.n_pages * m.hkv * 2 * 16 * m.dh * elt,
                 m.hq, m.hkv, m.dh};
  dev::ResOut ro{nullptr, 0};
  if (m.dtype == 1) return gemm_dispatch<bf16s, dev::EPI_QKV>(m, ws, h, T_, m.d, N, cm, qo, ro, s);
  return gemm_dispatch<float, dev::EPI_QKV>(m, ws, h, T_, m.d, N, cm, qo, ro, s);
}

hipError_t launch_oproj(const ModelDims& m, const LayerW& w, const void* o, int32_t T_, void* x, const GemmWs& ws,
                        hipStream_t s) {
  if (T_ <= 0) return hipSuccess;
  dev::ColMap cm{w.wo, nullptr, nullptr, 0, 0, m.dh, 0};
  dev::QkvOut qo{};
  dev::ResOut ro{x, m.d};
  if (m.dtype == 1) return gemm_dispatch<bf16s, dev::EPI_RES>(m, ws, o, T_, m.hq * m.dh, m.d, cm, qo, ro, s);
  return gemm_dispatch<float, dev::EPI_RES>(m, ws, o, T_, m.hq * m.dh, m.d, cm, qo, ro, s);
}

}  // namespace jev
