// MFMA tile engine for C = A * B^T with both operands K-contiguous
// ("NT": A is M x K row-major, B is N x K row-major), fp32 accumulation.
//
// All three contractions of the fused cross-entropy head run through this
// one engine (the caller lays every operand out K-contiguous first):
//   logits  Z  = X  * W^T      A = X   (C x H),   B = W   (V x H)
//   dX         = dZ * W        A = dZ  (C x V),   B = W^T (H x V)
//   dW        += dZ^T * X      A = dZ^T(V x C),   B = X^T (H x C)
//
// Block tile BM x BN, 256 threads = 4 waves in a 2 x 2 layout, each wave owns
// a (BM/2) x (BN/2) accumulator tile made of 16 x 16 MFMA fragments.  One
// K-stage covers 128 bytes per row (64 bf16 or 32 fp32), staged through LDS
// with a double buffer; rows are stored as eight 16-byte vectors whose
// positions are XOR-swizzled by the row index so that both the row-wise
// stores and the fragment reads are free of bank conflicts.
//
// MFMA layouts used (16 x 16 output fragments):
//   bf16:  v_mfma_f32_16x16x32_bf16, lane l holds A[l%16][8 consecutive k]
//          and B[l%16][the same 8 k]; one 16-byte LDS read per operand.
//   fp32:  v_mfma_f32_16x16x4_f32 issued four times on the four floats of
//          one 16-byte read, element q of lane l pairing A and B on the same
//          k, so the four issues together contract 16 consecutive k.
//   D:     lane l, register r holds row 4*(l/16) + r, column l%16.
// Grid order is XCD-aware: consecutive logical tiles land on one XCD (its
// own L2), walking M fastest inside groups of `group_m` rows of tiles so
// that blocks sharing a B tile run together.
#pragma once

#include "common.h"

namespace flce {

struct GemmShape {
  const void* A;
  const void* B;
  int64_t lda, ldb;  // leading dimensions in elements
  int M, N, K;       // K % Elem<T>::kVec == 0
  int tiles_m, tiles_n;
  int splits;        // split-K factor (1 = none)
  int k_per_split;   // multiple of the stage depth, unused when splits == 1
  int group_m;       // rows of tiles walked together (>= 1)
};

struct TileCoord {
  int tm, tn, split;
};

// Block id -> tile.  Hardware dispatches consecutive block ids to the 8 XCDs
// round-robin; give each XCD a contiguous range of logical tiles.
__device__ __forceinline__ TileCoord map_tile(const GemmShape& g) {
  const int nblk = (int)gridDim.x;
  const int bid = (int)blockIdx.x;
  const int q = nblk >> 3, r = nblk & 7;
  const int xcd = bid & 7, slot = bid >> 3;
  const int logical = xcd * q + min(xcd, r) + slot;
  const int per_split = g.tiles_m * g.tiles_n;
  TileCoord c;
  c.split = logical / per_split;
  const int tile = logical - c.split * per_split;
  const int per_group = g.group_m * g.tiles_n;
  const int gid = tile / per_group;
  const int first_m = gid * g.group_m;
  const int gsize = min(g.tiles_m - first_m, g.group_m);
  const int in_group = tile - gid * per_group;
  c.tm = first_m + in_group % gsize;
  c.tn = in_group / gsize;
  return c;
}

template <typename T> __device__ __forceinline__ f4 mma16(uint4 a, uint4 b, f4 c);
template <> __device__ __forceinline__ f4 mma16<bf16>(uint4 a, uint4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f4 mma16<float>(uint4 a, uint4 b, f4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, a.x),
                                           __builtin_bit_cast(float, b.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, a.y),
                                           __builtin_bit_cast(float, b.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, a.z),
                                           __builtin_bit_cast(float, b.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, a.w),
                                           __builtin_bit_cast(float, b.w), c, 0, 0, 0);
  return c;
}

template <int BM, int BN>
struct TileGeom {
  static constexpr int kThreads = 256;
  static constexpr int WM = BM / 2, WN = BN / 2;  // wave tile
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr int kAVec = BM * 8 / kThreads;  // 16-B vectors per thread per stage
  static constexpr int kBVec = BN * 8 / kThreads;
  static constexpr int kStageVecs = (BM + BN) * 8;
  static constexpr int kLdsBytes = 2 * kStageVecs * 16;
};

// Position of vector `kv` (0..7) of LDS row `row`.
__device__ __forceinline__ int swz(int row, int kv) { return row * 8 + (kv ^ (row & 7)); }

// What every epilogue receives: the wave's accumulator fragments and where
// they sit.  acc[i][j][r] is C[row0 + 16 i + 4 (lane/16) + r][col0 + 16 j + lane%16].
struct EpiCoord {
  int row0, col0;  // first row / column of this wave's tile
  int lane;
  int split;
};

template <typename T, int BM, int BN, class Epi>
__global__ void __launch_bounds__(256) gemm_nt_kernel(GemmShape g, Epi epi) {
  using G = TileGeom<BM, BN>;
  constexpr int EPV = Elem<T>::kVec;
  constexpr int BK = 8 * EPV;
  extern __shared__ uint4 smem[];

  const TileCoord tc = map_tile(g);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = tc.tm * BM, n0 = tc.tn * BN;

  int k_begin = 0, k_end = g.K;
  if (g.splits > 1) {
    k_begin = tc.split * g.k_per_split;
    k_end = min(g.K, k_begin + g.k_per_split);
  }
  const int nk = (k_end - k_begin + BK - 1) / BK;

  const T* __restrict__ Ablk = (const T*)g.A + (int64_t)m0 * g.lda;
  const T* __restrict__ Bblk = (const T*)g.B + (int64_t)n0 * g.ldb;
  const int lrow = tid >> 3, lkv = tid & 7;
  const int a_rows = min(BM, g.M - m0), b_rows = min(BN, g.N - n0);

  f4 acc[G::FM][G::FN];
#pragma unroll
  for (int i = 0; i < G::FM; ++i)
#pragma unroll
    for (int j = 0; j < G::FN; ++j) acc[i][j] = (f4){0.f, 0.f, 0.f, 0.f};

  uint4 ra[G::kAVec], rb[G::kBVec];
  const uint4 zero4 = {0u, 0u, 0u, 0u};

  auto gload = [&](int k0) {
    const int k = k0 + lkv * EPV;
    const bool kok = k < k_end;
#pragma unroll
    for (int i = 0; i < G::kAVec; ++i) {
      const int r = lrow + 32 * i;
      ra[i] = (kok && r < a_rows) ? *(const uint4*)(Ablk + (int64_t)r * g.lda + k) : zero4;
    }
#pragma unroll
    for (int i = 0; i < G::kBVec; ++i) {
      const int r = lrow + 32 * i;
      rb[i] = (kok && r < b_rows) ? *(const uint4*)(Bblk + (int64_t)r * g.ldb + k) : zero4;
    }
  };
  auto sstore = [&](int stage) {
    uint4* sa = smem + stage * G::kStageVecs;
    uint4* sb = sa + BM * 8;
#pragma unroll
    for (int i = 0; i < G::kAVec; ++i) sa[swz(lrow + 32 * i, lkv)] = ra[i];
#pragma unroll
    for (int i = 0; i < G::kBVec; ++i) sb[swz(lrow + 32 * i, lkv)] = rb[i];
  };
  auto compute = [&](int stage) {
    const uint4* sa = smem + stage * G::kStageVecs;
    const uint4* sb = sa + BM * 8;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int kv = 4 * s + (lane >> 4);
      uint4 af[G::FM], bfr[G::FN];
#pragma unroll
      for (int i = 0; i < G::FM; ++i) af[i] = sa[swz(wm * G::WM + 16 * i + (lane & 15), kv)];
#pragma unroll
      for (int j = 0; j < G::FN; ++j) bfr[j] = sb[swz(wn * G::WN + 16 * j + (lane & 15), kv)];
#pragma unroll
      for (int i = 0; i < G::FM; ++i)
#pragma unroll
        for (int j = 0; j < G::FN; ++j) acc[i][j] = mma16<T>(af[i], bfr[j], acc[i][j]);
    }
  };

  if (nk > 0) {
    gload(k_begin);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const bool more = kt + 1 < nk;
      if (more) gload(k_begin + (kt + 1) * BK);
      compute(kt & 1);
      if (more) sstore((kt + 1) & 1);
      __syncthreads();
    }
  }

  EpiCoord ec;
  ec.row0 = m0 + wm * G::WM;
  ec.col0 = n0 + wn * G::WN;
  ec.lane = lane;
  ec.split = tc.split;
  epi.template apply<G::FM, G::FN>(acc, ec);
}

}  // namespace flce
