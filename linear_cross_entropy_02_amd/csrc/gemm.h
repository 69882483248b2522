// MFMA tile engine for C = A * B^T with both operands K-contiguous
// ("NT": A is M x K row-major, B is N x K row-major), fp32 accumulation.
//
// All three contractions of the fused cross-entropy head run through this
// one engine (the caller lays every operand out K-contiguous first):
//   logits  Z  = X  * W^T      A = X   (C x H),   B = W   (V x H)
//   dX         = dZ * W        A = dZ  (C x V),   B = W^T (H x V)
//   dW        += dZ^T * X      A = dZ^T(V x C),   B = X^T (H x C)
//
// Block tile BM x BN, 4 waves in a 2 x 2 layout or 8 waves in a 2 x 4
// layout; each wave owns a (BM/2) x (BN/(WAVES/2)) accumulator tile made of
// 16 x 16 MFMA fragments.  One
// K-stage covers 128 bytes per row (64 bf16 or 32 fp32), staged through LDS
// with a double buffer; rows are stored as eight 16-byte vectors whose
// positions are XOR-swizzled by the row index so that both the direct-to-LDS
// writes and the fragment reads are free of bank conflicts.  (Full 128-byte
// row segments per load matter: a deeper ring of 64-byte stages in the same
// LDS was measured slower.)
//
// MFMA layouts used (16 x 16 output fragments):
//   bf16:  v_mfma_f32_16x16x32_bf16, lane l holds A[l%16][8 consecutive k]
//          and B[l%16][the same 8 k]; one 16-byte LDS read per operand.
//   fp32:  v_mfma_f32_16x16x4_f32 issued four times on the four floats of
//          one 16-byte read, element q of lane l pairing A and B on the same
//          k, so the four issues together contract 16 consecutive k.
//   D:     lane l, register r holds row 4*(l/16) + r, column l%16 of the
//          product of its first operand with the second; the engine passes
//          the B fragment first, so a fragment holds the C block transposed
//          (lane l: row l%16, columns 4*(l/16) .. +3).  Epilogues then store
//          16 (fp32) or 8 (bf16) contiguous bytes per lane and reduce a row
//          over four lanes instead of sixteen.
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
// bf16: in-place accumulate in one AGPR quad.  The tied operand keeps every
// accumulator in the same registers across the K-loop (the builtin lets the
// allocator rotate accumulators between iterations, which costs copies).
template <> __device__ __forceinline__ f4 mma16<bf16>(uint4 a, uint4 b, f4 c) {
#if defined(__HIP_DEVICE_COMPILE__)  // AMDGPU asm; the host pass only parses this
  typedef int i4v __attribute__((ext_vector_type(4)));
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
               : "+a"(c)
               : "v"(__builtin_bit_cast(i4v, a)), "v"(__builtin_bit_cast(i4v, b)));
#endif
  return c;
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

// Orders every accumulator after the preceding asm statements (the MFMA
// drain): each empty asm claims to modify one accumulator.
template <int FM, int FN>
__device__ __forceinline__ void drain_fence(f4 (&acc)[FM][FN]) {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) asm volatile("" : "+a"(acc[i][j]));
#endif
}

// WAVES = 4 (2 x 2 waves, one per SIMD) or 8 (2 x 4 waves, two per SIMD:
// while one wave waits to issue a load the other keeps the MFMA pipe busy).
template <int BM, int BN, int WAVES = 4>
struct TileGeom {
  static constexpr int kWaves = WAVES;
  static constexpr int kWavesN = WAVES / 2;
  static constexpr int kThreads = 64 * WAVES;
  static constexpr int WM = BM / 2, WN = BN / kWavesN;  // wave tile
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr int kStageVecs = (BM + BN) * 8;  // 16-byte vectors per stage
  static constexpr int kLdsBytes = 2 * kStageVecs * 16;
};

// Position of k-vector `kv` (0..7) of LDS row `row` within a stage.
__device__ __forceinline__ int swz(int row, int kv) { return row * 8 + (kv ^ (row & 7)); }

// What every epilogue receives: the wave's accumulator fragments and where
// they sit.  The MFMAs take the B fragment as their first operand, so each
// fragment holds a 16 x 16 block of C transposed: acc[i][j][r] is
// C[row0 + 16 i + lane%16][col0 + 16 j + 4 (lane/16) + r], i.e. a lane owns
// four consecutive columns of one row per fragment, and the four lanes
// lane%16 + {0, 16, 32, 48} together own 16 consecutive columns.
struct EpiCoord {
  int row0, col0;  // first row / column of this wave's tile
  int lane;
  int split;
};

// Accumulators starting at zero (the `init` of most epilogues).
template <int FM, int FN>
__device__ __forceinline__ void zero_init(f4 (&acc)[FM][FN]) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = (f4){0.f, 0.f, 0.f, 0.f};
}

// Buffer resource (4 SGPRs) for raw loads of `bytes` bytes from `base`: an
// offset at or beyond `bytes` reads zero, which supplies the M/N tails of a
// tile.  Word 3 selects 32-bit raw (untyped) access.
typedef int i4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i4v make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  return (i4v){(int)(uint32_t)a, (int)((a >> 32) & 0xffffu), (int)bytes, 0x00020000};
}
constexpr uint32_t kOobOffset = 0x80000000u;

// 16 bytes per lane from global memory straight into LDS at
// lds_addr + 16 * lane (buffer_load_dwordx4 ... lds; M0 holds the LDS base).
// Issued as asm so the compiler does not treat it as an LDS store it must
// wait on before unrelated LDS reads; callers wait on vmcnt before the
// barrier that publishes the stage.
__device__ __forceinline__ void dma16(i4v rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  // The LDS base, descriptor and scalar offset are wave-uniform: keep them
  // in SGPRs.  One wait state between the M0 write and the LDS DMA that
  // reads it.
  const i4v r = {__builtin_amdgcn_readfirstlane(rsrc[0]), __builtin_amdgcn_readfirstlane(rsrc[1]),
                 __builtin_amdgcn_readfirstlane(rsrc[2]), __builtin_amdgcn_readfirstlane(rsrc[3])};
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(r),
                 "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory");
#endif
}

// 16 bytes per lane from a buffer resource straight into an accumulator
// fragment.  Issued as asm, like dma16, so the compiler's wait-count model
// never sees it: it must be issued before the first stage's DMAs, whose
// vmcnt wait in the prologue then covers it too.
__device__ __forceinline__ void load16_acc(f4& dst, i4v rsrc, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  const i4v r = {__builtin_amdgcn_readfirstlane(rsrc[0]), __builtin_amdgcn_readfirstlane(rsrc[1]),
                 __builtin_amdgcn_readfirstlane(rsrc[2]), __builtin_amdgcn_readfirstlane(rsrc[3])};
  asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=a"(dst) : "v"(voff), "s"(r) : "memory");
#endif
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// K-loop schedule, one 128-byte K-stage per iteration, two LDS stages:
//   [A] substep-0 MFMAs on fragments already in registers, with the
//       substep-1 fragment reads of the same stage threaded through them;
//   barrier: this wave's reads of the stage are done and the next stage's
//       DMA has landed (vmcnt), in every wave;
//   [B] substep-1 MFMAs, with the DMA of the stage after next (into the
//       buffer just released) and the next stage's substep-0 fragment reads
//       threaded through them.
// The wave never waits on LDS after the barrier: the fragments its MFMAs
// need were read before it.
template <typename T, int BM, int BN, int WAVES, class Epi>
__global__ void __launch_bounds__(64 * WAVES) gemm_nt_kernel(GemmShape g, Epi epi) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass needs only the launch stub
  using G = TileGeom<BM, BN, WAVES>;
  constexpr int EPV = Elem<T>::kVec;
  constexpr int BK = 8 * EPV;
  constexpr int ES = (int)sizeof(T);
  constexpr int A_INS = BM / (8 * WAVES);  // 16-byte loads per lane per stage (A)
  constexpr int B_INS = BN / (8 * WAVES);
  constexpr int FM = G::FM, FN = G::FN;
  constexpr uint32_t kStageBytes = G::kStageVecs * 16;
  extern __shared__ uint4 lds[];  // 2 * kStageVecs, sized at launch

  const TileCoord tc = map_tile(g);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / G::kWavesN, wn = wave % G::kWavesN;
  const int m0 = tc.tm * BM, n0 = tc.tn * BN;

  int k_begin = 0, k_end = g.K;
  if (g.splits > 1) {
    k_begin = tc.split * g.k_per_split;
    k_end = min(g.K, k_begin + g.k_per_split);
  }
  const int nk = (k_end - k_begin + BK - 1) / BK;

  const int a_rows = min(BM, g.M - m0), b_rows = min(BN, g.N - n0);
  const i4v rA =
      make_rsrc((const T*)g.A + (int64_t)m0 * g.lda, (uint32_t)((int64_t)a_rows * g.lda * ES));
  const i4v rB =
      make_rsrc((const T*)g.B + (int64_t)n0 * g.ldb, (uint32_t)((int64_t)b_rows * g.ldb * ES));

  // Direct-to-LDS loads write lane i of a wave's load to the LDS slot
  // base + 16 i.  Slot p of a stage holds row p / 8 and logical k-vector
  // (p % 8) ^ (row % 8), i.e. the XOR-swizzled layout read by swz().  Every
  // load of a wave covers 8 whole rows, so the k-vector of a lane is the
  // same in all of its loads.
  uint32_t a_off[A_INS], b_off[B_INS];
  const int kv_lane = (lane & 7) ^ ((lane >> 3) & 7);
#pragma unroll
  for (int j = 0; j < A_INS; ++j) {
    const int row = wave * (BM / WAVES) + 8 * j + (lane >> 3);
    a_off[j] = (uint32_t)(((int64_t)row * g.lda + kv_lane * EPV) * ES);
  }
#pragma unroll
  for (int j = 0; j < B_INS; ++j) {
    const int row = wave * (BN / WAVES) + 8 * j + (lane >> 3);
    b_off[j] = (uint32_t)(((int64_t)row * g.ldb + kv_lane * EPV) * ES);
  }
  const uint32_t lds_base = (uint32_t)(size_t)((lds_ptr_t)lds);
  const uint32_t lds_a = lds_base + wave * (BM * 8 / WAVES) * 16;
  const uint32_t lds_b = lds_base + BM * 8 * 16 + wave * (BN * 8 / WAVES) * 16;

  EpiCoord ec;
  ec.row0 = m0 + wm * G::WM;
  ec.col0 = n0 + wn * G::WN;
  ec.lane = lane;
  ec.split = tc.split;

  // The epilogue chooses the starting accumulators: zero, or (to accumulate
  // into an existing output) its old values, loaded with load16_acc here,
  // before any DMA, so that the prologue's wait for stage 0 covers them.
  f4 acc[FM][FN];
  epi.template init<FM, FN>(acc, ec);

  // DMA j of stage `st` (0/1) for K-offset k0: j < A_INS loads A, else B.
  // Past the end of K every offset is out of range and the stage fills
  // with zeros.
  auto issue_one = [&](int st, int k0, int j) {
    const bool kin = kv_lane * EPV < k_end - k0;
    const uint32_t so = (uint32_t)st * kStageBytes;
    if (j < A_INS)
      dma16(rA, lds_a + so + 1024 * j, kin ? a_off[j] : kOobOffset, k0 * ES);
    else
      dma16(rB, lds_b + so + 1024 * (j - A_INS), kin ? b_off[j - A_INS] : kOobOffset, k0 * ES);
  };
  // Fragment read r of substep s of stage st: r < FM reads A fragment r,
  // else B fragment r - FM.
  auto read_one = [&](int st, int s, int r, uint4 (&fa)[FM], uint4 (&fb)[FN]) {
    const uint4* stage = lds + st * G::kStageVecs;
    const int kv = 4 * s + (lane >> 4);
    if (r < FM)
      fa[r] = stage[swz(wm * G::WM + 16 * r + (lane & 15), kv)];
    else
      fb[r - FM] = stage[BM * 8 + swz(wn * G::WN + 16 * (r - FM) + (lane & 15), kv)];
  };

  constexpr int NR = FM + FN;  // fragment reads per substep
  constexpr int NM = FM * FN;  // MFMAs per substep
  constexpr int NDMA = A_INS + B_INS;
  constexpr int SPA = NM / NR > 0 ? NM / NR : 1;                    // [A]: reads
  constexpr int SPB = NM / (NR + NDMA) > 0 ? NM / (NR + NDMA) : 1;  // [B]: DMA + reads
  static_assert(NR * SPA <= NM && (NR + NDMA) * SPB <= NM, "side operations must fit");
  static_assert(NDMA < 64, "vmcnt field");
  // s_waitcnt vmcnt(NDMA), expcnt/lgkmcnt not waited on
  constexpr int kWaitStage0 = (NDMA & 0xF) | ((NDMA >> 4) << 14) | 0x0F70;

  uint4 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
  if (nk > 0) {
#pragma unroll
    for (int j = 0; j < NDMA; ++j) issue_one(0, k_begin, j);
#pragma unroll
    for (int j = 0; j < NDMA; ++j) issue_one(1, k_begin + BK, j);
    __builtin_amdgcn_s_waitcnt(kWaitStage0);  // initial accumulators and stage 0 landed
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int r = 0; r < NR; ++r) read_one(0, 0, r, fa0, fb0);
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1, nxt = cur ^ 1;
      // [A]
#pragma unroll
      for (int q = 0; q < NM; ++q) {
        acc[q / FN][q % FN] = mma16<T>(fb0[q % FN], fa0[q / FN], acc[q / FN][q % FN]);
        if (q % SPA == SPA - 1 && q / SPA < NR) read_one(cur, 1, q / SPA, fa1, fb1);
      }
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
      // [B]
      const int k2 = k_begin + (kt + 2) * BK;  // past the end: zero fill, unused
#pragma unroll
      for (int q = 0; q < NM; ++q) {
        acc[q / FN][q % FN] = mma16<T>(fb1[q % FN], fa1[q / FN], acc[q / FN][q % FN]);
        // DMAs alternate with the fragment reads (bursts of DMA issue from
        // all waves at once stall on the address unit); reads go B
        // fragments first: [A] consumes all B fragments in its first FN
        // MFMAs but A fragment i only from MFMA i * FN on.
        if (q % SPB == SPB - 1 && q / SPB < NR + NDMA) {
          const int k = q / SPB;
          if ((k & 1) == 0 && k / 2 < NDMA)
            issue_one(cur, k2, k / 2);
          else
            read_one(nxt, 0, ((k - min(k / 2 + 1, NDMA)) + FM) % NR, fa0, fb0);
        }
      }
    }
  }
  // The last (unused) DMAs may still be in flight; results of the asm MFMAs
  // are read by ordinary code next, so let the last ones drain (the hazard
  // recognizer does not see inside asm), and tie every accumulator to an
  // empty asm after the drain so no read of it can be scheduled earlier.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  drain_fence(acc);
  epi.template apply<FM, FN>(acc, ec);
#endif
}

}  // namespace flce
