// MFMA tile engine for C = A * B^T with both operands K-contiguous
// ("NT": A is M x K row-major, B is N x K row-major), fp32 accumulation.
//
// All three contractions of the fused cross-entropy head run through this
// one engine (operands K-contiguous, or read as stored in the BT / AT modes
// below):
//   logits  Z  = X  * W^T      A = X   (C x H),   B = W   (V x H)
//   dX         = dZ * W        A = dZ  (C x V),   B = W^T (H x V)
//   dW        += dZ^T * X      A = dZ^T(V x C),   B = X^T (H x C)
// (dZ enters both gradients as the stored exponentials with per-row
// factors applied outside the K loop.)
//
// Block tile BM x BN, 4 waves in a 2 x 2 layout; each wave owns a
// (BM/2) x (BN/2) accumulator tile made of 16 x 16 MFMA fragments.  One
// K-stage covers 128 bytes per row (64 bf16 or 32 fp32), staged through LDS
// by direct-to-LDS loads; rows are stored as eight 16-byte vectors whose
// positions are XOR-swizzled by the row index so that both the DMA writes
// and the fragment reads are free of bank conflicts.  (Full 128-byte row
// segments per load matter: a deeper ring of 64-byte stages in the same LDS
// was measured slower.)
//
// Pipeline: each K-stage is split in two substeps around one barrier.  The
// LDS holds three A buffers and two B buffers (160 KB for 256 x 256), so the
// A half of stage kt + 2 can be loaded while stage kt is still being read:
//   [A] substep-0 MFMAs of stage kt | substep-1 reads of stage kt,
//       A DMAs of stage kt + 2 (into the A buffer of stage kt - 1)
//   wait: everything but those A DMAs; barrier
//   [B] substep-1 MFMAs of stage kt | substep-0 reads of stage kt + 1,
//       B DMAs of stage kt + 2 (into the B buffer of stage kt)
// The address unit thus sees half the DMAs in each phase instead of all of
// them in one.
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
//
// BT (bf16 only): B is given as stored, K rows of N contiguous elements
// (dX = dZ W reading W itself rather than a transposed copy).  A B stage is
// then 64 k-rows of BN elements; its fragments come from ds_read_b64_tr_b16,
// which in each group of 16 lanes hands slot i of lane d the element d % 4
// of what lane 4 i + d / 4 read.  Two such reads (k-rows k and k + 4) give
// lane l its column l % 16 at 8 consecutive k when lane s reads k-row
// 8 (s / 16) + (s % 16) / 4, columns 4 (s % 4) .. +3.  The 16-byte units of
// k-row r sit at unit ^ tr_swz(r), which keeps those reads free of bank
// conflicts.  The reads move 8 bytes per lane instead of 16, so this engine
// runs 8-12 % slower than with a transposed copy of B; it saves the copy's
// memory.
//
// AT (bf16 only): the same for A, given as K rows of M contiguous elements
// (dW = dZ^T X reading the exponentials as the logits epilogue stored them:
// token rows of vocabulary columns), with A stages of 64 k-rows of BM
// elements and the same transposing fragment reads.
//
#pragma once

#include "common.h"

namespace flce {

// MFMAs at the end of phase A kept free of side operations in kernels that
// read B (dX reading W) or A (dW reading the exponentials) as stored (see
// the K loop): measured on one box, 16 took the first 1.7 % faster and 8
// the second 0.3 %, against none; with the first's B fragment kept fixed
// between issues, 24 measured 0.4 % faster than 16 and 8 0.3 % slower.
#ifndef FLCE_TR_TAIL_B
#define FLCE_TR_TAIL_B 24
#endif
#ifndef FLCE_TR_TAIL_A
#define FLCE_TR_TAIL_A 8
#endif

struct GemmShape {
  const void* A;
  const void* B;
  int64_t lda, ldb;  // leading dimensions in elements
  int M, N, K;       // K % Elem<T>::kVec == 0
  int tiles_m, tiles_n;
  int splits;        // split-K factor (1 = none)
  int k_per_split;   // multiple of the stage depth, unused when splits == 1
  int group_m;       // rows of tiles walked together (>= 1)
  // Logical tiles this launch covers: [tile_first, tile_first + tile_count)
  // of the grid's walk order (set by the launcher; all tiles by default).
  int tile_first, tile_count;
};

struct TileCoord {
  int tm, tn, split;
  int slot;  // index of the tile within the launch's range
};

// Logical tile -> (row tile, column tile): M fastest inside groups of
// `group_m` rows of tiles.
__device__ __forceinline__ void tile_rc(const GemmShape& g, int tile, int& tm, int& tn) {
  const int per_group = g.group_m * g.tiles_n;
  const int gid = tile / per_group;
  const int first_m = gid * g.group_m;
  const int gsize = min(g.tiles_m - first_m, g.group_m);
  const int in_group = tile - gid * per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// Block id -> tile.  Hardware dispatches consecutive block ids to the 8 XCDs
// round-robin; give each XCD a contiguous range of logical tiles.
__device__ __forceinline__ TileCoord map_tile(const GemmShape& g) {
  const int nblk = (int)gridDim.x;
  const int bid = (int)blockIdx.x;
  const int q = nblk >> 3, r = nblk & 7;
  const int xcd = bid & 7, slot = bid >> 3;
  const int logical = xcd * q + min(xcd, r) + slot;
  TileCoord c;
  c.split = logical / g.tile_count;
  c.slot = logical - c.split * g.tile_count;
  tile_rc(g, g.tile_first + c.slot, c.tm, c.tn);
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
// Order of the FM x FN MFMAs of a substep (fragment row i = A fragment, the
// instruction's second source; column j = B fragment, its first source),
// chosen by the epilogue type (Epi::kOrder) for the contraction it serves:
//   0: row by row, j fastest;
//   1: row by row with the odd rows backwards, so that consecutive MFMAs
//      always share an operand (the A fragment within a row, the B fragment
//      at a row change);
//   2: column by column with the odd columns backwards (the B fragment
//      stays within a column).
// Every accumulator still sees the same K order, so results do not change.
// The order sets which operand's bits toggle between issues, and the matrix
// units' power -- and so the clock the chip sustains at its power limit --
// depends on that: keeping the operand with O(1) values (whose exponents
// straddle 1.0, where all eight exponent bits flip) fixed measured faster.
template <int FM, int FN, int ORDER>
__device__ __forceinline__ constexpr int mma_row(int q) {
  if constexpr (ORDER == 2) {
    const int c = q / FM, r = q % FM;
    return (c & 1) ? FM - 1 - r : r;
  } else {
    return q / FN;
  }
}
template <int FM, int FN, int ORDER>
__device__ __forceinline__ constexpr int mma_col(int q) {
  if constexpr (ORDER == 2) {
    return q / FM;
  } else {
    const int r = q / FN, c = q % FN;
    return (ORDER == 1 && (r & 1)) ? FN - 1 - c : c;
  }
}
// n-th fragment read of a substep: r < FM is A fragment r, else B fragment
// r - FM.  The first MFMAs of the order are served first: one A fragment and
// every B fragment (orders 0, 1), or one B fragment and every A fragment (2).
template <int FM, int FN, int ORDER>
__device__ __forceinline__ constexpr int read_slot(int n) {
  if constexpr (ORDER == 2)
    return n == 0 ? FM : n <= FM ? n - 1 : n;
  else
    return (n + FM) % (FM + FN);
}
// The same order counted in LDS read instructions: a fragment of an operand
// read as stored (A with TA, B with TB) takes two transposing 8-byte reads,
// each a slot of its own, so that the schedule spreads them like the others.
// Returns 4 r + h for fragment r (as read_slot) and h = 0 (the whole
// fragment), 1 (its first half) or 2 (its second half).
template <int FM, int FN, int ORDER, bool TA, bool TB>
__device__ __forceinline__ constexpr int read_part(int p) {
  for (int n = 0; n < FM + FN; ++n) {
    const int r = read_slot<FM, FN, ORDER>(n);
    const bool tr = r < FM ? TA : TB;
    if (p < (tr ? 2 : 1)) return 4 * r + (tr ? 1 + p : 0);
    p -= tr ? 2 : 1;
  }
  return -1;
}

template <int FM, int FN>
__device__ __forceinline__ void drain_fence(f4 (&acc)[FM][FN]) {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) asm volatile("" : "+a"(acc[i][j]));
#endif
}

// WAVES = 4: 2 x 2 waves, one per SIMD.
template <int BM, int BN, int WAVES = 4>
struct TileGeom {
  static constexpr int kWaves = WAVES;
  static constexpr int kWavesN = WAVES / 2;
  static constexpr int kThreads = 64 * WAVES;
  static constexpr int WM = BM / 2, WN = BN / kWavesN;  // wave tile
  static constexpr int FM = WM / 16, FN = WN / 16;
  // LDS: three A stage buffers and two B stage buffers of 128-byte rows
  static constexpr int kABufBytes = BM * 128, kBBufBytes = BN * 128;
  static constexpr int kLdsBytes = 3 * kABufBytes + 2 * kBBufBytes;
};

// Position of k-vector `kv` (0..7) of LDS row `row` within a stage.
__device__ __forceinline__ int swz(int row, int kv) { return row * 8 + (kv ^ (row & 7)); }

// BT stages: position of 16-byte unit u of k-row r is u ^ tr_swz(r).  The
// four k-rows one lane group reads land in four different 32-byte windows,
// and the groups served in the same cycle (k-rows 8 apart) in different
// 128-byte halves of the banks.
__device__ __forceinline__ int tr_swz(int r) { return (2 * (r & 3)) ^ (8 * ((r >> 3) & 1)); }

typedef short v4s_t __attribute__((ext_vector_type(4)));
// 8 bytes per lane from LDS, transposed within each group of 16 lanes.
__device__ __forceinline__ uint2 lds_read_tr16(uint32_t byte_addr) {
#if defined(__HIP_DEVICE_COMPILE__)
  const v4s_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s_t*)(size_t)byte_addr);
  return __builtin_bit_cast(uint2, v);
#else
  (void)byte_addr;
  return make_uint2(0u, 0u);
#endif
}

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
  int slot;        // the block tile's index within the launch's tile range
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

// K-loop schedule (the pipeline described at the top), per 128-byte stage:
//   [A] substep-0 MFMAs on fragments already in registers, with the
//       substep-1 fragment reads of the same stage and the A DMAs of the
//       stage after next threaded through them;
//   wait + barrier: this wave's reads of the stage are done and the next
//       stage has landed, in every wave;
//   [B] substep-1 MFMAs, with the next stage's substep-0 fragment reads and
//       the B DMAs of the stage after next threaded through them.
// The wave never waits on LDS after the barrier: the fragments its MFMAs
// need were read before it.
template <typename T, int BM, int BN, int WAVES, class Epi, bool BT = false, bool AT = false>
__global__ void __launch_bounds__(64 * WAVES) gemm_nt_kernel(GemmShape g, Epi epi) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass needs only the launch stub
  using G = TileGeom<BM, BN, WAVES>;
  constexpr int EPV = Elem<T>::kVec;
  constexpr int BK = 8 * EPV;
  constexpr int ES = (int)sizeof(T);
  constexpr int A_INS = BM / (8 * WAVES);  // 16-byte loads per lane per stage (A)
  constexpr int B_INS = BN / (8 * WAVES);
  constexpr int FM = G::FM, FN = G::FN;
  static_assert(!BT || (sizeof(T) == 2 && WAVES == 4), "stored-layout B: bf16, 4 waves");
  static_assert(!AT || (sizeof(T) == 2 && WAVES == 4), "stored-layout A: bf16, 4 waves");
  constexpr int UPR = BN / 8;   // BT: 16-byte units per k-row of a B stage
  constexpr int UPRA = BM / 8;  // AT: the same for an A stage
  extern __shared__ uint4 lds[];  // G::kLdsBytes, sized at launch

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
  // AT: from A's column m0 over all K rows (the host keeps K lda ES < 2^31)
  const i4v rA = AT ? make_rsrc((const T*)g.A + m0, (uint32_t)((int64_t)g.K * g.lda * ES))
                    : make_rsrc((const T*)g.A + (int64_t)m0 * g.lda,
                                (uint32_t)((int64_t)a_rows * g.lda * ES));
  // BT: from B's column n0 over all K rows (the host keeps K ldb ES < 2^31,
  // below the out-of-range offset)
  const i4v rB = BT ? make_rsrc((const T*)g.B + n0, (uint32_t)((int64_t)g.K * g.ldb * ES))
                    : make_rsrc((const T*)g.B + (int64_t)n0 * g.ldb,
                                (uint32_t)((int64_t)b_rows * g.ldb * ES));

  // Direct-to-LDS loads write lane i of a wave's load to the LDS slot
  // base + 16 i.  Slot p of a stage holds row p / 8 and logical k-vector
  // (p % 8) ^ (row % 8), i.e. the XOR-swizzled layout read by swz().  Every
  // load of a wave covers 8 whole rows, so the k-vector of a lane is the
  // same in all of its loads.
  uint32_t a_off[A_INS], b_off[B_INS];
  const int kv_lane = (lane & 7) ^ ((lane >> 3) & 7);
  // AT: as BT below, for the A stages (a_krow, a_min: the unit's k-row and
  // whether its columns lie inside M)
  int a_krow[A_INS];
  bool a_min[A_INS];
#pragma unroll
  for (int j = 0; j < A_INS; ++j) {
    if constexpr (!AT) {
      const int row = wave * (BM / WAVES) + 8 * j + (lane >> 3);
      a_off[j] = (uint32_t)(((int64_t)row * g.lda + kv_lane * EPV) * ES);
      a_krow[j] = 0;
      a_min[j] = true;
    } else {
      const int p = wave * (16 * UPRA) + 64 * j + lane;
      const int r = p / UPRA, u = (p % UPRA) ^ tr_swz(p / UPRA);
      a_off[j] = (uint32_t)(((int64_t)r * g.lda + 8 * u) * ES);
      a_krow[j] = r;
      a_min[j] = m0 + 8 * u < g.M;
    }
  }
  // BT: slot p of a B stage holds k-row p / UPR, unit (p % UPR) ^ tr_swz(row);
  // b_krow is that k-row, b_nin whether the unit's columns lie inside N.
  int b_krow[B_INS];
  bool b_nin[B_INS];
#pragma unroll
  for (int j = 0; j < B_INS; ++j) {
    if constexpr (!BT) {
      const int row = wave * (BN / WAVES) + 8 * j + (lane >> 3);
      b_off[j] = (uint32_t)(((int64_t)row * g.ldb + kv_lane * EPV) * ES);
      b_krow[j] = 0;
      b_nin[j] = true;
    } else {
      const int p = wave * (16 * UPR) + 64 * j + lane;
      const int r = p / UPR, u = (p % UPR) ^ tr_swz(p / UPR);
      b_off[j] = (uint32_t)(((int64_t)r * g.ldb + 8 * u) * ES);
      b_krow[j] = r;
      b_nin[j] = n0 + 8 * u < g.N;
    }
  }
  const uint32_t lds_base = (uint32_t)(size_t)((lds_ptr_t)lds);
  const uint32_t lds_a = lds_base + wave * (BM * 8 / WAVES) * 16;
  const uint32_t lds_b = lds_base + 3 * G::kABufBytes + wave * (BN * 8 / WAVES) * 16;

  EpiCoord ec;
  ec.row0 = m0 + wm * G::WM;
  ec.col0 = n0 + wn * G::WN;
  ec.lane = lane;
  ec.split = tc.split;
  ec.slot = tc.slot;

  // The epilogue chooses the starting accumulators: zero, or (to accumulate
  // into an existing output) its old values, loaded with load16_acc here,
  // before any DMA, so that the prologue's wait for stage 0 covers them.
  f4 acc[FM][FN];
  epi.template init<FM, FN>(acc, ec);

  // DMA j of one operand for K-offset k0 into A buffer `ab` (0..2) or B
  // buffer `bb` (0..1).  Past the end of K every offset is out of range and
  // the buffer fills with zeros.
  auto issue_a = [&](int ab, int k0, int j) {
    if constexpr (!AT) {
      const bool kin = kv_lane * EPV < k_end - k0;
      dma16(rA, lds_a + (uint32_t)ab * G::kABufBytes + 1024 * j, kin ? a_off[j] : kOobOffset,
            k0 * ES);
    } else {
      const bool in = a_min[j] && a_krow[j] < k_end - k0;
      dma16(rA, lds_a + (uint32_t)ab * G::kABufBytes + 1024 * j, in ? a_off[j] : kOobOffset,
            (uint32_t)((int64_t)k0 * g.lda * ES));
    }
  };
  auto issue_b = [&](int bb, int k0, int j) {
    if constexpr (!BT) {
      const bool kin = kv_lane * EPV < k_end - k0;
      dma16(rB, lds_b + (uint32_t)bb * G::kBBufBytes + 1024 * j, kin ? b_off[j] : kOobOffset,
            k0 * ES);
    } else {
      const bool in = b_nin[j] && b_krow[j] < k_end - k0;
      dma16(rB, lds_b + (uint32_t)bb * G::kBBufBytes + 1024 * j, in ? b_off[j] : kOobOffset,
            (uint32_t)((int64_t)k0 * g.ldb * ES));
    }
  };
  // Half h (1: k-rows k0 .. k0 + 3 of each group of 8, 2: the next four) of
  // a fragment of a stage read as stored: elements c16 .. c16 + 15 of rows
  // `row_bytes` long in the stage buffer at `buf`, substep s.  Into `f`'s
  // first (h = 1) or second (h = 2) 8 bytes.
  const int tr_g = lane >> 4, tr_i = (lane >> 2) & 3, tr_q = lane & 3;
  auto read_tr_half = [&](uint32_t buf, int row_bytes, int c16, int s, int h, uint4& f) {
    const int u = (c16 >> 3) + (tr_q >> 1);
    const int kr = 32 * s + 8 * tr_g + tr_i + (h == 2 ? 4 : 0);
    const uint2 v = lds_read_tr16(buf + kr * row_bytes + ((u ^ tr_swz(kr)) << 4) + (tr_q & 1) * 8);
    if (h == 1) {
      f.x = v.x;
      f.y = v.y;
    } else {
      f.z = v.x;
      f.w = v.y;
    }
  };
  // LDS read `code` (read_part) of substep s from A buffer ab / B buffer bb:
  // fragment r = code / 4 (r < FM: A fragment r, else B fragment r - FM),
  // whole or one half.
  auto read_one = [&](int ab, int bb, int s, int code, uint4 (&fa)[FM], uint4 (&fb)[FN]) {
    const int r = code >> 2, h = code & 3;
    const int kv = 4 * s + (lane >> 4);
    if (r < FM) {
      if constexpr (!AT)
        fa[r] = lds[ab * (G::kABufBytes / 16) + swz(wm * G::WM + 16 * r + (lane & 15), kv)];
      else
        read_tr_half(lds_base + (uint32_t)ab * G::kABufBytes, BM * 2, wm * G::WM + 16 * r, s, h,
                     fa[r]);
    } else if constexpr (!BT)
      fb[r - FM] = lds[(3 * G::kABufBytes + bb * G::kBBufBytes) / 16 +
                       swz(wn * G::WN + 16 * (r - FM) + (lane & 15), kv)];
    else
      read_tr_half(lds_base + 3 * G::kABufBytes + (uint32_t)bb * G::kBBufBytes, BN * 2,
                   wn * G::WN + 16 * (r - FM), s, h, fb[r - FM]);
  };

  // Reading B as stored (dX reading W), its transposed fragments are the
  // costlier reads: keeping B fixed between issues measured 2 % faster than
  // the epilogue's own order on that GEMM (alternating runs on one box).
  constexpr int ORD = BT ? 2 : Epi::kOrder;
  static_assert(ORD >= 0 && ORD <= 2, "MFMA order");
  constexpr int NR = FM * (AT ? 2 : 1) + FN * (BT ? 2 : 1);  // LDS reads per substep
  constexpr int NM = FM * FN;  // MFMAs per substep
  constexpr int NDMA = A_INS + B_INS;
  // each phase carries NR reads and the DMAs of one operand
  constexpr int NSA = NR + A_INS, NSB = NR + B_INS;
  constexpr int SPA = NM / NSA > 0 ? NM / NSA : 1;
  constexpr int SPB = NM / NSB > 0 ? NM / NSB : 1;
  static_assert(NSA * SPA <= NM && NSB * SPB <= NM, "side operations must fit");
  // Phase A ends in a wait for all of its LDS reads (the barrier after it
  // lets the B buffer they read be overwritten).  With operands read as
  // stored a phase carries so many reads that one every SPA MFMAs would put
  // the last of them just before that wait; they are spread over the first
  // NM - kTailA MFMAs instead (as far as they fit).
  constexpr int kTailWant = BT ? FLCE_TR_TAIL_B : AT ? FLCE_TR_TAIL_A : 0;
  constexpr int kTailA = kTailWant < NM - NSA ? kTailWant : NM - NSA;
  static_assert(NSA <= NM - kTailA, "side operations must fit before the tail");
  static_assert(NDMA < 64, "vmcnt field");
  // s_waitcnt vmcnt(NDMA), expcnt/lgkmcnt not waited on
  constexpr int kWaitStage0 = (NDMA & 0xF) | ((NDMA >> 4) << 14) | 0x0F70;
  // s_waitcnt vmcnt(A_INS) lgkmcnt(0): all but the A DMAs of this phase A
  constexpr int kWaitMid = (A_INS & 0xF) | ((A_INS >> 4) << 14) | 0x0070;

  uint4 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
  if (nk > 0) {
#pragma unroll
    for (int j = 0; j < A_INS; ++j) issue_a(0, k_begin, j);
#pragma unroll
    for (int j = 0; j < B_INS; ++j) issue_b(0, k_begin, j);
#pragma unroll
    for (int j = 0; j < A_INS; ++j) issue_a(1, k_begin + BK, j);
#pragma unroll
    for (int j = 0; j < B_INS; ++j) issue_b(1, k_begin + BK, j);
    __builtin_amdgcn_s_waitcnt(kWaitStage0);  // initial accumulators and stage 0 landed
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int n = 0; n < NR; ++n)
      read_one(0, 0, 0,
               (AT || BT || ORD == 2) ? read_part<FM, FN, ORD, AT, BT>(n) : 4 * n, fa0, fb0);
    // stage kt sits in A buffer kt % 3 and B buffer kt % 2
    int a_cur = 0, a_nxt = 1, a_dma = 2;
    for (int kt = 0; kt < nk; ++kt) {
      const int b_cur = kt & 1, b_nxt = b_cur ^ 1;
      const int k2 = k_begin + (kt + 2) * BK;  // past the end: zero fill, unused
      // [A]: substep-0 MFMAs; substep-1 reads of stage kt; A half of stage
      // kt + 2 into the A buffer stage kt - 1 used (read before the last barrier)
#pragma unroll
      for (int q = 0; q < NM; ++q) {
        const int i = mma_row<FM, FN, ORD>(q), j = mma_col<FM, FN, ORD>(q);
        acc[i][j] = mma16<T>(fb0[j], fa0[i], acc[i][j]);
        // side operation k after MFMA q: every SPA MFMAs, or side op k
        // after MFMA floor((k + 1) (NM - kTailA) / NSA) - 1 with a tail
        int k = -1;
        if constexpr (kTailA == 0) {
          if (q % SPA == SPA - 1 && q / SPA < NSA) k = q / SPA;
        } else {
          constexpr int M = NM - kTailA;
          const int kk = ((q + 1) * NSA + M - 1) / M;
          if (kk <= NSA && (kk * M) / NSA == q + 1) k = kk - 1;
        }
        if (k >= 0) {
          if (k % 3 == 2 && k / 3 < A_INS)  // one DMA after every second read
            issue_a(a_dma, k2, k / 3);
          else
            read_one(a_cur, b_cur, 1, read_part<FM, FN, ORD, AT, BT>(k - min((k + 1) / 3, A_INS)),
                     fa1, fb1);
        }
      }
      __builtin_amdgcn_s_waitcnt(kWaitMid);  // stage kt + 1 landed, own reads done
      __builtin_amdgcn_s_barrier();
      // [B]: substep-1 MFMAs; substep-0 reads of stage kt + 1; B half of
      // stage kt + 2 into the B buffer of stage kt (fully read before the barrier)
#pragma unroll
      for (int q = 0; q < NM; ++q) {
        const int i = mma_row<FM, FN, ORD>(q), j = mma_col<FM, FN, ORD>(q);
        acc[i][j] = mma16<T>(fb1[j], fa1[i], acc[i][j]);
        if (q % SPB == SPB - 1 && q / SPB < NSB) {
          const int k = q / SPB;
          if (k % 3 == 2 && k / 3 < B_INS)
            issue_b(b_cur, k2, k / 3);
          else
            read_one(a_nxt, b_nxt, 0, read_part<FM, FN, ORD, AT, BT>(k - min((k + 1) / 3, B_INS)),
                     fa0, fb0);
        }
      }
      const int t = a_cur;
      a_cur = a_nxt;
      a_nxt = a_dma;
      a_dma = t;
      // Drain the MFMA pipe before leaving the loop: the register allocator
      // may copy accumulators on the exit edge, and the hazard recognizer
      // does not see the asm MFMAs whose results those copies read.
      if (kt + 1 == nk) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
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
