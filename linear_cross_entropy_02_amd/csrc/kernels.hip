// Device kernels of the fused linear cross-entropy head (gfx950).
//
// Per token chunk of C rows the host enqueues:
//   logits GEMM   z = X_c W^T on MFMA, with an epilogue that reduces each row
//                 over its 128-column wave tile to (max, sum exp(z - max),
//                 argmax), records the target logit and stores the tile's
//                 exponentials relative to a power of two at or above its
//                 max -- the online-softmax partials of "Alisa's book of
//                 LLMs", Numerical stability and other tricks (running max
//                 with a rescaled denominator);
//   finalize      merges the partials of every row into lse, argmax and the
//                 per-token NLL, and emits the factors that turn the stored
//                 exponentials into dZ = s valid (softmax - onehot)
//                 ("gradient of softmax + CE loss" on the same page): a row
//                 scale beta, the target's correction and, per tile, how far
//                 its reference lies below the row's;
//   row reference rewrites the tiles whose reference lies below their row's
//                 and sets the target column, so that dZ = beta P;
//   dX GEMM       dX_c = dZ W (K = vocabulary) on P, each row finished as
//                 beta acc + correction W[target];
//   dW GEMM       dW += P^T (beta X) over a group of chunks (K = their
//                 tokens), the first group stores.
// A dZ pass (fixup) writes dZ in place and its transpose instead where the
// contractions cannot read P: soft targets, fp32 or wide hidden sizes for dW,
// or when asked to.
#include "kernels.h"

#include <type_traits>

#include "common.h"
#include "gemm.h"

// Rows of tiles walked together by the logits and dW grids (see map_tile):
// 4 for both, measured against 2, 8 and 16 (traffic, clock and time per
// launch; the build can override them to repeat that measurement).
#ifndef FLCE_LOGITS_GROUP_M
#define FLCE_LOGITS_GROUP_M 4
#endif
#ifndef FLCE_DW_GROUP_M
#define FLCE_DW_GROUP_M 4
#endif

namespace flce {

// Power-of-two references of the stored exponentials: a tile whose max (of
// z / tau) is m stores exp2(z log2(e) - k) with k = q ceil(m log2(e) / q),
// q = kRefQuantum.  Any whole power of two at or above the max would do; a
// coarse one makes the tiles of a row mostly share it (their maxima would
// have to straddle a multiple of 32 log2(e) ~ 22 nats), so that the
// row-reference pass can leave those rows' exponentials as they are for the
// contractions and rewrite only the lower tiles of the others.  Values more than ~65 nats
// below their tile's max flush to zero; their softmax is < e^-65 of it.
constexpr float kRefQuantum = 32.f;
__device__ __forceinline__ float ref_power(float m) {
  return __builtin_ceilf(m * kLog2e / kRefQuantum) * kRefQuantum;
}

// ------------------------------------------------------------ epilogues ---

// Stores four consecutive values of one row in the output type.
__device__ __forceinline__ void store4(float* p, f4 v) { *(f4*)p = v; }
__device__ __forceinline__ void store4(bf16* p, f4 v) {
  uint2 w;
  w.x = __builtin_bit_cast(uint32_t, __builtin_convertvector((f4){v[0], v[1], 0, 0}.xy, bf16x2));
  w.y = __builtin_bit_cast(uint32_t, __builtin_convertvector((f4){v[2], v[3], 0, 0}.xy, bf16x2));
  *(uint2*)p = w;
}
__device__ __forceinline__ f4 load4(const float* p) { return *(const f4*)p; }
__device__ __forceinline__ f4 load4(const bf16* p) {
  const uint2 w = *(const uint2*)p;
  return (f4){__builtin_bit_cast(float, w.x << 16), __builtin_bit_cast(float, w.x & 0xffff0000u),
              __builtin_bit_cast(float, w.y << 16), __builtin_bit_cast(float, w.y & 0xffff0000u)};
}

// Logits epilogue: online-logsumexp partials per (row, 128-column wave tile).
// A lane owns one row of each fragment row-block and 32 of the wave tile's
// 128 columns; the other 96 sit in lanes lane ^ 16, ^ 32, ^ 48, so a row
// reduction is a 32-value in-lane pass plus two cross-lane steps.  The
// partials are written tile-major ([tile][row], 16 consecutive rows per
// store) and exp(z - tile max) goes straight out as 4-element row segments.
//
// With a temperature tau the partials are those of z / tau (max m / tau,
// sum of exp(z / tau - m / tau)); with CROSS (soft targets) each (row, tile)
// also gets sum_v P_T z / tau, P_T being the teacher's stored
// exp(z_T / tau - m_T) of the same columns.
template <typename T, bool CROSS = false>
struct LogitsEpi {
  // MFMA issue order (gemm.h): X is the A operand here and W the B operand;
  // X's O(1) values toggle more exponent bits than W's small ones, so the
  // A fragment stays put within a fragment row
  static constexpr int kOrder = 1;
  T* P;
  int64_t ldp;
  float inv_temp;
  const T* Pq;  // CROSS: teacher exponentials, [M x ldp]
  float* pc;    // CROSS: cross partials, [nt x ldr]
  float* pm;
  float* ps;
  int* pa;
  int64_t ldr;  // row stride of the tile-major partial arrays
  float* ztgt;
  const int64_t* y;
  int64_t ignore_index;
  int64_t y_shift;  // vocabulary id of column 0 (a vocabulary shard's offset)
  int M, V;
  bool store_p;  // false: partials and target logit only (forward-only calls)

  template <int FM, int FN>
  __device__ __forceinline__ void init(f4 (&acc)[FM][FN], const EpiCoord&) const {
    zero_init(acc);
  }

  // FULL: every column of the wave tile is < V (no per-column test).
  template <bool FULL, int FM, int FN>
  __device__ __forceinline__ void rows(f4 (&acc)[FM][FN], const EpiCoord& ec) const {
    const int g = ec.lane >> 4, c = ec.lane & 15;
    const int ptile = ec.col0 / (FN * 16);
    const int lc0 = ec.col0 + 4 * g;  // this lane's first column
    // column of the row's target relative to this lane's first column, or
    // -1 when the target is ignored or outside the lane's columns
    int toff[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = ec.row0 + 16 * i + c;
      const int64_t yt = row < M ? y[row] : ignore_index;
      const int64_t off = yt - y_shift - lc0;
      toff[i] = (yt != ignore_index && off >= 0 && off < 16 * FN && (off & 12) == 0 &&
                 lc0 + off < V)
                    ? (int)off : -1;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = ec.row0 + 16 * i + c;
      // max and lowest-index argmax; the lane visits its columns in increasing
      // order, so a strict comparison keeps the first of equal values
      float mx = kNegInf;
      int ai = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float z = acc[i][j][r];
          if ((FULL || lc0 + 16 * j + r < V) && z > mx) {
            mx = z;
            ai = lc0 + 16 * j + r;
          }
        }
#pragma unroll
      for (int m = 16; m <= 32; m *= 2) {
        const float om = shfl_xor_f(mx, m);
        const int oa = shfl_xor_i(ai, m);
        const bool take = om > mx || (om == mx && oa < ai);
        mx = take ? om : mx;
        ai = take ? oa : ai;
      }
      // target logit: held by the one lane whose columns contain y (rare
      // branch: a row's target falls in one of V / 128 wave tiles)
      {
        if (toff[i] >= 0) {
          const int tk = 4 * (toff[i] >> 4) + (toff[i] & 3);
          float zt = 0.f;
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) zt = (4 * j + r == tk) ? acc[i][j][r] : zt;
          ztgt[row] = zt;
        }
      }
      float cross = 0.f;
      if constexpr (CROSS) {
        // columns >= V hold a zero teacher exponential and a zero logit
        if (row < M) {
          const T* const qrow = Pq + (int64_t)row * ldp + lc0;
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const f4 q = load4(qrow + 16 * j);
#pragma unroll
            for (int r = 0; r < 4; ++r) cross = __builtin_fmaf(q[r], acc[i][j][r], cross);
          }
        }
        cross += shfl_xor_f(cross, 16);
        cross += shfl_xor_f(cross, 32);
      }
      // exponentials relative to 2^kq, kq = q ceil(tile max log2(e) / q)
      // with q = kRefQuantum: a whole power of two, so that the merge turns
      // them into probabilities with a per-row scale and an exact
      // power-of-two factor per tile (q is a power of two: / q is exact)
      const float kl = kLog2e * inv_temp;
      const float pmv = mx * inv_temp;
      const float kq = (mx == kNegInf) ? 0.f : ref_power(pmv);
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = (FULL || lc0 + 16 * j + r < V)
                              ? __builtin_amdgcn_exp2f(__builtin_fmaf(acc[i][j][r], kl, -kq))
                              : 0.f;
          sum += e;
          acc[i][j][r] = e;
        }
      sum += shfl_xor_f(sum, 16);
      sum += shfl_xor_f(sum, 32);
      if (row < M) {
        if (g == 0 && ec.col0 < V) {
          const int64_t o = (int64_t)ptile * ldr + row;
          pm[o] = pmv;
          ps[o] = sum;
          pa[o] = ai;
          if constexpr (CROSS) pc[o] = cross * inv_temp;
        }
        // columns up to the padded row length are allocated; those >= V get 0
        if (store_p) {
          T* const prow = P + (int64_t)row * ldp + lc0;
#pragma unroll
          for (int j = 0; j < FN; ++j) store4(prow + 16 * j, acc[i][j]);
        }
      }
    }
  }

  template <int FM, int FN>
  __device__ __forceinline__ void apply(f4 (&acc)[FM][FN], const EpiCoord& ec) const {
    if (ec.col0 + 16 * FN <= V)
      rows<true>(acc, ec);
    else
      rows<false>(acc, ec);
  }
};

// Plain store epilogue (dX, dW, split-K partials): each lane stores four
// consecutive columns of one row per fragment.  To accumulate into the fp32
// output (dW over token chunks) the accumulators start from the old values,
// loaded before the K loop, so the epilogue is a plain store either way.
// ACC = false (dX, split-K partials) starts from zero with no loads.
// N % 4 == 0, so a 4-column segment is either whole or outside.
template <typename TO, bool ACC>
struct StoreEpi {
  static_assert(!ACC || std::is_same<TO, float>::value, "accumulation is fp32 only");
  // MFMA issue order (gemm.h).  ACC: dW = dZ^T X, whose B operand is X: the
  // B fragment stays put within a fragment column.  Otherwise dX = dZ W (or
  // its split-K partials): the A fragment (dZ) stays put within a row.
  static constexpr int kOrder = ACC ? 2 : 1;
  TO* out;
  int64_t ldo;
  int M, N;
  int64_t split_stride;
  bool accumulate;

  template <int FM, int FN>
  __device__ __forceinline__ void init(f4 (&acc)[FM][FN], const EpiCoord& ec) const {
    if constexpr (!ACC) {
      zero_init(acc);
    } else {
      // One unconditional path (no merge of a zero and a loaded value for
      // the register allocator to reconcile with copies): every fragment is
      // loaded through a buffer resource covering the wave's rows below M.
      // Rows past M read zero; columns past N, and everything when not
      // accumulating, get an out-of-range offset, which also reads zero.
      const int g = ec.lane >> 4, c = ec.lane & 15;
      const int rows = M - ec.row0 < 16 * FM ? M - ec.row0 : 16 * FM;
      const float* const base =
          out + (int64_t)ec.split * split_stride + (int64_t)ec.row0 * ldo + ec.col0;
      const i4v rs = make_rsrc(base, rows > 0 && accumulate ? (uint32_t)((int64_t)rows * ldo * 4) : 0u);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = 4 * g + 16 * j;
          const uint32_t off = (uint32_t)(((16 * i + c) * ldo + col) * 4);
          load16_acc(acc[i][j], rs, accumulate && ec.col0 + col < N ? off : kOobOffset);
        }
    }
  }

  template <int FM, int FN>
  __device__ __forceinline__ void apply(f4 (&acc)[FM][FN], const EpiCoord& ec) const {
    const int g = ec.lane >> 4, c = ec.lane & 15;
    TO* const base = out + (int64_t)ec.split * split_stride;
    const int lc0 = ec.col0 + 4 * g;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = ec.row0 + 16 * i + c;
      TO* const p = base + (int64_t)row * ldo + lc0;
#pragma unroll
      for (int j = 0; j < FN; ++j)
        if (row < M && lc0 + 16 * j < N) store4(p + 16 * j, acc[i][j]);
    }
  }
};

// dX epilogue when dZ is formed inside the contraction (the A operand is
// the stored exponentials scaled by 2^-shift in registers): row t of the
// output is beta_t acc_t + corr_t W[y_t - y_shift], the second term being
// the one-hot target's correction (corr is 0 when there is none).  TO is the
// input dtype, which dX and W share.
template <typename TO>
struct DxEpi {
  // MFMA issue order (gemm.h): as the other dX kernels, the A fragment (the
  // exponentials) stays put within a fragment row
  static constexpr int kOrder = 1;
  TO* out;
  int64_t ldo;
  int M, N;
  DxFuse f;

  template <int FM, int FN>
  __device__ __forceinline__ void init(f4 (&acc)[FM][FN], const EpiCoord&) const {
    zero_init(acc);
  }

  template <int FM, int FN>
  __device__ __forceinline__ void apply(f4 (&acc)[FM][FN], const EpiCoord& ec) const {
    const int g = ec.lane >> 4, c = ec.lane & 15;
    const int lc0 = ec.col0 + 4 * g;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = ec.row0 + 16 * i + c;
      if (row >= M) continue;
      const float b = f.beta[row], cr = f.corr[row];
      const TO* wr = nullptr;
      if (cr != 0.f) {
        const int64_t yl = f.y[row] - f.y_shift;
        if (yl >= 0 && yl < f.V) wr = (const TO*)f.W + yl * f.ldw;
      }
      TO* const p = out + (int64_t)row * ldo + lc0;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if (lc0 + 16 * j >= N) continue;
        f4 v = acc[i][j] * b;
        if (wr) v += load4(wr + lc0 + 16 * j) * cr;
        store4(p + 16 * j, v);
      }
    }
  }
};

// Split-K partial of one block tile, stored compactly: plane
// (split, slot) of `part` holds the BM x BN block tile row-major, slot being
// the tile's index within the launch's tile range.  Rows and columns past
// the matrix edge hold zeros (their operand rows read as zero).
template <int BM, int BN>
struct TilePartialEpi {
  static constexpr int kOrder = 2;  // dW's tail tiles: as StoreEpi<float, true>
  float* part;
  int tile_count;

  template <int FM, int FN>
  __device__ __forceinline__ void init(f4 (&acc)[FM][FN], const EpiCoord&) const {
    zero_init(acc);
  }

  template <int FM, int FN>
  __device__ __forceinline__ void apply(f4 (&acc)[FM][FN], const EpiCoord& ec) const {
    const int g = ec.lane >> 4, c = ec.lane & 15;
    float* const base = part + ((int64_t)ec.split * tile_count + ec.slot) * (BM * BN);
    const int r0 = ec.row0 % BM, c0 = ec.col0 % BN;  // wave tile within the block tile
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        *(f4*)(base + (r0 + 16 * i + c) * BN + c0 + 16 * j + 4 * g) = acc[i][j];
  }
};

// out[tile] = (accumulate ? out[tile] : 0) + part[0][slot] + ... +
// part[splits-1][slot], in that order, for the tiles [tile_first,
// tile_first + tile_count) of the grid walk `g`; 256 threads x 4 values per
// block, (BM x BN) / 1024 blocks per tile.
template <int BM, int BN>
__global__ void __launch_bounds__(256) tile_reduce_kernel(GemmShape g, const float* part,
                                                          int splits, float* out, int64_t ldo,
                                                          bool accumulate) {
  constexpr int kPerTile = BM * BN / 1024;
  const int slot = blockIdx.x / kPerTile;
  const int e = ((blockIdx.x % kPerTile) * 256 + (int)threadIdx.x) * 4;
  int tm, tn;
  tile_rc(g, g.tile_first + slot, tm, tn);
  const int row = tm * BM + e / BN, col = tn * BN + e % BN;
  if (row >= g.M || col >= g.N) return;  // N % 4 == 0: a 4-column group is whole
  f4* const o = (f4*)(out + (int64_t)row * ldo + col);
  f4 acc = accumulate ? *o : (f4){0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < splits; ++sp)
    acc += *(const f4*)(part + ((int64_t)sp * g.tile_count + slot) * (BM * BN) + e);
  *o = acc;
}

// ------------------------------------------------------------ launchers ---

static inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

template <typename T, int BM, int BN, int WAVES, class Epi, bool BT = false, bool AT = false>
static hipError_t run_gemm(const GemmShape& g0, const Epi& epi, hipStream_t s) {
  using G = TileGeom<BM, BN, WAVES>;
  GemmShape g = g0;
  g.tiles_m = cdiv(g.M, BM);
  g.tiles_n = cdiv(g.N, BN);
  if (g.tiles_m == 0 || g.tiles_n == 0) return hipSuccess;
  if (g.splits < 1) g.splits = 1;
  if (g.group_m < 1) g.group_m = 1;
  if (g.group_m > g.tiles_m) g.group_m = g.tiles_m;
  if (g.tile_count <= 0) {
    g.tile_first = 0;
    g.tile_count = g.tiles_m * g.tiles_n;
  }
  if (g.tile_first < 0 || g.tile_first + g.tile_count > g.tiles_m * g.tiles_n)
    return hipErrorInvalidValue;
  const int nblk = g.tile_count * g.splits;
  hipLaunchKernelGGL((gemm_nt_kernel<T, BM, BN, WAVES, Epi, BT, AT>), dim3(nblk),
                     dim3(G::kThreads), G::kLdsBytes, s, g, epi);
  return hipGetLastError();
}

// The GEMM kernels use more than the default 64 KB of dynamic LDS.
template <typename T, int BM, int BN, int WAVES, class Epi, bool BT = false, bool AT = false>
static hipError_t set_lds_attr() {
  using G = TileGeom<BM, BN, WAVES>;
  return hipFuncSetAttribute((const void*)gemm_nt_kernel<T, BM, BN, WAVES, Epi, BT, AT>,
                             hipFuncAttributeMaxDynamicSharedMemorySize, G::kLdsBytes);
}

// The dX instantiations that finish dZ W rows themselves (DxEpi: row scale
// and target correction), for one B layout, 256- or 128-wide tiles (their
// split-K partials are the plain fp32-partial kernels).
template <typename T, bool BT>
static hipError_t setup_fused_dx() {
  hipError_t e;
  if ((e = set_lds_attr<T, 256, 256, 4, DxEpi<T>, BT>()) != hipSuccess) return e;
  return set_lds_attr<T, 128, 128, 4, DxEpi<T>, BT>();
}

template <typename T>
static hipError_t setup_t() {
  hipError_t e;
  if ((e = set_lds_attr<T, 256, 256, 4, LogitsEpi<T, false>>()) != hipSuccess) return e;
  if ((e = set_lds_attr<T, 256, 256, 4, LogitsEpi<T, true>>()) != hipSuccess) return e;
  if ((e = set_lds_attr<T, 256, 256, 4, StoreEpi<T, false>>()) != hipSuccess) return e;
  if ((e = set_lds_attr<T, 256, 256, 4, StoreEpi<float, false>>()) != hipSuccess) return e;
  if ((e = set_lds_attr<T, 256, 256, 4, StoreEpi<float, true>>()) != hipSuccess) return e;
  if ((e = set_lds_attr<T, 256, 256, 4, TilePartialEpi<256, 256>>()) != hipSuccess) return e;
  if ((e = set_lds_attr<T, 128, 128, 4, StoreEpi<T, false>>()) != hipSuccess) return e;
  if ((e = set_lds_attr<T, 128, 128, 4, StoreEpi<float, false>>()) != hipSuccess) return e;
  if ((e = set_lds_attr<T, 128, 128, 4, StoreEpi<float, true>>()) != hipSuccess) return e;
  if ((e = setup_fused_dx<T, false>()) != hipSuccess) return e;
  if constexpr (std::is_same<T, bf16>::value) {
    // dW reading the exponentials as stored
    if ((e = set_lds_attr<T, 256, 256, 4, StoreEpi<float, true>, false, true>()) != hipSuccess)
      return e;
    if ((e = set_lds_attr<T, 128, 128, 4, StoreEpi<float, true>, false, true>()) != hipSuccess)
      return e;
    if ((e = set_lds_attr<T, 256, 256, 4, TilePartialEpi<256, 256>, false, true>()) != hipSuccess)
      return e;
    // dX reading W as stored
    if ((e = setup_fused_dx<T, true>()) != hipSuccess) return e;
    if ((e = set_lds_attr<T, 256, 256, 4, StoreEpi<T, false>, true>()) != hipSuccess) return e;
    if ((e = set_lds_attr<T, 256, 256, 4, StoreEpi<float, false>, true>()) != hipSuccess) return e;
    if ((e = set_lds_attr<T, 128, 128, 4, StoreEpi<T, false>, true>()) != hipSuccess) return e;
    if ((e = set_lds_attr<T, 128, 128, 4, StoreEpi<float, false>, true>()) != hipSuccess) return e;
  }
  return hipSuccess;
}

// Compute units of the device set up last (all devices of a process are
// taken to be alike): the blocks one round of 256 x 256 tiles occupies.
static int g_num_cus = 256;

hipError_t gemm_setup() {
  hipError_t e = setup_t<bf16>();
  if (e != hipSuccess) return e;
  e = setup_t<float>();
  if (e != hipSuccess) return e;
  int dev = 0, cus = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
    return e;
  if (cus > 0) g_num_cus = cus;
  return hipSuccess;
}

template <typename T, bool CROSS>
static hipError_t logits_run(const LogitsArgs& a, const GemmShape& g, hipStream_t s) {
  LogitsEpi<T, CROSS> epi;
  epi.P = (T*)a.P;
  epi.ldp = a.ldp;
  epi.inv_temp = a.inv_temp;
  epi.Pq = (const T*)a.Pq;
  epi.pc = a.pc;
  epi.pm = a.pm;
  epi.ps = a.ps;
  epi.pa = a.pa;
  epi.ldr = a.ldr;
  epi.ztgt = a.ztgt;
  epi.y = a.y;
  epi.ignore_index = a.ignore_index;
  epi.y_shift = a.y_shift;
  epi.M = a.M;
  epi.V = a.V;
  epi.store_p = a.P != nullptr;
  return run_gemm<T, 256, 256, 4>(g, epi, s);
}

template <typename T>
static hipError_t logits_t(const LogitsArgs& a, hipStream_t s) {
  GemmShape g{};
  g.A = a.X;
  g.B = a.W;
  g.lda = a.H;
  g.ldb = a.H;
  g.M = a.M;
  g.N = a.V;
  g.K = a.H;
  g.splits = 1;
  // Four row tiles per group: the 32 blocks an XCD runs at once form a 4 x 8
  // patch, which keeps both the X chunk and W tiles resident in its L2
  // (walking all 16 row tiles per W tile re-streams X from beyond L2).
  g.group_m = FLCE_LOGITS_GROUP_M;
  return a.Pq ? logits_run<T, true>(a, g, s) : logits_run<T, false>(a, g, s);
}

hipError_t launch_logits(Dt dt, const LogitsArgs& a, hipStream_t s) {
  return dt == Dt::BF16 ? logits_t<bf16>(a, s) : logits_t<float>(a, s);
}

// The dX contraction with dZ formed inside it (GemmOutArgs::fuse): A holds
// the exponentials, each row relative to one power of two.  With splits the
// raw partial planes go out and splitk_reduce finishes them; else DxEpi
// finishes each row (row scale, target correction).
template <typename T, typename TO>
static hipError_t fused_dx(TileCfg tc, const GemmOutArgs& a, const GemmShape& g,
                           const StoreEpi<TO, false>& epi, hipStream_t s) {
  if (g.splits > 1) {
    if constexpr (std::is_same<TO, float>::value) {
      if (a.b_stored) {
        if constexpr (std::is_same<T, bf16>::value) {
          if (tc != TileCfg::T256)
            return run_gemm<T, 128, 128, 4, StoreEpi<float, false>, true>(g, epi, s);
          return run_gemm<T, 256, 256, 4, StoreEpi<float, false>, true>(g, epi, s);
        }
        return hipErrorInvalidValue;
      }
      if (tc != TileCfg::T256) return run_gemm<T, 128, 128, 4, StoreEpi<float, false>>(g, epi, s);
      return run_gemm<T, 256, 256, 4, StoreEpi<float, false>>(g, epi, s);
    }
    return hipErrorInvalidValue;
  } else if constexpr (std::is_same<TO, T>::value) {
    DxEpi<T> de;
    de.out = (T*)a.out;
    de.ldo = a.ldo;
    de.M = a.M;
    de.N = a.N;
    de.f = *a.fuse;
    if (a.b_stored) {
      if constexpr (std::is_same<T, bf16>::value) {
        if (tc != TileCfg::T256) return run_gemm<T, 128, 128, 4, DxEpi<T>, true>(g, de, s);
        return run_gemm<T, 256, 256, 4, DxEpi<T>, true>(g, de, s);
      }
      return hipErrorInvalidValue;
    }
    if (tc != TileCfg::T256) return run_gemm<T, 128, 128, 4, DxEpi<T>>(g, de, s);
    return run_gemm<T, 256, 256, 4, DxEpi<T>>(g, de, s);
  }
  return hipErrorInvalidValue;
}

// The plain grid of a store (not fused, B in the K-contiguous layout), A
// K-contiguous or (AT, dW reading the exponentials as stored) as stored.
template <typename T, typename TO, bool ACC, bool AT>
static hipError_t grid_store(TileCfg tc, const GemmOutArgs& a, const GemmShape& g,
                             const StoreEpi<TO, ACC>& epi, hipStream_t s) {
  if constexpr (ACC) {
    // The grid's last partial round (rem tiles, under half the CUs busy for
    // a whole tile) is split 2-4 ways in K instead: the full rounds run as
    // usual, the rem tiles' K-slices write fp32 partial tiles, and a pass
    // sums them (with the old output) in a fixed order.  A 256-wide grid of
    // under half a round splits whole that way rather than fall back to
    // 128-wide tiles.
    constexpr int BK = 8 * Elem<T>::kVec;
    const int tiles = cdiv(a.M, 256) * cdiv(a.N, 256);
    const int nfull = tiles / g_num_cus * g_num_cus, rem = tiles - nfull;
    const int sp = rem > 0 ? min(4, g_num_cus / rem) : 0;
    if (a.tail_part && g.splits == 1 && (nfull >= g_num_cus || (nfull == 0 && tc != TileCfg::T256)) &&
        rem > 0 && 2 * rem <= g_num_cus && cdiv(a.K, BK) >= 8 * sp &&
        (size_t)sp * rem * 256 * 256 * sizeof(float) <= a.tail_part_bytes) {
      if (nfull > 0) {
        GemmShape gm = g;
        gm.tile_first = 0;
        gm.tile_count = nfull;
        hipError_t e = run_gemm<T, 256, 256, 4, StoreEpi<TO, ACC>, false, AT>(gm, epi, s);
        if (e != hipSuccess) return e;
      }
      hipError_t e;
      GemmShape gt = g;
      gt.tile_first = nfull;
      gt.tile_count = rem;
      gt.splits = sp;
      gt.k_per_split = cdiv(cdiv(a.K, BK), sp) * BK;
      TilePartialEpi<256, 256> pe;
      pe.part = a.tail_part;
      pe.tile_count = rem;
      if ((e = run_gemm<T, 256, 256, 4, TilePartialEpi<256, 256>, false, AT>(gt, pe, s)) != hipSuccess)
        return e;
      // the walk the GEMM used (run_gemm's own view of the grid)
      gt.tiles_m = cdiv(a.M, 256);
      gt.tiles_n = cdiv(a.N, 256);
      gt.group_m = min(max(gt.group_m, 1), gt.tiles_m);
      hipLaunchKernelGGL((tile_reduce_kernel<256, 256>), dim3(rem * (256 * 256 / 1024)),
                         dim3(256), 0, s, gt, (const float*)a.tail_part, sp, (float*)a.out,
                         a.ldo, (bool)(ACC && a.accumulate));
      return hipGetLastError();
    }
  }
  if (tc != TileCfg::T256) return run_gemm<T, 128, 128, 4, StoreEpi<TO, ACC>, false, AT>(g, epi, s);
  return run_gemm<T, 256, 256, 4, StoreEpi<TO, ACC>, false, AT>(g, epi, s);
}

template <typename T, typename TO, bool ACC>
static hipError_t store_t2(TileCfg tc, const GemmOutArgs& a, hipStream_t s) {
  GemmShape g{};
  g.A = a.A;
  g.B = a.B;
  g.lda = a.lda;
  g.ldb = a.ldb;
  g.M = a.M;
  g.N = a.N;
  g.K = a.K;
  g.splits = a.splits < 1 ? 1 : a.splits;
  if (g.splits > 1) {
    constexpr int BK = 8 * Elem<T>::kVec;
    const int ksteps = cdiv(a.K, BK);
    g.k_per_split = cdiv(ksteps, g.splits) * BK;
  }
  g.group_m = ACC ? FLCE_DW_GROUP_M : 4;
  StoreEpi<TO, ACC> epi;
  epi.out = (TO*)a.out;
  epi.ldo = a.ldo;
  epi.M = a.M;
  epi.N = a.N;
  epi.split_stride = a.split_stride;
  epi.accumulate = ACC && a.accumulate;
  if (a.fuse) {
    // dZ formed inside the contraction; split-K: the partial planes, summed
    // and finished by splitk_reduce
    if constexpr (!ACC) return fused_dx<T, TO>(tc, a, g, epi, s);
    return hipErrorInvalidValue;
  }
  if (a.b_stored) {
    if constexpr (std::is_same<T, bf16>::value && !ACC) {
      if (tc != TileCfg::T256) return run_gemm<T, 128, 128, 4, StoreEpi<TO, ACC>, true>(g, epi, s);
      return run_gemm<T, 256, 256, 4, StoreEpi<TO, ACC>, true>(g, epi, s);
    }
    return hipErrorInvalidValue;
  }
  if (a.a_stored) {
    if constexpr (std::is_same<T, bf16>::value && ACC) return grid_store<T, TO, ACC, true>(tc, a, g, epi, s);
    return hipErrorInvalidValue;
  }
  return grid_store<T, TO, ACC, false>(tc, a, g, epi, s);
}

template <typename T>
static hipError_t store_t(TileCfg tc, const GemmOutArgs& a, hipStream_t s) {
  if (a.accumulate && !(a.out_f32 && a.may_accumulate)) return hipErrorInvalidValue;
  if (!a.out_f32) return store_t2<T, T, false>(tc, a, s);
  return a.may_accumulate ? store_t2<T, float, true>(tc, a, s) : store_t2<T, float, false>(tc, a, s);
}

hipError_t launch_gemm_store(Dt dt, TileCfg tc, const GemmOutArgs& a, hipStream_t s) {
  return dt == Dt::BF16 ? store_t<bf16>(tc, a, s) : store_t<float>(tc, a, s);
}

// ------------------------------------------------- n_valid and the scale ---
// n_valid = number of targets that are not the ignore index (the masked
// mean's denominator, "Information theory > implementing the loss");
// out-of-range targets are counted separately and treated as ignored.
__device__ __forceinline__ void count_finish(long long n, long long nb, int reduction_sum,
                                             int64_t* n_valid, float* scale, int64_t* bad,
                                             int64_t* n_valid_out) {
  *n_valid = n;
  *bad = nb;
  // backward seed: 1 for the sum, 1/n for the mean (0 when n = 0)
  *scale = reduction_sum ? 1.f : (n > 0 ? 1.f / (float)n : 0.f);
  if (n_valid_out) *n_valid_out = n;
}

// Counts over a grid-stride range of the targets: a grid of one block writes
// the results, a larger grid writes per-block counts to part ([nblk] valid,
// then [nblk] out of range) for count_sum_kernel.
__global__ void __launch_bounds__(1024) count_kernel(const int64_t* __restrict__ y, int64_t T,
                                                     int64_t ignore_index, int64_t V,
                                                     int reduction_sum, int64_t* n_valid,
                                                     float* scale, int64_t* bad,
                                                     int64_t* n_valid_out, long long* part) {
  __shared__ long long s_nv[1024], s_nb[1024];
  long long nv = 0, nb = 0;
  // unrolled so that eight independent target loads are in flight per thread
#pragma unroll 8
  for (int64_t t = (int64_t)blockIdx.x * 1024 + threadIdx.x; t < T;
       t += (int64_t)gridDim.x * 1024) {
    const int64_t v = y[t];
    if (v != ignore_index) {
      if (v >= 0 && v < V)
        ++nv;
      else
        ++nb;
    }
  }
  s_nv[threadIdx.x] = nv;
  s_nb[threadIdx.x] = nb;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      s_nv[threadIdx.x] += s_nv[threadIdx.x + w];
      s_nb[threadIdx.x] += s_nb[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    if (gridDim.x == 1) {
      count_finish(s_nv[0], s_nb[0], reduction_sum, n_valid, scale, bad, n_valid_out);
    } else {
      part[blockIdx.x] = s_nv[0];
      part[gridDim.x + blockIdx.x] = s_nb[0];
    }
  }
}

// Sum of the per-block counts (integers: exact in any order).
__global__ void count_sum_kernel(const long long* __restrict__ part, int nblk, int reduction_sum,
                                 int64_t* n_valid, float* scale, int64_t* bad,
                                 int64_t* n_valid_out) {
  if (threadIdx.x != 0) return;
  long long nv = 0, nb = 0;
  for (int i = 0; i < nblk; ++i) {
    nv += part[i];
    nb += part[nblk + i];
  }
  count_finish(nv, nb, reduction_sum, n_valid, scale, bad, n_valid_out);
}

hipError_t launch_count(const int64_t* y, int64_t T, int64_t ignore_index, int64_t V,
                        int reduction_sum, int64_t* n_valid, float* scale, int64_t* bad,
                        int64_t* n_valid_out, long long* part, hipStream_t s) {
  // one block up to 32768 targets; beyond, a block per 8192 of them, at most
  // kCountBlocks, and a second pass over their counts
  const int64_t want = (T + 8191) / 8192;
  const int nblk = (part && T >= 32768) ? (int)(want < kCountBlocks ? want : kCountBlocks) : 1;
  hipLaunchKernelGGL(count_kernel, dim3(nblk), dim3(1024), 0, s, y, T, ignore_index, V,
                     reduction_sum, n_valid, scale, bad, n_valid_out, part);
  if (nblk > 1)
    hipLaunchKernelGGL(count_sum_kernel, dim3(1), dim3(64), 0, s, (const long long*)part, nblk,
                       reduction_sum, n_valid, scale, bad, n_valid_out);
  return hipGetLastError();
}

// ------------------------------------------------------------ transpose ---
// 64 x 64 tiles through LDS, 16-byte global accesses on both sides.
template <typename T>
__global__ void __launch_bounds__(256) transpose_kernel(const T* __restrict__ src, int rows, int cols,
                                                        int64_t ld_src, T* __restrict__ dst,
                                                        int64_t ld_dst, int rows_out,
                                                        const float* __restrict__ row_scale) {
  constexpr int EPV = Elem<T>::kVec;
  constexpr int VPR = 64 / EPV;              // vectors per 64-element row
  constexpr int PER = 64 * VPR / 256;        // vectors per thread
  __shared__ T tile[64][64 + 2];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int v = tid + 256 * p;
    const int r = v / VPR, cv = v % VPR;
    const int gr = r0 + r, gc = c0 + cv * EPV;
    uint4 val = {0u, 0u, 0u, 0u};
    if (gr < rows && gc < cols) val = *(const uint4*)(src + (int64_t)gr * ld_src + gc);
    const T* e = (const T*)&val;
    const float sc = (row_scale && gr < rows) ? row_scale[gr] : 1.f;
#pragma unroll
    for (int k = 0; k < EPV; ++k)
      tile[r][cv * EPV + k] = row_scale ? Elem<T>::from_f32(sc * Elem<T>::to_f32(e[k])) : e[k];
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int v = tid + 256 * p;
    const int c = v / VPR, rv = v % VPR;
    const int gc = c0 + c, gr = r0 + rv * EPV;
    if (gc >= cols || gr >= rows_out) continue;
    uint4 val;
    T* e = (T*)&val;
#pragma unroll
    for (int k = 0; k < EPV; ++k) e[k] = tile[rv * EPV + k][c];
    *(uint4*)(dst + (int64_t)gc * ld_dst + gr) = val;
  }
}

// bf16 with 8-element alignment everywhere: 64 source rows x 256 source
// columns per block, the layout and 8 x 8 register transpose of the bf16
// fixup (swizzled 512-byte LDS rows, 16-byte accesses on both sides, eight
// neighbouring threads per 128-byte destination run).
__global__ void __launch_bounds__(256) transpose_bf16_kernel(const uint16_t* __restrict__ src,
                                                             int rows, int cols, int64_t ld_src,
                                                             uint16_t* __restrict__ dst,
                                                             int64_t ld_dst, int rows_out,
                                                             const float* __restrict__ row_scale) {
  __shared__ uint4 tile[64 * 32];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 256;
  const int tid = threadIdx.x;
  const int cv = tid & 31;
  const int gc = c0 + 8 * cv;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int r = (tid >> 5) + 8 * p;
    const int gr = r0 + r;
    uint4 val = make_uint4(0u, 0u, 0u, 0u);
    if (gr < rows && gc < cols) val = *(const uint4*)(src + (int64_t)gr * ld_src + gc);
    if (row_scale && gr < rows) {  // row gr times its scale, rounded to bf16
      float e[8];
      unpack8_bf16(val, e);
      const float sc = row_scale[gr];
#pragma unroll
      for (int k = 0; k < 8; ++k) e[k] *= sc;
      val = pack8_bf16(e);
    }
    tile[r * 32 + (cv ^ ((r >> 3) & 7))] = val;
  }
  __syncthreads();
  const int tg = tid & 7, vo = tid >> 3;
  uint4 rd[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) rd[k] = tile[(8 * tg + k) * 32 + (vo ^ tg)];
  const int gr = r0 + 8 * tg;
  if (gr >= rows_out) return;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int dc = c0 + 8 * vo + j;  // destination row
    if (dc >= cols) break;
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint4 x = rd[k];
      w[k] = (j >> 1) == 0 ? x.x : (j >> 1) == 1 ? x.y : (j >> 1) == 2 ? x.z : x.w;
    }
    uint4 o;
    o.x = __builtin_amdgcn_perm(w[1], w[0], sel);
    o.y = __builtin_amdgcn_perm(w[3], w[2], sel);
    o.z = __builtin_amdgcn_perm(w[5], w[4], sel);
    o.w = __builtin_amdgcn_perm(w[7], w[6], sel);
    *(uint4*)(dst + (int64_t)dc * ld_dst + gr) = o;
  }
}

hipError_t launch_transpose(Dt dt, const void* src, int rows, int cols, int64_t ld_src, void* dst,
                            int64_t ld_dst, int rows_out, hipStream_t s, const float* row_scale) {
  if (rows_out <= 0 || cols <= 0) return hipSuccess;
  if (dt == Dt::BF16 && cols % 8 == 0 && rows_out % 8 == 0 && ld_src % 8 == 0 && ld_dst % 8 == 0) {
    dim3 grid(cdiv(rows_out, 64), cdiv(cols, 256));
    hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(256), 0, s, (const uint16_t*)src, rows,
                       cols, ld_src, (uint16_t*)dst, ld_dst, rows_out, row_scale);
    return hipGetLastError();
  }
  dim3 grid(cdiv(rows_out, 64), cdiv(cols, 64));
  if (dt == Dt::BF16)
    hipLaunchKernelGGL(transpose_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)src, rows, cols,
                       ld_src, (bf16*)dst, ld_dst, rows_out, row_scale);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, s, (const float*)src, rows,
                       cols, ld_src, (float*)dst, ld_dst, rows_out, row_scale);
  return hipGetLastError();
}

// ------------------------------------------------------------- finalize ---
// Block of 8 rows x 128 slices of the partial tiles (tile-major layout:
// the 8 rows of a slice read 32 contiguous bytes); 8 rows per block puts a
// 2048-row chunk on 256 blocks, one per compute unit.  Three passes over the
// row's partials, each a parallel reduction over the slices:
//   1. m = max_j m_j and the argmax of the first tile reaching it (tiles
//      are in column order, so this is the lowest column index);
//   2. sum = sum_j s_j exp(m_j - m), lse = m + ln sum (the merge of
//      online-softmax states: each partial sum rescaled to the common max);
//   3. alpha_j = s valid exp(m_j - lse), overwriting m_j.
// A tile whose sum is zero holds no column (or only -inf logits) and is
// skipped; a NaN sum (a NaN or +inf logit in the tile) is not, so it
// reaches the row's lse, loss and gradients as NaN.
// ROWS rows per block, 1024 / ROWS slices of each row's partials per row:
// 8 x 128 for long rows (a 128256-word vocabulary has 1002 partial tiles),
// 32 x 32 for rows of at most 256 tiles, which otherwise leave most slices
// idle and spend the block's time in three 128-slice tree reductions.
template <int ROWS>
__global__ void __launch_bounds__(1024) finalize_kernel(FinalizeArgs a) {
  constexpr int kFinRows = ROWS, kFinSlices = 1024 / ROWS, kFinCache = 8;
  __shared__ float s_f[kFinSlices][kFinRows + 1];
  __shared__ float s_c[kFinSlices][kFinRows + 1];
  __shared__ int s_i[kFinSlices][kFinRows + 1];
  __shared__ float s_m[kFinRows], s_k[kFinRows], s_sc[kFinRows], s_beta[kFinRows];
  __shared__ float s_dzt[kFinRows];
  __shared__ int s_yl[kFinRows];
  __shared__ double s_nll[kFinRows];
  const int rl = threadIdx.x % kFinRows, sl = threadIdx.x / kFinRows;
  // a partial array row of 32 tokens (one 128-byte line) spans 32 / ROWS
  // row blocks: keep them on one XCD so the line is fetched into one L2
  const int rb = xcd_local_block();
  const int row = rb * kFinRows + rl;
  const bool live = row < a.M;
  // The first kFinCache tiles of this slice (all of them up to
  // kFinCache * kFinSlices tiles: 1024 with 8 rows per block) are
  // read once, all loads in flight together, and kept in registers for the
  // three passes; tiles beyond are read again by each pass.
  float cm[kFinCache], cs[kFinCache];
  int ca[kFinCache];
#pragma unroll
  for (int q = 0; q < kFinCache; ++q) {
    const int j = sl + q * kFinSlices;
    cm[q] = kNegInf;
    cs[q] = 0.f;
    ca[q] = 0x7fffffff;
    if (live && j < a.nt) {
      const int64_t o = (int64_t)j * a.ldr + row;
      cm[q] = a.pm[o];
      cs[q] = a.ps[o];
      ca[q] = a.pa[o];
    }
  }
  // pass 1: max and argmax
  float m = kNegInf;
  int am = 0x7fffffff;
#pragma unroll
  for (int q = 0; q < kFinCache; ++q)
    if (cs[q] != 0.f && (cm[q] > m || (cm[q] == m && ca[q] < am))) {
      m = cm[q];
      am = ca[q];
    }
  if (live)
    for (int j = sl + kFinCache * kFinSlices; j < a.nt; j += kFinSlices) {
      const int64_t o = (int64_t)j * a.ldr + row;
      const float mj = a.pm[o];
      if (a.ps[o] != 0.f && (mj > m || (mj == m && a.pa[o] < am))) {
        m = mj;
        am = a.pa[o];
      }
    }
  s_f[sl][rl] = m;
  s_i[sl][rl] = am;
  __syncthreads();
  // tree over the slices: slice sl takes in slice sl + w (the combine is
  // commutative: larger max, then lower index), then writes its own slot
  for (int w = kFinSlices / 2; w > 0; w >>= 1) {
    if (sl < w) {
      const float mk = s_f[sl + w][rl];
      const int ak = s_i[sl + w][rl];
      if (mk > m || (mk == m && ak < am)) {
        m = mk;
        am = ak;
      }
      s_f[sl][rl] = m;
      s_i[sl][rl] = am;
    }
    __syncthreads();
  }
  if (sl == 0) {
    s_m[rl] = m;
    if (live && a.argmax_out) a.argmax_out[row] = am == 0x7fffffff ? am : am + (int)a.y_shift;
  }
  __syncthreads();
  // The stored exponentials of tile j are relative to 2^k_j, k_j =
  // ref_power(m_j) (0 for an all -inf tile), exactly as the logits epilogue
  // computed it; K = ref_power(m) is the largest k_j.
  auto kq_of = [](float mj) { return mj == kNegInf ? 0.f : ref_power(mj); };
  // pass 2: sum = sum_j s_j 2^(k_j - K) (exact power-of-two rescaling)
  // (soft targets: also sum_j alpha_q_j pc_j = sum_v q_v z_v / tau)
  m = s_m[rl];
  const float K = kq_of(m);
  float sum = 0.f, cr = 0.f;
#pragma unroll
  for (int q = 0; q < kFinCache; ++q) {
    const int j = sl + q * kFinSlices;
    if (cs[q] != 0.f) sum += cs[q] * __builtin_amdgcn_exp2f(kq_of(cm[q]) - K);
    if (a.cross_pc && live && j < a.nt) {
      const int64_t o = (int64_t)j * a.ldr + row;
      cr += a.cross_pc[o] * a.alpha_q[o];
    }
  }
  if (live)
    for (int j = sl + kFinCache * kFinSlices; j < a.nt; j += kFinSlices) {
      const int64_t o = (int64_t)j * a.ldr + row;
      const float sj = a.ps[o];
      if (sj != 0.f) sum += sj * __builtin_amdgcn_exp2f(kq_of(a.pm[o]) - K);
      if (a.cross_pc) cr += a.cross_pc[o] * a.alpha_q[o];
    }
  s_f[sl][rl] = sum;
  s_c[sl][rl] = cr;
  __syncthreads();
  for (int w = kFinSlices / 2; w > 0; w >>= 1) {  // fixed-order tree sum
    if (sl < w) {
      sum += s_f[sl + w][rl];
      cr += s_c[sl + w][rl];
      s_f[sl][rl] = sum;
      s_c[sl][rl] = cr;
    }
    __syncthreads();
  }
  if (sl == 0) {
    double nll = 0.0;
    float lse = 0.f, beta = 0.f, sc = 0.f;
    if (live) {
      // validity against the whole vocabulary; ownership of the target by
      // these columns (all of them unless this is a vocabulary shard)
      const int64_t yt = a.y[row];
      const bool valid = target_valid(yt, a.ignore_index, a.v_total);
      const int64_t yl = yt - a.y_shift;
      const bool owned = valid && !a.no_target && yl >= 0 && yl < a.V;
      // lse = ln(2^K sum) = (K + log2 sum) ln 2
      lse = a.lse_in ? a.lse_in[row] : (K + __builtin_amdgcn_logf(sum)) * kLn2;
      sc = valid ? (a.unit_scale ? 1.f : *a.scale) * a.alpha_mul : 0.f;
      // probability of column v in tile j: P_v 2^(k_j - K) beta / sc, beta =
      // sc 2^K e^-lse (= sc / sum when lse is this call's own)
      if (sc != 0.f)
        beta = a.lse_in ? sc * __builtin_amdgcn_exp2f(K - a.lse_in[row] * kLog2e) : sc / sum;
      const float zt = owned ? a.ztgt[row] : 0.f;
      const float dzt = owned ? sc * (exp_fast(zt - lse) - 1.f) : 0.f;
      if (a.backward) a.dzt[row] = dzt;
      if (a.beta) a.beta[row] = beta;
      s_dzt[rl] = dzt;
      s_yl[rl] = owned ? (int)yl : -1;
      if (a.lse_out) a.lse_out[row] = lse;
      if (a.logprob_out) a.logprob_out[row] = valid ? zt - lse : 0.f;
      if (a.m_out) a.m_out[row] = m;
      // relative to the max itself: sum_v exp(z_v - m) = sum 2^(K - m log2 e)
      if (a.sum_out) a.sum_out[row] = sum * __builtin_amdgcn_exp2f(K - m * kLog2e);
      if (a.zt_out) a.zt_out[row] = zt;
      // hard target: lse - z_y; soft targets: lse - sum_v q_v z_v / tau
      nll = valid ? (double)lse - (double)(a.cross_pc ? cr : zt) : 0.0;
    }
    s_k[rl] = K;
    s_sc[rl] = sc;
    s_beta[rl] = beta;
    s_nll[rl] = nll;
  }
  __syncthreads();
  // pass 3 (only when the gradient follows): alpha_j = beta 2^(k_j - K),
  // the factor taking tile j's stored exponentials to s valid softmax.
  // With dZ formed inside the contractions (shift non-null) the rows'
  // exponentials are brought to 2^K by the row-reference pass instead: the
  // shift byte of tile j is K - k_j (255 for 255 and more: the tile flushes
  // to zero; 0 for rows with no scale), and alpha_j = beta for every tile.
  if (live && a.backward) {
    const float Kr = s_k[rl], beta = s_beta[rl], sc = s_sc[rl];
    auto put = [&](int j, float mj, float sj) {
      const int64_t o = (int64_t)j * a.ldr + row;
      const float kj = kq_of(mj);
      if (a.shift) {
        a.pm[o] = (sj != 0.f) ? beta : 0.f;
        a.shift[(int64_t)row * a.ld_shift + j] =
            (uint8_t)((sj != 0.f && beta != 0.f) ? __builtin_fminf(Kr - kj, 255.f) : 0.f);
      } else {
        a.pm[o] = (sj != 0.f) ? beta * __builtin_amdgcn_exp2f(kj - Kr) : 0.f;
      }
      if (a.alpha_q) a.alpha_q[o] *= sc;
    };
#pragma unroll
    for (int q = 0; q < kFinCache; ++q) {
      const int j = sl + q * kFinSlices;
      if (j < a.nt) put(j, cm[q], cs[q]);
    }
    for (int j = sl + kFinCache * kFinSlices; j < a.nt; j += kFinSlices)
      put(j, a.pm[(int64_t)j * a.ldr + row], a.ps[(int64_t)j * a.ldr + row]);
  }
  if (a.shift && a.backward && live && sl == 0) {
    // The target's column will hold round(dzt / beta) (the row-reference
    // pass writes it), so that beta times it is the target's dZ for the dW
    // contraction; corr = dzt - beta round(dzt / beta) is what the dX
    // contraction adds to it (times W's target row).  A row whose beta is 0
    // with a target (a non-finite sum) keeps corr = dzt, NaN or not.
    const int yl = s_yl[rl];
    const float beta = s_beta[rl], dzt = s_dzt[rl];
    float c = 0.f, q = 0.f;
    int col = -1;
    if (yl >= 0) {
      if (beta != 0.f) {
        q = dzt / beta;
        if (a.round_bf16) q = Elem<bf16>::to_f32(Elem<bf16>::from_f32(q));
        c = dzt - beta * q;
        col = yl;
      } else {
        c = dzt;
      }
    }
    a.corr[row] = c;
    a.tcol[row] = col;
    a.tval[row] = q;
  }
  if (threadIdx.x == 0 && a.loss_part) {
    double total = 0.0;
    for (int k = 0; k < kFinRows; ++k) total += s_nll[k];
    a.loss_part[rb] = a.first_chunk ? total : a.loss_part[rb] + total;
  }
}

hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.block_rows == 32)
    hipLaunchKernelGGL(finalize_kernel<32>, dim3(cdiv(a.M, 32)), dim3(1024), 0, s, a);
  else if (a.block_rows == 8)
    hipLaunchKernelGGL(finalize_kernel<8>, dim3(cdiv(a.M, 8)), dim3(1024), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ------------------------------------------------------- row reference ---
// With dZ formed inside the contractions: brings every row of P to its
// row's reference (a 128-column segment whose tile reference lies below it
// is rewritten as P 2^-s, s being the merge's shift byte) and writes the
// target's column as the merge's tval.  One wave per row: the row's shift
// bytes come in one 16-byte load per lane (tiles 16 l .. 16 l + 15, up to
// 1024 tiles; beyond, the wave reads them again per 1024), staged in LDS.
// A row whose tiles all share its reference is left as it is; otherwise the
// wave streams the row, 16 bytes per lane and four loads in flight, and
// rewrites the vectors of the tiles that change.  The target's column is
// written last, after the wave's stores have completed.
template <typename T>
__global__ void __launch_bounds__(256) rowref_kernel(RowRefArgs a) {
  constexpr int EPV = Elem<T>::kVec;
  constexpr int VPT = kPartialWidth / EPV;  // 16-byte vectors per tile
  __shared__ uint8_t s_sh[4][1024];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= a.M) return;  // wave-uniform
  T* const prow = (T*)a.P + (int64_t)t * a.ldp;
  const uint8_t* const srow = a.shift + (int64_t)t * a.ld_shift;
  for (int j0 = 0; j0 < a.nt; j0 += 1024) {
    const int nj = min(1024, a.nt - j0);
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    if (16 * lane < nj) w = *(const uint4*)(srow + j0 + 16 * lane);
    // bytes of tiles past nt are padding: cleared
    const int valid = min(16, max(0, nj - 16 * lane));
    uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int b = 0; b < 16; ++b)
      if (b >= valid) wd[b >> 2] &= ~(0xffu << (8 * (b & 3)));
    const bool mine = (wd[0] | wd[1] | wd[2] | wd[3]) != 0;
    if (!__builtin_amdgcn_ballot_w64(mine)) continue;  // the row keeps these tiles
    *(uint4*)&s_sh[wv][16 * lane] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    __builtin_amdgcn_wave_barrier();
    // vectors q of tiles j0 .. j0 + nj - 1, lane-strided, four at a time
    const int nvec = nj * VPT;
    uint4* const base = (uint4*)(prow + (int64_t)j0 * kPartialWidth);
    for (int q0 = lane; q0 < nvec; q0 += 4 * 64) {
      uint4 v[4];
      int sb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int q = q0 + 64 * u;
        sb[u] = q < nvec ? s_sh[wv][q / VPT] : 0;
        if (sb[u] != 0) v[u] = base[q];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (sb[u] == 0) continue;
        T* const e = (T*)&v[u];
#pragma unroll
        for (int k = 0; k < EPV; ++k)
          e[k] = Elem<T>::from_f32(__builtin_ldexpf(Elem<T>::to_f32(e[k]), -sb[u]));
        base[q0 + 64 * u] = v[u];
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  const int tc = a.tcol[t];
  if (lane == 0 && tc >= 0) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's rewrite of the tile has landed
    __threadfence_block();
    prow[tc] = Elem<T>::from_f32(a.tval[t]);
  }
}

hipError_t launch_rowref(Dt dt, const RowRefArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.V <= 0) return hipSuccess;
  if (a.ld_shift % 16 != 0 || a.ld_shift < a.nt) return hipErrorInvalidValue;
  const dim3 grid(cdiv(a.M, 4));
  if (dt == Dt::BF16)
    hipLaunchKernelGGL(rowref_kernel<bf16>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(rowref_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- fixup ---
// dZ = alpha_tile * exp(z - m_tile) except on the target column, where the
// exact s (p_y - 1) from the fp32 target logit is used; written in place and
// transposed.  64 x 64 tiles; a 64-column tile never straddles a partial.
template <typename T>
__global__ void __launch_bounds__(256) fixup_kernel(FixupArgs a) {
  constexpr int EPV = Elem<T>::kVec;
  constexpr int VPR = 64 / EPV;
  constexpr int PER = 64 * VPR / 256;
  __shared__ T tile[64][64 + 2];
  const int v0 = blockIdx.x * 64, t0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  T* P = (T*)a.P;
  T* Pt = (T*)a.Pt;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int q = tid + 256 * p;
    const int r = q / VPR, cv = q % VPR;
    const int t = t0 + r, v = v0 + cv * EPV;
    float d[EPV];
#pragma unroll
    for (int k = 0; k < EPV; ++k) d[k] = 0.f;
    if (t < a.M) {
      T* src = P + (int64_t)t * a.ldp + v;
      uint4 pv = *(const uint4*)src;
      const T* pe = (const T*)&pv;
      const float al = (v < a.V) ? a.alpha[(int64_t)(v / kPartialWidth) * a.ldr + t] : 0.f;
      const int64_t yt = a.y[t];
      const int64_t yl = yt - a.y_shift;  // target's column among these V
      const bool owned = yt != a.ignore_index && yl >= 0 && yl < a.V;
#pragma unroll
      for (int k = 0; k < EPV; ++k) d[k] = (v + k < a.V) ? al * Elem<T>::to_f32(pe[k]) : 0.f;
      if (a.Pq) {  // soft targets: minus the teacher's probability, same scale
        uint4 qv = *(const uint4*)((const T*)a.Pq + (int64_t)t * a.ldp + v);
        const T* qe = (const T*)&qv;
        const float aq = (v < a.V) ? a.alpha_q[(int64_t)(v / kPartialWidth) * a.ldr + t] : 0.f;
#pragma unroll
        for (int k = 0; k < EPV; ++k)
          d[k] = (v + k < a.V) ? d[k] - aq * Elem<T>::to_f32(qe[k]) : 0.f;
      }
      if (owned && !a.no_target && yl >= v && yl < v + EPV) d[yl - v] = a.dzt[t];
      uint4 ov;
      T* oe = (T*)&ov;
#pragma unroll
      for (int k = 0; k < EPV; ++k) oe[k] = Elem<T>::from_f32(d[k]);
      if (a.write_rows) *(uint4*)src = ov;
#pragma unroll
      for (int k = 0; k < EPV; ++k) tile[r][cv * EPV + k] = oe[k];
    } else {
#pragma unroll
      for (int k = 0; k < EPV; ++k) tile[r][cv * EPV + k] = Elem<T>::from_f32(0.f);
    }
  }
  if (!a.write_t) return;  // block-uniform
  __syncthreads();
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int q = tid + 256 * p;
    const int c = q / VPR, rv = q % VPR;
    const int v = v0 + c, t = t0 + rv * EPV;
    if (v >= a.Vpad || t >= a.rows_out) continue;
    uint4 val;
    T* e = (T*)&val;
#pragma unroll
    for (int k = 0; k < EPV; ++k) e[k] = tile[rv * EPV + k][c];
    *(uint4*)(Pt + (int64_t)v * a.ldpt + t) = val;
  }
}

// bf16 fixup with a wider tile: 64 tokens x 256 columns per block.  Each
// thread forms eight 8-column vectors of dZ (written back in place and into
// LDS), then transposes one 8 x 8 block (8 tokens x 8 columns) in registers
// and writes eight 16-byte dZ^T segments; the 8 threads with the same column
// octet write one 128-byte run of a dZ^T row.  LDS rows are 512 bytes with
// the 16-byte slot XOR-swizzled by the row's token group (row / 8), which
// keeps both the row-wise writes and the transposing reads free of bank
// conflicts.
constexpr int kFixT = 64, kFixV = 256;
__global__ void __launch_bounds__(256) fixup_bf16_kernel(FixupArgs a) {
  __shared__ uint4 tile[kFixT * (kFixV / 8)];  // 32 KB
  const int v0 = blockIdx.x * kFixV, t0 = blockIdx.y * kFixT;
  const int tid = threadIdx.x;
  uint16_t* const P = (uint16_t*)a.P;
  uint16_t* const Pt = (uint16_t*)a.Pt;
  // phase 1: row r = tid / 32 + 8 p, column octet cv = tid % 32.  The eight
  // rows' loads go out first (rows past M read row 0 and columns past V tile
  // 0's partials: in bounds, their values unused), then the rows are formed,
  // and the row stores come last, so that no store stands between loads the
  // compiler may not move across it.
  const int cv = tid & 31;
  const int v = v0 + cv * 8;
  const bool vlive = v < a.V;
  const int64_t aoff = vlive ? (int64_t)(v / kPartialWidth) * a.ldr : 0;
  uint4 pv[8];
  float al[8];
  int64_t yt[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int t = t0 + (tid >> 5) + 8 * p;
    const int tc = t < a.M ? t : 0;
    pv[p] = *(const uint4*)(P + (int64_t)tc * a.ldp + v);
    al[p] = a.alpha[aoff + tc];
    yt[p] = a.y[tc];
  }
  uint4 ov[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int r = (tid >> 5) + 8 * p;
    const int t = t0 + r;
    const bool live = t < a.M;
    float d[8];
    unpack8_bf16(pv[p], d);
    const float alp = (live && vlive) ? al[p] : 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) d[k] = (v + k < a.V) ? alp * d[k] : 0.f;
    if (a.Pq) {  // soft targets: minus the teacher's probability, same scale
      const int tc = live ? t : 0;
      float q[8];
      unpack8_bf16(*(const uint4*)((const uint16_t*)a.Pq + (int64_t)tc * a.ldp + v), q);
      const float aq = (live && vlive) ? a.alpha_q[aoff + tc] : 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) d[k] = (v + k < a.V) ? __builtin_fmaf(-aq, q[k], d[k]) : 0.f;
    }
    const int64_t yl = yt[p] - a.y_shift;
    if (live && !a.no_target && yt[p] != a.ignore_index && yl >= v && yl < v + 8 && yl < a.V) {
      const float dz = a.dzt[t];
#pragma unroll
      for (int k = 0; k < 8; ++k) d[k] = (yl == v + k) ? dz : d[k];
    }
    ov[p] = pack8_bf16(d);
    if (a.write_t) tile[r * 32 + (cv ^ ((r >> 3) & 7))] = ov[p];
  }
  if (a.write_rows) {
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int t = t0 + (tid >> 5) + 8 * p;
      if (t < a.M) *(uint4*)(P + (int64_t)t * a.ldp + v) = ov[p];
    }
  }
  if (!a.write_t) return;  // block-uniform: dZ only
  __syncthreads();
  // phase 2: token group tg = tid % 8, column octet vo = tid / 8
  const int tg = tid & 7, vo = tid >> 3;
  uint4 rd[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) rd[k] = tile[(8 * tg + k) * 32 + (vo ^ tg)];
  const int t = t0 + 8 * tg;
  if (t < a.rows_out) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // element j of each token's vector: dword j / 2, half j % 2
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
      uint32_t w[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint4 x = rd[k];
        w[k] = (j >> 1) == 0 ? x.x : (j >> 1) == 1 ? x.y : (j >> 1) == 2 ? x.z : x.w;
      }
      uint4 o;
      o.x = __builtin_amdgcn_perm(w[1], w[0], sel);
      o.y = __builtin_amdgcn_perm(w[3], w[2], sel);
      o.z = __builtin_amdgcn_perm(w[5], w[4], sel);
      o.w = __builtin_amdgcn_perm(w[7], w[6], sel);
      *(uint4*)(Pt + (int64_t)(v0 + 8 * vo + j) * a.ldpt + t) = o;
    }
  }
}

hipError_t launch_fixup(Dt dt, const FixupArgs& a, hipStream_t s) {
  if (a.rows_out <= 0) return hipSuccess;
  if (!a.write_rows && !a.write_t) return hipSuccess;
  if (dt == Dt::BF16) {
    // Vpad is a multiple of 256 and rows_out of 64: the grid covers them exactly
    dim3 grid(cdiv(a.Vpad, kFixV), cdiv(a.rows_out, kFixT));
    hipLaunchKernelGGL(fixup_bf16_kernel, grid, dim3(256), 0, s, a);
  } else {
    dim3 grid(cdiv(a.Vpad, 64), cdiv(a.rows_out, 64));
    hipLaunchKernelGGL(fixup_kernel<float>, grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

// -------------------------------------------------------- split-K reduce ---
template <typename T>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* __restrict__ part, int splits,
                                                            int64_t stride, int M, int N,
                                                            T* __restrict__ out, int64_t ldo,
                                                            DxFuse f, bool fused) {
  const int64_t idx = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  const int64_t total = (int64_t)M * N;
  if (idx >= total) return;
  const int row = (int)(idx / N), col = (int)(idx % N);  // N % 4 == 0
  f4 s = *(const f4*)(part + idx);
  for (int k = 1; k < splits; ++k) s += *(const f4*)(part + (int64_t)k * stride + idx);
  if (fused) {
    // dZ formed inside the contraction: the row scale and the target's term
    const float cr = f.corr[row];
    s *= f.beta[row];
    if (cr != 0.f) {
      const int64_t yl = f.y[row] - f.y_shift;
      if (yl >= 0 && yl < f.V) s += load4((const T*)f.W + yl * f.ldw + col) * cr;
    }
  }
  store4(out + (int64_t)row * ldo + col, s);
}

hipError_t launch_splitk_reduce(Dt dt, const float* part, int splits, int64_t stride, int M, int N,
                                void* out, int64_t ldo, hipStream_t s, const DxFuse* fuse) {
  const int64_t total = (int64_t)M * N / 4;
  if (total <= 0) return hipSuccess;
  dim3 grid(cdiv(total, 256));
  const DxFuse f = fuse ? *fuse : DxFuse{};
  if (dt == Dt::BF16)
    hipLaunchKernelGGL(splitk_reduce_kernel<bf16>, grid, dim3(256), 0, s, part, splits, stride, M,
                       N, (bf16*)out, ldo, f, fuse != nullptr);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<float>, grid, dim3(256), 0, s, part, splits, stride, M,
                       N, (float*)out, ldo, f, fuse != nullptr);
  return hipGetLastError();
}

// ----------------------------------------------------------------- loss ---
// Fixed-order float64 sum of the per-block NLL partials, then the mean's
// division by n_valid (0 when n_valid = 0).
__global__ void __launch_bounds__(256) loss_kernel(const double* __restrict__ part, int n,
                                                   const int64_t* __restrict__ n_valid,
                                                   int reduction_sum, float* loss) {
  __shared__ double s[256];
  double acc = 0.0;
  for (int i = threadIdx.x; i < n; i += 256) acc += part[i];
  s[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) s[threadIdx.x] += s[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const long long nv = *n_valid;
    double total = s[0];
    if (!reduction_sum) total = nv > 0 ? total / (double)nv : 0.0;
    *loss = (float)total;
  }
}

hipError_t launch_loss(const double* loss_part, int nparts, const int64_t* n_valid, int reduction_sum,
                       float* loss, hipStream_t s) {
  hipLaunchKernelGGL(loss_kernel, dim3(1), dim3(256), 0, s, loss_part, nparts, n_valid,
                     reduction_sum, loss);
  return hipGetLastError();
}

// ----------------------------------------------------------------- zero ---
__global__ void zero_kernel(uint32_t* p, size_t words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  size_t blocks = (words + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint32_t*)p, words);
  return hipGetLastError();
}

}  // namespace flce
