// Launch wrappers for the fused linear cross-entropy kernels.  Host code
// calls only these; every function enqueues on `stream` and returns the
// hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

enum class Dt { F32 = 0, BF16 = 1 };

// Tile shape of a GEMM launch: 256 x 256 blocks for large problems, 128 x 128
// when the 256 x 256 grid would leave compute units idle.
enum class TileCfg { T256 = 0, T128 = 1 };

struct LogitsArgs {
  const void* X;        // chunk rows, [M x H]
  const void* W;        // [V x H]
  int M, V, H;
  void* P;              // exp(z - m_tile), [M x ldp] in the input dtype; null: not stored
  int64_t ldp;
  float* pm;            // partial tile max         [nt x ldr], tile-major
  float* ps;            // partial tile sum of exp  [nt x ldr]
  int* pa;              // partial tile argmax      [nt x ldr]
  int64_t ldr;          // row stride of the partials (>= M)
  float* ztgt;          // logit of the target, [M]
  const int64_t* y;     // chunk targets, [M]
  int64_t ignore_index;
  int64_t y_shift;      // vocabulary id of W's row 0 (0 unless W is a vocabulary shard)
  float inv_temp = 1.f; // logits are divided by the softmax temperature
  // Soft targets: the teacher's exp(z_T / tau - m_tile) of the same chunk
  // ([M x ldp], input dtype) and, per (tile, row), sum_v P_T z / tau out.
  const void* Pq = nullptr;
  float* pc = nullptr;
};
// The stored exponentials of a (row, 128-column tile) are exp2(z log2(e) /
// tau - k) with k = 32 ceil(m log2(e) / 32), m the tile's max of z / tau:
// relative to a whole power of two, so that the factor taking them to
// probabilities is a per-row scale times 2^-s(row, tile) (see FinalizeArgs).
// Width in columns of one online-logsumexp partial (the wave tile width of
// the 256 x 256 logits GEMM).
constexpr int kPartialWidth = 128;

hipError_t launch_logits(Dt dt, const LogitsArgs& a, hipStream_t s);

// dX = dZ W with dZ formed inside the contraction: A is the chunk's stored
// exponentials P, brought to one reference per row by the row-reference
// pass (see FinalizeArgs), and the output row t is beta_t acc_t + corr_t
// W[y_t - y_shift] (the target term only when that row of W is in [0, V)).
struct DxFuse {
  const float* beta;
  const float* corr;
  const int64_t* y;   // chunk targets
  int64_t ignore_index;
  int64_t y_shift;
  int V;              // rows of W
  const void* W;      // [V x ldw], input dtype
  int64_t ldw;
};

struct GemmOutArgs {
  const void* A; int64_t lda;
  const void* B; int64_t ldb;
  int M, N, K;
  void* out; int64_t ldo;
  bool out_f32;           // store fp32 (dW, split-K partials) or the input dtype
  bool may_accumulate;    // fp32 only: the instantiation that can start from the
                          // output's old values (dW); `accumulate` picks per launch
  bool accumulate;        // out += result (requires may_accumulate)
  int splits;             // split-K factor; partial planes `split_stride` apart
  int64_t split_stride;
  // Optional scratch for the last partial round of a large accumulating
  // grid (dW): those tiles are split in K into fp32 partial tiles here and
  // summed, with the old output, by a second pass.  nullptr: never split.
  float* tail_part = nullptr;
  size_t tail_part_bytes = 0;
  // B as stored, K rows of N contiguous elements (ldb >= N), rather than
  // N x K: bf16 only, not accumulating, K * ldb * 2 < 2^31 bytes.
  bool b_stored = false;
  // A as stored, K rows of M contiguous elements (lda >= M), rather than
  // M x K: bf16 only, the accumulating fp32 store (dW), K * lda * 2 < 2^31
  // bytes; K need not be a multiple of 8 (rows past K read as zero).
  bool a_stored = false;
  // dX with dZ formed inside the contraction (not accumulating); with
  // splits > 1 the partial planes are raw and launch_splitk_reduce applies it.
  const DxFuse* fuse = nullptr;
};
hipError_t launch_gemm_store(Dt dt, TileCfg tc, const GemmOutArgs& a, hipStream_t s);

// part: scratch for per-block counts, 2 * kCountBlocks values (nullable: one
// block counts every target).
constexpr int kCountBlocks = 64;
hipError_t launch_count(const int64_t* y, int64_t T, int64_t ignore_index, int64_t V,
                        int reduction_sum, int64_t* n_valid, float* scale, int64_t* bad,
                        int64_t* n_valid_out, long long* part, hipStream_t s);

// dst[c][r] = src[r][c] for r < rows, 0 for rows <= r < rows_out; c < cols.
// row_scale (nullable, [rows]): each source row is multiplied by its entry
// on the way, rounded to the dtype.
hipError_t launch_transpose(Dt dt, const void* src, int rows, int cols, int64_t ld_src,
                            void* dst, int64_t ld_dst, int rows_out, hipStream_t s,
                            const float* row_scale = nullptr);

struct FinalizeArgs {
  int M, nt, V;
  int64_t ldr;           // row stride of the tile-major partials
  float* pm; const float* ps; const int* pa;   // pm is overwritten by alpha
  const float* ztgt;
  float* dzt;
  const int64_t* y; int64_t ignore_index;
  int64_t y_shift;       // vocabulary id of column 0 (shard offset; argmax_out adds it)
  int64_t v_total;       // whole vocabulary, for target validity
  const float* lse_in;   // nullable: the whole vocabulary's lse, given (shard backward)
  float* m_out;          // nullable: max over these columns
  float* sum_out;        // nullable: sum of exp(z - max) over these columns
  float* zt_out;         // nullable: target logit if these columns hold it, else 0
  // Soft targets: per (tile, row) cross partials of the student's logits
  // with the teacher's exponentials, and the teacher's alpha (its
  // exp(m_tile - lse), read for the cross term, then scaled like the
  // student's alpha for the dZ pass).
  const float* cross_pc = nullptr;
  float* alpha_q = nullptr;
  float alpha_mul = 1.f;     // extra factor of alpha (1 / temperature)
  bool unit_scale = false;   // alpha without the reduction's 1/n_valid (teacher)
  bool no_target = false;    // no one-hot term (soft targets, teacher)
  const float* scale;
  float* lse_out;        // nullable, chunk-relative
  int32_t* argmax_out;   // nullable, chunk-relative
  float* logprob_out;    // nullable, chunk-relative: z_target - lse (0 if ignored)
  bool backward;         // also form dzt and turn pm into alpha
  double* loss_part;     // one slot per block_rows rows; nullable
  int first_chunk;
  int block_rows = 8;    // finalize_rows(nt, C): 8 or 32
  // Backward with dZ formed inside the contractions (shift non-null): the
  // row-reference pass (RowRefArgs) then brings each row's stored
  // exponentials to one reference 2^K_t and sets the target's column, so that
  // dZ_tv = beta_t P_tv throughout; pm becomes beta for every tile (the
  // factor a dZ pass applies).  Per row or (tile, row):
  //   shift [M x ld_shift] K_t - k_tj as a byte (255: 255 or more, the
  //                    tile flushes to zero; 0: as it is), row-major
  //   beta  [M]  the row scale
  //   corr  [M]  dzt_t - beta_t tval_t: what the dX contraction adds times
  //              W's target row (0 when the target is ignored or not in
  //              these columns)
  //   tcol, tval [M]  the target's column (-1: none) and its value
  //              round(dzt_t / beta_t) in the input dtype (round_bf16)
  uint8_t* shift = nullptr;
  int64_t ld_shift = 0;       // >= nt, a multiple of 16
  float* beta = nullptr;
  float* corr = nullptr;
  int* tcol = nullptr;
  float* tval = nullptr;
  bool round_bf16 = false;
};

struct RowRefArgs {
  void* P; int64_t ldp;  // [M x ldp], the input dtype
  int M, V, nt;
  const uint8_t* shift;  // [M x ld_shift], 16-byte aligned rows
  int64_t ld_shift;      // a multiple of 16, >= nt
  const int* tcol;
  const float* tval;
};
hipError_t launch_rowref(Dt dt, const RowRefArgs& a, hipStream_t s);
// Rows per finalize block, hence rows per loss partial: 32 when rows hold
// at most 256 partial tiles and a chunk of C rows still gives 256 blocks,
// else 8.  kFinalizeRows is the smaller, which sizes the partial buffer.
constexpr int kFinalizeRows = 8;
inline int finalize_rows(int64_t nt, int64_t C) { return nt <= 256 && C >= 8192 ? 32 : 8; }
hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t s);

struct FixupArgs {
  void* P; int64_t ldp;          // in: exp(z - m_tile); out: dZ (in place)
  void* Pt; int64_t ldpt;        // out: dZ^T, [Vpad x ldpt] (unused without write_t)
  int M;                         // valid rows
  int rows_out;                  // rows written to Pt (zero beyond M)
  int V, Vpad, nt;
  int64_t ldr;
  const float* alpha;            // [nt x ldr], tile-major
  const float* dzt;              // [M]
  const int64_t* y; int64_t ignore_index;
  int64_t y_shift;               // vocabulary id of column 0 (shard offset)
  bool no_target = false;        // soft targets: no one-hot column

  const void* Pq = nullptr;      // soft targets: teacher exponentials, subtracted
  const float* alpha_q = nullptr;  //   with this scale, [nt x ldr]
  bool write_rows = true;        // false: only dZ^T is written (P keeps the exponentials)
  bool write_t = true;           // false: only dZ is written (dW reads it as stored)
};
hipError_t launch_fixup(Dt dt, const FixupArgs& a, hipStream_t s);

hipError_t launch_splitk_reduce(Dt dt, const float* part, int splits, int64_t stride, int M,
                                int N, void* out, int64_t ldo, hipStream_t s,
                                const DxFuse* fuse = nullptr);

hipError_t launch_loss(const double* loss_part, int nparts, const int64_t* n_valid,
                       int reduction_sum, float* loss, hipStream_t s);

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

// Dynamic LDS opt-in for the GEMM kernels (call once per process/device).
hipError_t gemm_setup();

}  // namespace flce
