/*
 * flce.h -- fused linear cross-entropy head for AMD Instinct MI355X (gfx950).
 *
 * One call computes, for hidden states X (T x H), an lm_head weight W (V x H,
 * nn.Linear layout) and integer targets y:
 *
 *   z      = X W^T                          logits, never stored whole
 *   lse_t  = logsumexp_v z_tv
 *   loss   = sum_t valid_t (lse_t - z_{t,y_t})  [ / n_valid for the mean ]
 *   dZ_tv  = s valid_t (softmax(z_t)_v - [v = y_t]),  s = 1/n_valid or 1
 *   dX     = dZ W          dW = dZ^T X
 *
 * Sources: the softmax+CE gradient (p - onehot) from "Alisa's book of LLMs",
 * section "gradient of softmax + CE loss"; the masked mean with an ignore
 * (padding) index from its "Information theory > implementing the loss"; the
 * stable and online logsumexp from its "Numerical stability and other
 * tricks"; and the fused structure -- per token chunk the three matmuls run
 * inside the forward, so the gradients are finished when the scalar loss
 * returns and the T x V logits are never materialised -- from the
 * efficient-llm-anatomy README, "Selected insights > Fused cross-entropy
 * computes backward during forward".
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller, row-major and
 *    contiguous, 16-byte aligned.  The library never frees them.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    All device work is enqueued on it; flce_fwd_bwd never synchronises.
 *  - Every function returns a status; on an argument error nothing is
 *    enqueued and no output is touched.
 *  - A handle is bound to the device that was current at flce_create and
 *    must be used with that device current.  A handle is not thread-safe and
 *    calls that share a handle must be ordered (one stream per handle, or
 *    external synchronisation): the workspace is reused by every call.
 */
#ifndef FLCE_H
#define FLCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FLCE_OK = 0,
  FLCE_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad size or enum   */
  FLCE_ERR_UNSUPPORTED = 2,      /* valid request this build does not implement */
  FLCE_ERR_HIP = 3,              /* a HIP runtime call failed                    */
  FLCE_ERR_OUT_OF_MEMORY = 4,    /* workspace allocation failed                  */
  FLCE_ERR_BAD_TARGET = 5        /* (flce_query_error) targets outside [0, V)    */
} flce_status_t;

/* Element type of X, W and dX.  dW, loss and lse are always float32. */
typedef enum { FLCE_F32 = 0, FLCE_BF16 = 1 } flce_dtype_t;

/* Reduction of the per-token losses.  There is no "none": the fused
 * backward needs a scalar loss whose gradient seed is 1 ("Alisa's book of
 * LLMs", Backpropagation: backward starts from a scalar seeded with 1). */
typedef enum { FLCE_MEAN = 1, FLCE_SUM = 2 } flce_reduction_t;

typedef struct {
  int64_t hidden;       /* H: > 0, multiple of 8 (bf16) or 4 (fp32)          */
  int64_t vocab;        /* V: > 0                                              */
  int32_t dtype;        /* flce_dtype_t                                        */
  int32_t dw_chunks;    /* G: chunks whose exponentials, dZ or dZ^T are kept for
                           one dW GEMM of depth K = G*C; 0 = default (1), at
                           most 8.  The dW tiles are then read and written
                           once per G chunks instead of once per chunk, for
                           about (G-1)*C*V more workspace elements.            */
  int64_t chunk_tokens; /* C: tokens per chunk; 0 = default (4096).  Rounded up
                           to a multiple of 256.  The workspace is O(G*C*V +
                           V*H) (O((1+G)*C*V + V*H) where dZ^T is written;
                           the soft-target call adds C*V for the teacher) and
                           does not depend on the number of tokens T.          */
  int32_t flags;        /* 0, or any of FLCE_FLAG_NO_WEIGHT_COPY, FLCE_FLAG_DZ_IN_PLACE and
                           FLCE_FLAG_FORWARD_ONLY                             */
} flce_config_t;

/* The dX GEMM reads W in its stored [V x H] layout instead of a transposed
 * copy made at every call: the workspace shrinks by H*V*2 bytes and the
 * per-call transpose goes away, for a dX GEMM that runs 8-12 % slower
 * (its LDS reads of W are transposing 8-byte reads).  bf16 only, and
 * V*H*2 must stay below 2^31 bytes; FLCE_ERR_UNSUPPORTED otherwise. */
#define FLCE_FLAG_NO_WEIGHT_COPY 1

/* How dZ reaches the dX and dW contractions ("gradient of softmax + CE loss"
 * in "Alisa's book of LLMs": dZ = p - onehot).  By default dZ is formed
 * inside them and never written: the logits epilogue stores each (row,
 * 128-column tile) of exponentials relative to a power of two 2^(32 j); a
 * small pass after the merge rewrites, in place, the tiles whose power lies
 * below their row's (so a row's exponentials share one, dZ = beta P) and
 * sets the target's column; the dX GEMM reads the exponentials and finishes
 * each output row with the row's scale and the target's correction times
 * that row of W, and the dW GEMM reads them as stored against X^T scaled by
 * the row scales.  With this flag a pass writes dZ over the exponentials
 * and both GEMMs read it (one more T*V write; measured ~3 % slower per call
 * at 16384 x 4096 x 128256, and faster where many rows' tiles sit far below
 * their row's reference, as with a few far-outlying rows of W).  Same
 * results to the tolerances.  The soft-target call always writes dZ (its
 * rows hold two sets of exponentials).  Either way the dW GEMM reads P --
 * exponentials or dZ -- as stored where the dtype is bf16, H <= 4096 and
 * G*C*Vpad*2 < 2^31 bytes (Vpad = V rounded up to 256); elsewhere the pass
 * also writes dZ^T for it. */
#define FLCE_FLAG_DZ_IN_PLACE 2

/* The handle serves only the forward-only calls (flce_forward and
 * flce_vocab_shard_forward): its workspace holds the merge's partials, about
 * 12*ceil(V/128)*C bytes, and a few small buffers -- no exponentials, no
 * W^T, nothing of the backward -- so large chunks cost little memory.
 * flce_fwd_bwd, flce_vocab_shard_backward and flce_fwd_bwd_noalloc return
 * INVALID_ARGUMENT for it with nothing enqueued, and flce_distill_create
 * refuses it (the soft-target call has no forward-only form). */
#define FLCE_FLAG_FORWARD_ONLY 4

typedef struct flce_handle* flce_handle_t;

/* Create a handle for fixed (H, V, dtype, C, G, flags) on the current HIP
 * device and allocate its workspace.  Returns INVALID_ARGUMENT for a bad
 * config (unknown flag bits included) and UNSUPPORTED when H, V rounded up to
 * a multiple of 256, or G*C exceeds 2^20, or FLCE_FLAG_NO_WEIGHT_COPY is
 * asked for fp32 or for V*H*2 >= 2^31 bytes (no device call is made in any
 * of these cases), OUT_OF_MEMORY / HIP if allocation fails.  *out is set to
 * NULL on failure. */
flce_status_t flce_create(const flce_config_t* cfg, flce_handle_t* out);

/* Bytes of device workspace the handle owns (independent of T). */
size_t flce_workspace_bytes(flce_handle_t h);

/* Tokens per chunk after rounding (C). */
int64_t flce_chunk_tokens(flce_handle_t h);

/* Chunks per dW GEMM (G), after applying the default. */
int32_t flce_dw_chunks(flce_handle_t h);

/*
 * Fused forward + backward of the linear cross-entropy head.
 *
 *   X        [T x H]  dtype          hidden states (device)
 *   W        [V x H]  dtype          lm_head weight (device)
 *   targets  [T]      int64          target ids (device)
 *   T        >= 0                    number of tokens (T = 0 is valid)
 *   ignore_index                     tokens whose target equals it are
 *                                    excluded (it may be a real vocab id)
 *   reduction                        FLCE_MEAN or FLCE_SUM
 * Outputs (device, overwritten, never accumulated):
 *   loss     [1]      float32        the reduced loss (required)
 *   dX       [T x H]  dtype          gradient wrt X for grad_output = 1 (required)
 *   dW       [V x H]  float32        gradient wrt W for grad_output = 1 (required)
 *   lse      [T]      float32        per-token logsumexp (nullable)
 *   argmax   [T]      int32          per-token argmax of z, lowest index on
 *                                    ties (nullable)
 *   n_valid  [1]      int64          number of non-ignored tokens (nullable)
 *
 * Mean with n_valid = 0 gives loss 0 and zero gradients.  A target that is
 * neither ignore_index nor in [0, V) is treated as ignored and counted on
 * the device; flce_query_error reports it.  dW and dX must not alias X, W or
 * each other.  Returns without enqueuing anything on an argument error.
 */
flce_status_t flce_fwd_bwd(flce_handle_t h, const void* X, const void* W,
                           const int64_t* targets, int64_t T, int64_t ignore_index,
                           int32_t reduction, float* loss, void* dX, float* dW,
                           float* lse, int32_t* argmax, int64_t* n_valid,
                           void* stream);

/*
 * Forward only: per-token log-probabilities of the targets and the reduced
 * loss, without gradients (evaluation; the token log-prob ratios of
 * policy-gradient methods).  "Alisa's book of LLMs", Mathy things >
 * Information theory > implementing the loss: the per-token log-prob is the
 * log-softmax at the target, z_target - lse, and the loss averages (or sums)
 * its negation over the non-ignored tokens.
 *
 * Inputs as for flce_fwd_bwd.  Outputs (device, overwritten, each nullable):
 *   loss           [1]  float32  reduced loss (reduction as for flce_fwd_bwd)
 *   token_logprob  [T]  float32  z_target - lse; 0 for ignored tokens
 *   lse            [T]  float32  per-token logsumexp
 *   argmax         [T]  int32    per-token argmax of z, lowest index on ties
 *   n_valid        [1]  int64    number of non-ignored tokens
 * Only the logits GEMM and the merge of its partials run: no T x V or
 * C x V values are written, and a handle created with FLCE_FLAG_FORWARD_ONLY
 * is enough.  The handle's
 * workspace is reused, so a handle must not run flce_forward and
 * flce_fwd_bwd concurrently.  Out-of-range
 * targets are treated as ignored and counted for flce_query_error.
 * Returns without enqueuing anything on an argument error.
 */
flce_status_t flce_forward(flce_handle_t h, const void* X, const void* W, const int64_t* targets,
                           int64_t T, int64_t ignore_index, int32_t reduction, float* loss,
                           float* token_logprob, float* lse, int32_t* argmax, int64_t* n_valid,
                           void* stream);

/*
 * Vocabulary-parallel building blocks.  With W split by rows over G devices
 * (a column-parallel lm_head), each device holds W_shard = W[vocab_offset :
 * vocab_offset + V] (V as given to flce_create) and runs two calls around the
 * caller's collectives.  The per-shard (max, sum of exp) pairs merge exactly
 * like the online-softmax partials of "Alisa's book of LLMs", Numerical
 * stability and other tricks: the global lse is M + ln sum_s sumexp_s
 * exp(m_s - M) with M = max_s m_s.  Targets are replicated: a target is valid
 * when it is not ignore_index and lies in [0, vocab_total); the shard holding
 * it "owns" it.
 *
 * Step 1, flce_vocab_shard_forward: per token of this shard's columns
 *   m        [T] float32  max logit (required)
 *   sumexp   [T] float32  sum of exp(z - m) (required)
 *   argmax   [T] int32    global id of the first max (nullable)
 *   ztarget  [T] float32  the target's logit if this shard owns the target,
 *                         else 0 -- a sum over shards gives z_target (required)
 * The caller then all-reduces: M = max m, sumexp * exp(m - M) summed, ztarget
 * summed; lse = M + ln(sum), loss = s * sum_t valid_t (lse_t - ztarget_t).
 *
 * Step 2, flce_vocab_shard_backward, given that global lse [T]:
 *   dX_partial [T x H] dtype   this shard's dZ W_shard; summed over shards
 *                              by the caller, it is dX
 *   dW_shard   [V x H] float32 this shard's rows of dW (complete)
 * with dZ = s valid (exp(z - lse) - onehot) as for flce_fwd_bwd and s from
 * `reduction` over the valid targets.  Step 2 recomputes the shard's logits
 * (the call keeps nothing of step 1), so a vocabulary-parallel step costs
 * 8 T H V_shard flops per device instead of 6.
 *
 * Both return INVALID_ARGUMENT, with nothing enqueued, for a shard outside
 * [0, vocab_total) or vocab_total >= 2^31, and as flce_fwd_bwd otherwise.
 */
flce_status_t flce_vocab_shard_forward(flce_handle_t h, const void* X, const void* W_shard,
                                       const int64_t* targets, int64_t T, int64_t ignore_index,
                                       int64_t vocab_offset, int64_t vocab_total, float* m,
                                       float* sumexp, int32_t* argmax, float* ztarget,
                                       void* stream);
flce_status_t flce_vocab_shard_backward(flce_handle_t h, const void* X, const void* W_shard,
                                        const int64_t* targets, int64_t T, int64_t ignore_index,
                                        int64_t vocab_offset, int64_t vocab_total,
                                        int32_t reduction, const float* lse, void* dX_partial,
                                        float* dW_shard, void* stream);

/*
 * Soft targets (distillation) with a temperature.  "Alisa's book of LLMs",
 * Mathy things > Information theory: the cross-entropy of a target
 * distribution q against the model's p is KL(q || p) plus the entropy of q,
 * and reduces to the NLL of the target for a one-hot q; Neural net basics:
 * the softmax with a temperature divides the logits by it first.  Here q
 * comes from a teacher head evaluated on the fly, so neither model's T x V
 * logits are held:
 *
 *   p_t = softmax(X_t W^T / tau),  q_t = softmax(X_teacher_t W_teacher^T / tau)
 *   loss = s sum_t valid_t H(q_t, p_t),   dZ = s valid (p - q) / tau
 *   dX = dZ W (X's dtype),  dW = dZ^T X (fp32); the teacher gets no gradient
 *
 * with valid_t and s from `targets`, ignore_index and `reduction` as for
 * flce_fwd_bwd (the targets serve only as the mask; out-of-range ids count
 * as ignored and are reported by flce_query_error).  No tau^2 factor is
 * applied: multiply loss and gradients by tau^2 for the usual distillation
 * scaling.
 *
 * flce_distill_create: as flce_create, plus the teacher's hidden size
 * (> 0, a multiple of 8 for bf16 or 4 for fp32, at most 2^20) and a second
 * C x V workspace buffer for the teacher's exponentials.
 * flce_distill_fwd_bwd: X [T x H], W [V x H], X_teacher [T x Ht],
 * W_teacher [V x Ht], all in the handle's dtype; temperature > 0 and
 * finite.  INVALID_ARGUMENT, with nothing enqueued, for a handle made by
 * flce_create or a bad argument.
 */
flce_status_t flce_distill_create(const flce_config_t* cfg, int64_t teacher_hidden,
                                  flce_handle_t* out);
flce_status_t flce_distill_fwd_bwd(flce_handle_t h, const void* X, const void* W,
                                   const void* X_teacher, const void* W_teacher,
                                   const int64_t* targets, int64_t T, int64_t ignore_index,
                                   float temperature, int32_t reduction, float* loss, void* dX,
                                   float* dW, int64_t* n_valid, void* stream);

/*
 * Allocation-free variant of flce_fwd_bwd, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It takes the configuration instead of a handle and
 * runs the same kernels, in the same order, with the same results, as
 * flce_fwd_bwd on a handle made by flce_create(cfg); arguments, outputs and
 * their errors are those of flce_fwd_bwd.  The workspace lives in a static
 * device array of FLCE_NOALLOC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends; the call itself allocates nothing
 * (no hipMalloc, no allocating library routine).  Its first call on a device
 * looks the array's address up (hipGetSymbolAddress).
 *  - Returns FLCE_ERR_UNSUPPORTED, with nothing enqueued, when the
 *    configuration's workspace (what flce_workspace_bytes would report for a
 *    handle of cfg) exceeds FLCE_NOALLOC_SCRATCH_BYTES; flce_last_error then
 *    gives the size needed.  A smaller chunk_tokens or dw_chunks, or
 *    FLCE_FLAG_NO_WEIGHT_COPY, lowers it.
 *  - Every call on one GPU shares that GPU's array: calls that overlap on one
 *    GPU (other streams, other threads) race and must be ordered by the
 *    caller.  The array keeps the last call's contents; no buffer in it needs
 *    to start at zero.
 *  - flce_query_error, the timing calls and the soft-target, forward-only and
 *    vocabulary-shard calls need a handle; this call has none.
 */
#define FLCE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
flce_status_t flce_fwd_bwd_noalloc(const flce_config_t* cfg, const void* X, const void* W,
                                   const int64_t* targets, int64_t T, int64_t ignore_index,
                                   int32_t reduction, float* loss, void* dX, float* dW,
                                   float* lse, int32_t* argmax, int64_t* n_valid, void* stream);

/* Synchronise `stream` and read the number of out-of-range targets seen by
 * the last flce_fwd_bwd or flce_forward on this handle.  Returns FLCE_ERR_BAD_TARGET when it
 * is > 0, FLCE_OK otherwise.  bad_targets may be NULL. */
flce_status_t flce_query_error(flce_handle_t h, void* stream, int64_t* bad_targets);

/* Per-kernel timing with HIP events recorded on the call's stream around
 * every launch of flce_fwd_bwd while enabled (adds two event records per
 * launch; off by default).  flce_timing_read synchronises the events and
 * returns, for kernel class `kind` (0 .. flce_timing_kinds()-1), the summed
 * duration in milliseconds and the number of launches since the last reset;
 * flce_timing_enable(h, 1) resets the counters. */
flce_status_t flce_timing_enable(flce_handle_t h, int32_t enable);
int32_t flce_timing_kinds(void);
const char* flce_timing_kind_name(int32_t kind);
flce_status_t flce_timing_read(flce_handle_t h, int32_t kind, double* total_ms,
                               int64_t* launches);

/* Free the workspace and the handle (NULL is accepted). */
flce_status_t flce_destroy(flce_handle_t h);

/* Static, human-readable name of a status code. */
const char* flce_status_string(flce_status_t s);

/* Text of the last HIP error seen by this library on the calling thread
 * (empty when none). */
const char* flce_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* FLCE_H */
