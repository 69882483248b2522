// C ABI of the fused linear cross-entropy head (see include/flce.h).
//
// Host side only: argument validation, the per-handle workspace, the token
// chunk loop and optional per-kernel event timing.  Every arithmetic step
// runs in the kernels of kernels.hip.
#include "../../include/flce.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"

using namespace flce;

// Device scratch of flce_fwd_bwd_noalloc: a file-scope array, one copy on
// every GPU the library runs on, held until the process ends.  Host code
// never passes the array's name to a kernel (in host code it is only a
// stand-in); it uses the address hipGetSymbolAddress returns per device.
static __device__ __align__(256) unsigned char scratch[FLCE_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

enum Kind {
  K_COUNT = 0,
  K_TRANSPOSE_W,
  K_TRANSPOSE_X,
  K_LOGITS,
  K_FINALIZE,
  K_FIXUP,
  K_DX,
  K_SPLITK,
  K_DW,
  K_LOSS,
  K_ZERO,
  K_ROWREF,
  K_NUM
};
const char* kKindNames[K_NUM] = {"count_valid",   "transpose_w", "transpose_x", "logits_gemm",
                                 "finalize",      "fixup_dz",    "dx_gemm",     "splitk_reduce",
                                 "dw_gemm",       "loss",        "zero_fill",   "row_reference"};

constexpr int64_t kDefaultChunk = 4096;
constexpr int kMaxDwChunks = 8;
// The dW GEMM reads P -- the exponentials, or dZ where the dZ pass wrote it
// in place -- as stored (no dZ^T) up to this hidden size: its transposing
// LDS reads cost ~7 % of that GEMM, whose time grows with H while the
// transposed write they replace does not.
#ifndef FLCE_DW_READS_P_MAX_H
#define FLCE_DW_READS_P_MAX_H 4096
#endif

inline int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }
inline int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Pending {
  int kind;
  hipEvent_t start, stop;
};

}  // namespace

struct flce_handle {
  int device = 0;
  Dt dt = Dt::BF16;
  int64_t H = 0, V = 0, C = 0, Vpad = 0, nt = 0;
  int G = 1;               // chunks per dW GEMM
  int64_t Ht = 0;          // teacher hidden size (soft-target handles only)
  int splitk_alloc = 1;  // split-K planes the workspace holds for a full chunk
  bool w_copy = true;      // dX reads W^T (a copy made per call) or W as stored
  bool dz_in_dx = true;    // dZ formed inside the dX contraction (not FLCE_FLAG_DZ_IN_PLACE)
  bool fwd_only = false;   // FLCE_FLAG_FORWARD_ONLY: no buffer of the backward
  // The dW contraction reads P as stored, G chunks of it side by side (bf16,
  // H up to FLCE_DW_READS_P_MAX_H, G C Vpad 2 < 2^31 bytes): the exponentials
  // against beta-scaled X^T when dZ is formed inside the contractions, else
  // the dZ the dZ pass wrote in place; no dZ^T either way
  bool dw_reads_p = false;
  // ... and then (hard targets, G > 1) the logits GEMM runs once per group of
  // chunks, its partials kept for the G chunks (one partial round of tiles
  // per group instead of one per chunk)
  bool group_logits = false;
  size_t ws_bytes = 0;
  char* ws = nullptr;
  void* Wt = nullptr;      // W^T           [H x Vpad]
  void* P = nullptr;       // exp / dZ      [C x Vpad], or [G*C x Vpad] (dw_reads_p)
  void* Pt = nullptr;      // dZ^T of G chunks [Vpad x G*C] (not with dw_reads_p)
  void* Xt = nullptr;      // X^T of G chunks  [H x G*C]
  float* pm = nullptr;     // tile max / alpha [nt x C], tile-major
  float* ps = nullptr;     // tile sum      [nt x C]
  int* pa = nullptr;       // tile argmax   [nt x C]
  float* ztgt = nullptr;   // [C]
  float* dzt = nullptr;    // [C]
  float* beta = nullptr;   // [C], or [G*C]: row scale of dZ inside the contractions
  float* corr = nullptr;   // [C] target correction of the dX rows
  uint8_t* shift = nullptr;  // [nt x C] tile reference below the row's, as a shift
  int* tcol = nullptr;     // [C] target column to set in P (-1: none)
  float* tval = nullptr;   // [C] its value
  double* loss_part = nullptr;  // [C / kFinalizeRows]
  float* splitk = nullptr;      // [splitk_alloc x C x H]
  void* Pq = nullptr;           // teacher exp(z_T / tau - m_tile) [C x Vpad]
  float* pmq = nullptr;         // teacher partials / alpha [nt x C]
  float* psq = nullptr;
  int* paq = nullptr;
  float* pc = nullptr;          // cross partials [nt x C]
  int64_t* nvalid = nullptr;
  float* scale = nullptr;
  int64_t* bad = nullptr;
  long long* count_part = nullptr;  // per-block target counts of long batches
  // timing
  bool timing = false;
  std::vector<Pending> pending;
  std::vector<hipEvent_t> pool;
  double total_ms[K_NUM] = {};
  int64_t launches[K_NUM] = {};
};

namespace {

flce_status_t hip_fail(hipError_t e, const char* what) {
  char buf[256];
  snprintf(buf, sizeof buf, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
  g_last_error = buf;
  return e == hipErrorOutOfMemory ? FLCE_ERR_OUT_OF_MEMORY : FLCE_ERR_HIP;
}

hipEvent_t take_event(flce_handle* h) {
  if (!h->pool.empty()) {
    hipEvent_t e = h->pool.back();
    h->pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs one launch, bracketed by events when timing is on.
template <class F>
hipError_t timed(flce_handle* h, int kind, hipStream_t s, F&& launch) {
  if (!h->timing) return launch();
  hipEvent_t a = take_event(h), b = take_event(h);
  if (!a || !b) return launch();
  (void)hipEventRecord(a, s);
  hipError_t e = launch();
  (void)hipEventRecord(b, s);
  h->pending.push_back({kind, a, b});
  return e;
}

flce_status_t drain_timing(flce_handle* h) {
  for (auto& p : h->pending) {
    hipError_t e = hipEventSynchronize(p.stop);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, p.start, p.stop);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    h->total_ms[p.kind] += ms;
    h->launches[p.kind] += 1;
    h->pool.push_back(p.start);
    h->pool.push_back(p.stop);
  }
  h->pending.clear();
  return FLCE_OK;
}

int elems_per_vec(Dt dt) { return dt == Dt::BF16 ? 8 : 4; }
size_t elem_size(Dt dt) { return dt == Dt::BF16 ? 2 : 4; }

// Tile shape and split-K factor for an output of M x N with K-depth K.
void plan_gemm(int64_t M, int64_t N, int64_t K, int max_splits, TileCfg* tc, int* splits) {
  const int64_t t256 = cdiv64(M, 256) * cdiv64(N, 256);
  const int64_t t128 = cdiv64(M, 128) * cdiv64(N, 128);
  *splits = 1;
  if (t256 >= 240) {
    *tc = TileCfg::T256;
    return;
  }
  const int64_t ksteps = cdiv64(K, 64);
  // A grid of 64 to 239 256-wide tiles with at least 32 K-steps per split:
  // split K two to four ways to fill the chip rather than fall back to
  // 128-wide tiles, whose 64 x 64 wave tiles read twice the LDS bytes per
  // MFMA (the dX GEMM of an 8192-token chunk at H = 512, V = 16000, with 62
  // K-steps per split, runs in 0.12 instead of 0.22 ms that way).
  // The split is the one that finishes soonest in whole rounds of 256
  // blocks: a tile's time is its K-depth / s, and t x s blocks take
  // ceil(t s / 256) rounds (96 tiles: 2 ways, 192 blocks, not 3 ways, whose
  // 288 blocks need two rounds); ties go to fewer splits (less to sum).
  if (t256 >= 64) {
    int64_t best = 0;
    double best_t = 1e30;
    for (int64_t s = 1; s <= 4 && s <= max_splits && ksteps / s >= 32; ++s) {
      const double t = (double)cdiv64(t256 * s, 256) / (double)s;
      if (t < best_t - 1e-9) {
        best_t = t;
        best = s;
      }
    }
    if (best >= 1) {  // (unsplit when no split saves a round: still 256-wide)
      *tc = TileCfg::T256;
      *splits = (int)best;
      return;
    }
  }
  *tc = TileCfg::T128;
  if (t128 >= 256 || max_splits <= 1) return;
  int64_t s = cdiv64(512, t128);
  if (s > ksteps / 4) s = ksteps / 4;
  if (s > max_splits) s = max_splits;
  if (s < 1) s = 1;
  *splits = (int)s;
}

std::once_flag g_setup_once;
hipError_t g_setup_err = hipSuccess;

}  // namespace

extern "C" {

const char* flce_status_string(flce_status_t s) {
  // A C caller may pass any int: read the value through its bytes rather than
  // as the enumeration type, whose range is only the listed codes.
  int32_t code;
  static_assert(sizeof code == sizeof s, "flce_status_t is int-sized");
  std::memcpy(&code, &s, sizeof code);
  switch (code) {
    case FLCE_OK: return "FLCE_OK";
    case FLCE_ERR_INVALID_ARGUMENT: return "FLCE_ERR_INVALID_ARGUMENT";
    case FLCE_ERR_UNSUPPORTED: return "FLCE_ERR_UNSUPPORTED";
    case FLCE_ERR_HIP: return "FLCE_ERR_HIP";
    case FLCE_ERR_OUT_OF_MEMORY: return "FLCE_ERR_OUT_OF_MEMORY";
    case FLCE_ERR_BAD_TARGET: return "FLCE_ERR_BAD_TARGET";
  }
  return "FLCE_ERR_UNKNOWN";
}

const char* flce_last_error(void) { return g_last_error.c_str(); }

int32_t flce_timing_kinds(void) { return K_NUM; }

const char* flce_timing_kind_name(int32_t kind) {
  if (kind < 0 || kind >= K_NUM) return "";
  return kKindNames[kind];
}

}  // extern "C"

namespace {

// Byte offsets of the workspace buffers of one handle, from (H, V, C, G,
// dtype, weight copy, teacher) only.
struct Layout {
  size_t Wt, P, Pt, Xt, pm, ps, pa, zt, dz, be, co, sh, tc, tv, lp, sk, sc, cp, Pq, pmq, psq, paq, pc;
  size_t total;
};

// Validates cfg and fills the handle's sizes and the workspace layout; no
// device call.  The workspace pointers are set by bind_workspace.
flce_status_t configure(const flce_config_t* cfg, int64_t Ht, flce_handle* h, Layout* L) {
  if (!cfg) return FLCE_ERR_INVALID_ARGUMENT;
  if (cfg->dtype != FLCE_F32 && cfg->dtype != FLCE_BF16) return FLCE_ERR_INVALID_ARGUMENT;
  if (cfg->dw_chunks < 0 || cfg->dw_chunks > kMaxDwChunks) return FLCE_ERR_INVALID_ARGUMENT;
  const Dt dt = cfg->dtype == FLCE_BF16 ? Dt::BF16 : Dt::F32;
  const int64_t H = cfg->hidden, V = cfg->vocab;
  if (H <= 0 || V <= 0) return FLCE_ERR_INVALID_ARGUMENT;
  if (H % elems_per_vec(dt) != 0) return FLCE_ERR_INVALID_ARGUMENT;
  if (cfg->chunk_tokens < 0) return FLCE_ERR_INVALID_ARGUMENT;
  // The GEMM kernels address a 256-row operand tile with 32-bit byte
  // offsets (row x leading dimension x element size < 2^31): leading
  // dimensions H, the padded vocabulary and G x C stay at or below 2^20.
  if (H > (1 << 20) || round_up(V, 256) > (1 << 20)) return FLCE_ERR_UNSUPPORTED;
  int64_t C = cfg->chunk_tokens ? cfg->chunk_tokens : kDefaultChunk;
  C = round_up(C, 256);
  const int64_t G = cfg->dw_chunks ? cfg->dw_chunks : 1;
  if (C * G > (1 << 20)) return FLCE_ERR_UNSUPPORTED;
  if (cfg->flags & ~(FLCE_FLAG_NO_WEIGHT_COPY | FLCE_FLAG_DZ_IN_PLACE | FLCE_FLAG_FORWARD_ONLY))
    return FLCE_ERR_INVALID_ARGUMENT;
  const bool no_wcopy = (cfg->flags & FLCE_FLAG_NO_WEIGHT_COPY) != 0;
  const bool fwd_only = (cfg->flags & FLCE_FLAG_FORWARD_ONLY) != 0;
  if (fwd_only && Ht) return FLCE_ERR_INVALID_ARGUMENT;  // the soft-target call has no forward
  // W as stored: bf16 transposing LDS reads; one buffer descriptor spans W,
  // whose size must stay below the out-of-range offset (2^31) that reads 0
  if (no_wcopy && (dt != Dt::BF16 || V * H * 2 >= ((int64_t)1 << 31))) return FLCE_ERR_UNSUPPORTED;

  h->dt = dt;
  h->H = H;
  h->V = V;
  h->C = C;
  h->G = (int)G;
  h->Ht = Ht;
  h->fwd_only = fwd_only;
  h->w_copy = !no_wcopy && !fwd_only;
  h->dz_in_dx = (cfg->flags & FLCE_FLAG_DZ_IN_PLACE) == 0;
  h->Vpad = round_up(V, 256);
  // the dW GEMM's one buffer descriptor spans the G chunks of P
  h->dw_reads_p = !fwd_only && dt == Dt::BF16 && H <= FLCE_DW_READS_P_MAX_H &&
                  G * C * h->Vpad * 2 < ((int64_t)1 << 31);
  h->group_logits = h->dw_reads_p && G > 1 && Ht == 0;
  h->nt = cdiv64(V, kPartialWidth);
  h->splitk_alloc = 1;
  if (!fwd_only) {
    TileCfg tc;
    int sp;
    plan_gemm(C, H, round_up(V, 64), 8, &tc, &sp);
    h->splitk_alloc = sp;
  }
  const size_t es = elem_size(dt);
  size_t off = 0;
  auto carve = [&](size_t bytes) {
    const size_t o = off;
    off += round_up((int64_t)bytes, 256);
    return o;
  };
  // a forward-only handle keeps the merge partials, the target logits and
  // the loss and count partials; nothing of the backward
  const bool bwd = !fwd_only;
  L->Wt = h->w_copy ? carve((size_t)H * h->Vpad * es) : 0;
  L->P = bwd ? carve((size_t)(h->dw_reads_p ? h->G * C : C) * h->Vpad * es) : 0;
  L->Pt = bwd && !h->dw_reads_p ? carve((size_t)h->Vpad * h->G * C * es) : 0;
  L->Xt = bwd ? carve((size_t)H * h->G * C * es) : 0;
  const int64_t Cp = h->group_logits ? h->G * C : C;  // rows of the logits partials
  L->pm = carve((size_t)Cp * h->nt * 4);
  L->ps = carve((size_t)Cp * h->nt * 4);
  L->pa = carve((size_t)Cp * h->nt * 4);
  L->zt = carve((size_t)Cp * 4);
  L->dz = carve((size_t)C * 4);
  L->be = bwd ? carve((size_t)(h->dw_reads_p ? h->G * C : C) * 4) : 0;
  L->co = bwd ? carve((size_t)C * 4) : 0;
  L->sh = bwd ? carve((size_t)C * round_up(h->nt, 16)) : 0;
  L->tc = bwd ? carve((size_t)C * 4) : 0;
  L->tv = bwd ? carve((size_t)C * 4) : 0;
  L->lp = carve((size_t)cdiv64(C, kFinalizeRows) * 8);
  L->sk = h->splitk_alloc > 1 ? carve((size_t)h->splitk_alloc * C * H * 4) : 0;
  L->sc = carve(64);
  L->cp = carve(2 * kCountBlocks * sizeof(long long));
  // soft targets: the teacher's exponentials and partials, and the cross partials
  L->Pq = Ht ? carve((size_t)C * h->Vpad * es) : 0;
  L->pmq = Ht ? carve((size_t)C * h->nt * 4) : 0;
  L->psq = Ht ? carve((size_t)C * h->nt * 4) : 0;
  L->paq = Ht ? carve((size_t)C * h->nt * 4) : 0;
  L->pc = Ht ? carve((size_t)C * h->nt * 4) : 0;
  L->total = off;
  h->ws_bytes = off;
  return FLCE_OK;
}

// Points the handle's buffers into a workspace of L.total bytes at base.
void bind_workspace(flce_handle* h, const Layout& L, char* base) {
  h->ws = base;
  h->Wt = h->w_copy ? base + L.Wt : nullptr;
  const bool bwd = !h->fwd_only;
  h->P = bwd ? base + L.P : nullptr;
  h->Pt = bwd && !h->dw_reads_p ? base + L.Pt : nullptr;
  h->Xt = bwd ? base + L.Xt : nullptr;
  h->pm = (float*)(base + L.pm);
  h->ps = (float*)(base + L.ps);
  h->pa = (int*)(base + L.pa);
  h->ztgt = (float*)(base + L.zt);
  h->dzt = (float*)(base + L.dz);
  h->beta = bwd ? (float*)(base + L.be) : nullptr;
  h->corr = bwd ? (float*)(base + L.co) : nullptr;
  h->shift = bwd ? (uint8_t*)(base + L.sh) : nullptr;
  h->tcol = bwd ? (int*)(base + L.tc) : nullptr;
  h->tval = bwd ? (float*)(base + L.tv) : nullptr;
  h->loss_part = (double*)(base + L.lp);
  h->splitk = h->splitk_alloc > 1 ? (float*)(base + L.sk) : nullptr;
  h->nvalid = (int64_t*)(base + L.sc);
  h->scale = (float*)(base + L.sc + 16);
  h->bad = (int64_t*)(base + L.sc + 32);
  h->count_part = (long long*)(base + L.cp);
  if (h->Ht) {
    h->Pq = base + L.Pq;
    h->pmq = (float*)(base + L.pmq);
    h->psq = (float*)(base + L.psq);
    h->paq = (int*)(base + L.paq);
    h->pc = (float*)(base + L.pc);
  }
}

flce_status_t ensure_setup() {
  std::call_once(g_setup_once, [] { g_setup_err = gemm_setup(); });
  if (g_setup_err != hipSuccess) return hip_fail(g_setup_err, "gemm_setup");
  return FLCE_OK;
}

flce_status_t create_impl(const flce_config_t* cfg, int64_t Ht, flce_handle_t* out) {
  if (!out) return FLCE_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  flce_handle* h = new (std::nothrow) flce_handle();
  if (!h) return FLCE_ERR_OUT_OF_MEMORY;
  Layout L;
  flce_status_t st = configure(cfg, Ht, h, &L);
  if (st != FLCE_OK) {
    delete h;
    return st;
  }
  hipError_t e = hipGetDevice(&h->device);
  if (e != hipSuccess) {
    delete h;
    return hip_fail(e, "hipGetDevice");
  }
  if ((st = ensure_setup()) != FLCE_OK) {
    delete h;
    return st;
  }
  char* ws = nullptr;
  e = hipMalloc((void**)&ws, L.total);
  if (e != hipSuccess) {
    st = hip_fail(e, "hipMalloc(workspace)");
    delete h;
    (void)hipGetLastError();
    return st == FLCE_ERR_HIP ? FLCE_ERR_OUT_OF_MEMORY : st;
  }
  bind_workspace(h, L, ws);
  e = hipMemset(ws + L.sc, 0, 64);
  if (e != hipSuccess) {
    (void)hipFree(ws);
    delete h;
    return hip_fail(e, "hipMemset");
  }
  *out = h;
  return FLCE_OK;
}

}  // namespace

extern "C" {

flce_status_t flce_create(const flce_config_t* cfg, flce_handle_t* out) {
  return create_impl(cfg, 0, out);
}

flce_status_t flce_distill_create(const flce_config_t* cfg, int64_t teacher_hidden,
                                  flce_handle_t* out) {
  if (out) *out = nullptr;
  if (!cfg || teacher_hidden <= 0) return FLCE_ERR_INVALID_ARGUMENT;
  const Dt dt = cfg->dtype == FLCE_BF16 ? Dt::BF16 : Dt::F32;
  if (teacher_hidden % elems_per_vec(dt) != 0) return FLCE_ERR_INVALID_ARGUMENT;
  if (teacher_hidden > (1 << 20)) return FLCE_ERR_UNSUPPORTED;
  return create_impl(cfg, teacher_hidden, out);
}

size_t flce_workspace_bytes(flce_handle_t h) { return h ? h->ws_bytes : 0; }

int64_t flce_chunk_tokens(flce_handle_t h) { return h ? h->C : 0; }

int32_t flce_dw_chunks(flce_handle_t h) { return h ? h->G : 0; }

flce_status_t flce_destroy(flce_handle_t h) {
  if (!h) return FLCE_OK;
  drain_timing(h);
  for (hipEvent_t e : h->pool) (void)hipEventDestroy(e);
  if (h->ws) (void)hipFree(h->ws);
  delete h;
  return FLCE_OK;
}

namespace {

// Columns this call sees: W's rows are vocabulary ids [y_shift, y_shift + V)
// of a vocabulary of v_total ids (y_shift = 0, v_total = V unless W is a
// vocabulary shard).  lse_in, when given, replaces the lse of these columns
// by the whole vocabulary's.
struct Cols {
  int64_t y_shift;
  int64_t v_total;
  const float* lse_in;
};

// Soft targets: a teacher head (its hidden states and weight, hidden size
// h->Ht) whose tempered softmax replaces the one-hot target.
struct Soft {
  const void* Xq;
  const void* Wq;
  float inv_temp;
};

flce_status_t check_device(flce_handle_t h, const char* who) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != h->device) {
    g_last_error = std::string(who) + ": current device differs from the handle's device";
    return FLCE_ERR_INVALID_ARGUMENT;
  }
  return FLCE_OK;
}

bool misaligned(const void* p, uintptr_t mask) { return ((uintptr_t)p & mask) != 0; }

// Argument checks shared by flce_fwd_bwd and flce_fwd_bwd_noalloc.
flce_status_t check_fwd_bwd_args(const void* X, const void* W, const int64_t* targets, int64_t T,
                                 int32_t reduction, const float* loss, const void* dX,
                                 const float* dW, const float* lse, const int32_t* argmax,
                                 const int64_t* n_valid) {
  if (T < 0) return FLCE_ERR_INVALID_ARGUMENT;
  if (reduction != FLCE_MEAN && reduction != FLCE_SUM) return FLCE_ERR_INVALID_ARGUMENT;
  if (!W || !loss || !dW) return FLCE_ERR_INVALID_ARGUMENT;
  if (T > 0 && (!X || !targets || !dX)) return FLCE_ERR_INVALID_ARGUMENT;
  if (!aligned16(W) || !aligned16(dW) || (T > 0 && (!aligned16(X) || !aligned16(dX))))
    return FLCE_ERR_INVALID_ARGUMENT;
  if (misaligned(loss, 3) || misaligned(lse, 3) || misaligned(argmax, 3) ||
      misaligned(n_valid, 7) || misaligned(targets, 7))
    return FLCE_ERR_INVALID_ARGUMENT;
  return FLCE_OK;
}

flce_status_t run_fwd_bwd(flce_handle_t h, const void* X, const void* W, const int64_t* targets,
                          int64_t T, int64_t ignore_index, int32_t reduction, float* loss,
                          void* dX, float* dW, float* lse, int32_t* argmax, int64_t* n_valid,
                          const Cols& cols, void* stream, const Soft* soft = nullptr) {
  hipStream_t s = (hipStream_t)stream;
  const Dt dt = h->dt;
  const size_t es = elem_size(dt);
  const int64_t H = h->H, V = h->V, C = h->C, Vpad = h->Vpad, nt = h->nt;
  const int64_t G = h->G, GC = G * C;  // P or dZ^T, and X^T, of G chunks side by side
  const int rsum = reduction == FLCE_SUM ? 1 : 0;

#define FLCE_LAUNCH(kind, expr)                                      \
  do {                                                               \
    hipError_t _e = timed(h, kind, s, [&] { return (expr); });       \
    if (_e != hipSuccess) return hip_fail(_e, kKindNames[kind]);     \
  } while (0)

  FLCE_LAUNCH(K_COUNT, launch_count(targets, T, ignore_index, cols.v_total, rsum, h->nvalid,
                                    h->scale, h->bad, n_valid, h->count_part, s));
  if (T == 0) {
    FLCE_LAUNCH(K_ZERO, launch_zero(dW, (size_t)V * H * 4, s));
    if (loss) {
      FLCE_LAUNCH(K_ZERO, launch_zero(h->loss_part, 8, s));
      FLCE_LAUNCH(K_LOSS, launch_loss(h->loss_part, 1, h->nvalid, rsum, loss, s));
    }
    return FLCE_OK;
  }

  // W^T (zero-padded to Vpad columns): K-contiguous operand of dX = dZ W,
  // unless the handle reads W as stored.
  if (h->w_copy)
    FLCE_LAUNCH(K_TRANSPOSE_W,
                launch_transpose(dt, W, (int)V, (int)H, H, h->Wt, Vpad, (int)Vpad, s));

  const int64_t KV = round_up(V, 64);  // K-depth of the dX GEMM
  for (int64_t t0 = 0, c = 0; t0 < T; t0 += C, ++c) {
    const int64_t Cc = (T - t0 < C) ? (T - t0) : C;
    const int64_t Ck = round_up(Cc, 64);
    const char* Xc = (const char*)X + (size_t)t0 * H * es;
    const int64_t* yc = targets + t0;
    // slot of this chunk in the G-chunk dZ^T / X^T buffers; every chunk but
    // the batch's last is full, so the slots of a group are contiguous in K
    const int64_t gs = c % G;
    const bool last = t0 + Cc >= T;
    // dZ formed inside the contractions (hard targets); dW reading P as
    // stored (the exponentials when fused, else dZ), each chunk's in its own
    // slot of the G-chunk buffer
    const bool fused = !soft && h->dz_in_dx;
    const bool dw_p = h->dw_reads_p;
    char* const Pc = (char*)h->P + (dw_p ? (size_t)gs * C * Vpad * es : 0);
    float* const beta_c = h->beta + (dw_p ? gs * C : 0);
    // logits partials of this chunk: its rows among the group's when the
    // logits GEMM covers a whole group (launched at the group's first chunk)
    const bool grp = !soft && h->group_logits;
    const int64_t ldr = grp ? GC : C;
    float* const pm_c = h->pm + (grp ? gs * C : 0);
    float* const ps_c = h->ps + (grp ? gs * C : 0);
    int* const pa_c = h->pa + (grp ? gs * C : 0);
    float* const zt_c = h->ztgt + (grp ? gs * C : 0);

    // X^T of the whole group at its first chunk (X is an input, all of it
    // available): one transpose per dW GEMM; the previous group's dW GEMM,
    // earlier in the stream, has finished reading the buffer.  When dW reads
    // P, X^T is made at the group's last chunk instead, carrying the rows'
    // beta when P holds the exponentials (all of them known by then).
    if (gs == 0 && !dw_p) {
      const int64_t Cg = (T - t0 < GC) ? (T - t0) : GC;
      FLCE_LAUNCH(K_TRANSPOSE_X, launch_transpose(dt, Xc, (int)Cg, (int)H, H, h->Xt, GC,
                                                  (int)round_up(Cg, 64), s));
    }

    if (soft) {
      // teacher: tempered logits, their exponentials and partials, then its
      // alpha = exp(m_tile - lse) (no reduction scale, no one-hot column)
      LogitsArgs qa{};
      qa.X = (const char*)soft->Xq + (size_t)t0 * h->Ht * es;
      qa.W = soft->Wq;
      qa.M = (int)Cc;
      qa.V = (int)V;
      qa.H = (int)h->Ht;
      qa.P = h->Pq;
      qa.ldp = Vpad;
      qa.pm = h->pmq;
      qa.ps = h->psq;
      qa.pa = h->paq;
      qa.ldr = C;
      qa.ztgt = h->ztgt;
      qa.y = yc;
      qa.ignore_index = ignore_index;
      qa.y_shift = 0;
      qa.inv_temp = soft->inv_temp;
      FLCE_LAUNCH(K_LOGITS, launch_logits(dt, qa, s));
      FinalizeArgs qf{};
      qf.block_rows = finalize_rows(nt, C);
      qf.M = (int)Cc;
      qf.nt = (int)nt;
      qf.V = (int)V;
      qf.pm = h->pmq;
      qf.ps = h->psq;
      qf.pa = h->paq;
      qf.ldr = C;
      qf.ztgt = h->ztgt;
      qf.dzt = h->dzt;
      qf.y = yc;
      qf.ignore_index = ignore_index;
      qf.scale = h->scale;
      qf.y_shift = 0;
      qf.v_total = V;
      qf.unit_scale = true;
      qf.no_target = true;
      qf.backward = true;
      qf.loss_part = nullptr;
      FLCE_LAUNCH(K_FINALIZE, launch_finalize(qf, s));
    }

    if (!grp || gs == 0) {
      // this chunk's logits, or those of its whole group (every chunk of a
      // group but the batch's last is full: the group's rows are contiguous)
      const int64_t Mr = grp ? ((T - t0 < GC) ? (T - t0) : GC) : Cc;
      LogitsArgs la{};
      la.X = Xc;
      la.W = W;
      la.M = (int)Mr;
      la.V = (int)V;
      la.H = (int)H;
      la.P = Pc;
      la.ldp = Vpad;
      la.pm = pm_c;
      la.ps = ps_c;
      la.pa = pa_c;
      la.ldr = ldr;
      la.ztgt = zt_c;
      la.y = yc;
      la.ignore_index = ignore_index;
      la.y_shift = cols.y_shift;
      if (soft) {
        la.inv_temp = soft->inv_temp;
        la.Pq = h->Pq;
        la.pc = h->pc;
      }
      FLCE_LAUNCH(K_LOGITS, launch_logits(dt, la, s));
    }

    FinalizeArgs fa{};
    fa.block_rows = finalize_rows(nt, C);
    fa.M = (int)Cc;
    fa.nt = (int)nt;
    fa.V = (int)V;
    fa.pm = pm_c;
    fa.ps = ps_c;
    fa.pa = pa_c;
    fa.ldr = ldr;
    fa.ztgt = zt_c;
    fa.dzt = h->dzt;
    fa.y = yc;
    fa.ignore_index = ignore_index;
    fa.scale = h->scale;
    fa.lse_out = lse ? lse + t0 : nullptr;
    fa.argmax_out = argmax ? argmax + t0 : nullptr;
    fa.logprob_out = nullptr;
    fa.y_shift = cols.y_shift;
    fa.v_total = cols.v_total;
    fa.lse_in = cols.lse_in ? cols.lse_in + t0 : nullptr;
    if (soft) {
      fa.cross_pc = h->pc;
      fa.alpha_q = h->pmq;
      fa.alpha_mul = soft->inv_temp;
      fa.no_target = true;
    } else if (fused) {
      // dZ is formed inside the contractions from the stored exponentials,
      // which the row-reference pass below brings to one reference per row
      // (setting the target's column); the row scale, target correction and
      // what that pass needs come out
      fa.shift = h->shift;
      fa.ld_shift = round_up(nt, 16);
      fa.beta = beta_c;
      fa.corr = h->corr;
      fa.tcol = h->tcol;
      fa.tval = h->tval;
      fa.round_bf16 = dt == Dt::BF16;
    }
    fa.backward = true;
    fa.loss_part = h->loss_part;
    fa.first_chunk = c == 0;
    FLCE_LAUNCH(K_FINALIZE, launch_finalize(fa, s));
    if (fused) {
      RowRefArgs ra{};
      ra.P = Pc;
      ra.ldp = Vpad;
      ra.M = (int)Cc;
      ra.V = (int)V;
      ra.nt = (int)nt;
      ra.shift = h->shift;
      ra.ld_shift = round_up(nt, 16);
      ra.tcol = h->tcol;
      ra.tval = h->tval;
      FLCE_LAUNCH(K_ROWREF, launch_rowref(dt, ra, s));
    }

    // The dZ pass: dZ over the exponentials unless dZ is formed inside the
    // contractions, and dZ^T for the dW contraction unless it reads P;
    // nothing to do when both hold
    FixupArgs xa{};
    xa.P = Pc;
    xa.ldp = Vpad;
    xa.Pt = dw_p ? nullptr : (char*)h->Pt + (size_t)gs * C * es;
    xa.ldpt = GC;
    xa.M = (int)Cc;
    xa.rows_out = (int)Ck;
    xa.V = (int)V;
    xa.Vpad = (int)Vpad;
    xa.nt = (int)nt;
    xa.ldr = ldr;
    xa.alpha = pm_c;
    xa.dzt = h->dzt;
    xa.y = yc;
    xa.ignore_index = ignore_index;
    xa.y_shift = cols.y_shift;
    if (soft) {
      xa.no_target = true;
      xa.Pq = h->Pq;
      xa.alpha_q = h->pmq;
    }
    xa.write_rows = !fused;
    xa.write_t = !dw_p;
    if (xa.write_rows || xa.write_t) FLCE_LAUNCH(K_FIXUP, launch_fixup(dt, xa, s));

    // dX_c = dZ W   (M = Cc, N = H, K = vocabulary); without soft targets
    // A holds the exponentials and dZ is formed in the contraction
    DxFuse fz{};
    fz.beta = beta_c;
    fz.corr = h->corr;
    fz.y = yc;
    fz.ignore_index = ignore_index;
    fz.y_shift = cols.y_shift;
    fz.V = (int)V;
    fz.W = W;
    fz.ldw = H;
    const DxFuse* fuse = fused ? &fz : nullptr;
    {
      TileCfg tc;
      int splits;
      int max_splits = h->splitk_alloc > 1 ? (int)((h->splitk_alloc * C) / Ck) : 1;
      if (max_splits > 8) max_splits = 8;
      plan_gemm(Cc, H, KV, max_splits, &tc, &splits);
      GemmOutArgs ga{};
      ga.A = Pc;
      ga.lda = Vpad;
      if (h->w_copy) {
        ga.B = h->Wt;
        ga.ldb = Vpad;
        ga.K = (int)KV;
      } else {
        // W's V rows as stored; dZ's columns from V on are zero
        ga.B = W;
        ga.ldb = H;
        ga.K = (int)V;
        ga.b_stored = true;
      }
      ga.M = (int)Cc;
      ga.N = (int)H;
      ga.accumulate = false;
      ga.fuse = fuse;
      char* dXc = (char*)dX + (size_t)t0 * H * es;
      if (splits == 1) {
        ga.out = dXc;
        ga.ldo = H;
        ga.out_f32 = dt == Dt::F32;
        ga.splits = 1;
        ga.split_stride = 0;
        FLCE_LAUNCH(K_DX, launch_gemm_store(dt, tc, ga, s));
      } else {
        ga.out = h->splitk;
        ga.ldo = H;
        ga.out_f32 = true;
        ga.splits = splits;
        ga.split_stride = Ck * H;
        FLCE_LAUNCH(K_DX, launch_gemm_store(dt, tc, ga, s));
        FLCE_LAUNCH(K_SPLITK, launch_splitk_reduce(dt, h->splitk, splits, Ck * H, (int)Cc,
                                                   (int)H, dXc, H, s, fuse));
      }
    }
    // dW (+)= dZ^T X over the chunks of a group (M = V, N = H, K = gs C + Ck)
    // once its last chunk is in (as P^T (beta X) when dW reads the
    // exponentials); the first group stores.
    if (gs == G - 1 || last) {
      const int64_t Kg = gs * C + Ck;
      TileCfg tc;
      int splits;
      plan_gemm(V, H, Kg, 1, &tc, &splits);
      GemmOutArgs ga{};
      if (dw_p) {
        // dW = sum_t P_t^T (beta_t X_t) with the exponentials (the target
        // columns hold dZ / beta, set by the merge), or sum_t dZ_t^T X_t with
        // dZ in place: A is the group's P as stored (token rows, K = its
        // tokens exactly: rows past them read as zero), B the rows' X^T,
        // scaled by beta in the first case
        const int64_t g0 = t0 - gs * C;  // the group's first token
        const int64_t Cg = gs * C + Cc;
        FLCE_LAUNCH(K_TRANSPOSE_X,
                    launch_transpose(dt, (const char*)X + (size_t)g0 * H * es, (int)Cg, (int)H, H,
                                     h->Xt, GC, (int)round_up(Cg, 64), s,
                                     fused ? h->beta : nullptr));
        ga.A = h->P;
        ga.lda = Vpad;
        ga.a_stored = true;
      } else {
        ga.A = h->Pt;
        ga.lda = GC;
      }
      ga.B = h->Xt;
      ga.ldb = GC;
      ga.M = (int)V;
      ga.N = (int)H;
      ga.K = (int)(dw_p ? gs * C + Cc : Kg);
      ga.out = dW;
      ga.ldo = H;
      ga.out_f32 = true;
      ga.may_accumulate = true;
      ga.accumulate = c >= G;
      ga.splits = 1;
      ga.split_stride = 0;
      // the dX split-K planes are free again here (summed before this launch)
      ga.tail_part = h->splitk;
      ga.tail_part_bytes = h->splitk ? (size_t)h->splitk_alloc * C * H * sizeof(float) : 0;
      FLCE_LAUNCH(K_DW, launch_gemm_store(dt, tc, ga, s));
    }
  }
  if (loss) {
    const int nparts = (int)cdiv64(T < C ? T : C, finalize_rows(nt, C));  // finalize blocks of the first chunk
    FLCE_LAUNCH(K_LOSS, launch_loss(h->loss_part, nparts, h->nvalid, rsum, loss, s));
  }
#undef FLCE_LAUNCH
  return FLCE_OK;
}

flce_status_t run_forward(flce_handle_t h, const void* X, const void* W, const int64_t* targets,
                          int64_t T, int64_t ignore_index, int32_t reduction, float* loss,
                          float* token_logprob, float* lse, int32_t* argmax, int64_t* n_valid,
                          float* m_out, float* sum_out, float* zt_out, const Cols& cols,
                          void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const Dt dt = h->dt;
  const size_t es = elem_size(dt);
  const int64_t H = h->H, V = h->V, C = h->C, nt = h->nt;
  const int rsum = reduction == FLCE_SUM ? 1 : 0;

#define FLCE_LAUNCH(kind, expr)                                      \
  do {                                                               \
    hipError_t _e = timed(h, kind, s, [&] { return (expr); });       \
    if (_e != hipSuccess) return hip_fail(_e, kKindNames[kind]);     \
  } while (0)

  FLCE_LAUNCH(K_COUNT, launch_count(targets, T, ignore_index, cols.v_total, rsum, h->nvalid,
                                    h->scale, h->bad, n_valid, h->count_part, s));
  if (T == 0) {
    if (loss) {
      FLCE_LAUNCH(K_ZERO, launch_zero(h->loss_part, 8, s));
      FLCE_LAUNCH(K_LOSS, launch_loss(h->loss_part, 1, h->nvalid, rsum, loss, s));
    }
    return FLCE_OK;
  }
  // Only the logits GEMM (its epilogue keeps the online-softmax partials
  // and the target logit, nothing T x V-shaped) and the merge run.
  for (int64_t t0 = 0, c = 0; t0 < T; t0 += C, ++c) {
    const int64_t Cc = (T - t0 < C) ? (T - t0) : C;
    LogitsArgs la{};
    la.X = (const char*)X + (size_t)t0 * H * es;
    la.W = W;
    la.M = (int)Cc;
    la.V = (int)V;
    la.H = (int)H;
    la.P = nullptr;
    la.ldp = 0;
    la.pm = h->pm;
    la.ps = h->ps;
    la.pa = h->pa;
    la.ldr = C;
    la.ztgt = h->ztgt;
    la.y = targets + t0;
    la.ignore_index = ignore_index;
    la.y_shift = cols.y_shift;
    FLCE_LAUNCH(K_LOGITS, launch_logits(dt, la, s));

    FinalizeArgs fa{};
    fa.block_rows = finalize_rows(nt, C);
    fa.M = (int)Cc;
    fa.nt = (int)nt;
    fa.V = (int)V;
    fa.pm = h->pm;
    fa.ps = h->ps;
    fa.pa = h->pa;
    fa.ldr = C;
    fa.ztgt = h->ztgt;
    fa.dzt = h->dzt;
    fa.y = targets + t0;
    fa.ignore_index = ignore_index;
    fa.scale = h->scale;
    fa.lse_out = lse ? lse + t0 : nullptr;
    fa.argmax_out = argmax ? argmax + t0 : nullptr;
    fa.logprob_out = token_logprob ? token_logprob + t0 : nullptr;
    fa.y_shift = cols.y_shift;
    fa.v_total = cols.v_total;
    fa.lse_in = nullptr;
    fa.m_out = m_out ? m_out + t0 : nullptr;
    fa.sum_out = sum_out ? sum_out + t0 : nullptr;
    fa.zt_out = zt_out ? zt_out + t0 : nullptr;
    fa.backward = false;
    fa.loss_part = h->loss_part;
    fa.first_chunk = c == 0;
    FLCE_LAUNCH(K_FINALIZE, launch_finalize(fa, s));
  }
  if (loss) {
    const int nparts = (int)cdiv64(T < C ? T : C, finalize_rows(nt, C));
    FLCE_LAUNCH(K_LOSS, launch_loss(h->loss_part, nparts, h->nvalid, rsum, loss, s));
  }
#undef FLCE_LAUNCH
  return FLCE_OK;
}

}  // namespace

flce_status_t flce_fwd_bwd(flce_handle_t h, const void* X, const void* W, const int64_t* targets,
                           int64_t T, int64_t ignore_index, int32_t reduction, float* loss,
                           void* dX, float* dW, float* lse, int32_t* argmax, int64_t* n_valid,
                           void* stream) {
  if (!h || h->fwd_only) return FLCE_ERR_INVALID_ARGUMENT;
  flce_status_t st =
      check_fwd_bwd_args(X, W, targets, T, reduction, loss, dX, dW, lse, argmax, n_valid);
  if (st != FLCE_OK) return st;
  st = check_device(h, "flce_fwd_bwd");
  if (st != FLCE_OK) return st;
  return run_fwd_bwd(h, X, W, targets, T, ignore_index, reduction, loss, dX, dW, lse, argmax,
                     n_valid, Cols{0, h->V, nullptr}, stream);
}

flce_status_t flce_forward(flce_handle_t h, const void* X, const void* W, const int64_t* targets,
                           int64_t T, int64_t ignore_index, int32_t reduction, float* loss,
                           float* token_logprob, float* lse, int32_t* argmax, int64_t* n_valid,
                           void* stream) {
  if (!h) return FLCE_ERR_INVALID_ARGUMENT;
  if (T < 0) return FLCE_ERR_INVALID_ARGUMENT;
  if (reduction != FLCE_MEAN && reduction != FLCE_SUM) return FLCE_ERR_INVALID_ARGUMENT;
  if (!W) return FLCE_ERR_INVALID_ARGUMENT;
  if (T > 0 && (!X || !targets)) return FLCE_ERR_INVALID_ARGUMENT;
  if (!aligned16(W) || (T > 0 && !aligned16(X))) return FLCE_ERR_INVALID_ARGUMENT;
  if (misaligned(loss, 3) || misaligned(token_logprob, 3) || misaligned(lse, 3) ||
      misaligned(argmax, 3) || misaligned(n_valid, 7) || misaligned(targets, 7))
    return FLCE_ERR_INVALID_ARGUMENT;
  const flce_status_t st = check_device(h, "flce_forward");
  if (st != FLCE_OK) return st;
  return run_forward(h, X, W, targets, T, ignore_index, reduction, loss, token_logprob, lse,
                     argmax, n_valid, nullptr, nullptr, nullptr, Cols{0, h->V, nullptr}, stream);
}

// A shard's columns must lie inside the vocabulary.
static bool bad_shard(flce_handle_t h, int64_t vocab_offset, int64_t vocab_total) {
  return vocab_offset < 0 || vocab_total < h->V || vocab_offset > vocab_total - h->V ||
         vocab_total > ((int64_t)1 << 31) - 1;
}

flce_status_t flce_vocab_shard_forward(flce_handle_t h, const void* X, const void* W_shard,
                                       const int64_t* targets, int64_t T, int64_t ignore_index,
                                       int64_t vocab_offset, int64_t vocab_total, float* m,
                                       float* sumexp, int32_t* argmax, float* ztarget,
                                       void* stream) {
  if (!h) return FLCE_ERR_INVALID_ARGUMENT;
  if (T < 0 || bad_shard(h, vocab_offset, vocab_total)) return FLCE_ERR_INVALID_ARGUMENT;
  if (!W_shard) return FLCE_ERR_INVALID_ARGUMENT;
  if (T > 0 && (!X || !targets || !m || !sumexp || !ztarget)) return FLCE_ERR_INVALID_ARGUMENT;
  if (!aligned16(W_shard) || (T > 0 && !aligned16(X))) return FLCE_ERR_INVALID_ARGUMENT;
  if (misaligned(m, 3) || misaligned(sumexp, 3) || misaligned(argmax, 3) ||
      misaligned(ztarget, 3) || misaligned(targets, 7))
    return FLCE_ERR_INVALID_ARGUMENT;
  const flce_status_t st = check_device(h, "flce_vocab_shard_forward");
  if (st != FLCE_OK) return st;
  return run_forward(h, X, W_shard, targets, T, ignore_index, FLCE_SUM, nullptr, nullptr, nullptr,
                     argmax, nullptr, m, sumexp, ztarget, Cols{vocab_offset, vocab_total, nullptr},
                     stream);
}

flce_status_t flce_vocab_shard_backward(flce_handle_t h, const void* X, const void* W_shard,
                                        const int64_t* targets, int64_t T, int64_t ignore_index,
                                        int64_t vocab_offset, int64_t vocab_total,
                                        int32_t reduction, const float* lse, void* dX_partial,
                                        float* dW_shard, void* stream) {
  if (!h || h->fwd_only) return FLCE_ERR_INVALID_ARGUMENT;
  if (T < 0 || bad_shard(h, vocab_offset, vocab_total)) return FLCE_ERR_INVALID_ARGUMENT;
  if (reduction != FLCE_MEAN && reduction != FLCE_SUM) return FLCE_ERR_INVALID_ARGUMENT;
  if (!W_shard || !dW_shard) return FLCE_ERR_INVALID_ARGUMENT;
  if (T > 0 && (!X || !targets || !lse || !dX_partial)) return FLCE_ERR_INVALID_ARGUMENT;
  if (!aligned16(W_shard) || !aligned16(dW_shard) ||
      (T > 0 && (!aligned16(X) || !aligned16(dX_partial))))
    return FLCE_ERR_INVALID_ARGUMENT;
  if (misaligned(lse, 3) || misaligned(targets, 7)) return FLCE_ERR_INVALID_ARGUMENT;
  const flce_status_t st = check_device(h, "flce_vocab_shard_backward");
  if (st != FLCE_OK) return st;
  return run_fwd_bwd(h, X, W_shard, targets, T, ignore_index, reduction, nullptr, dX_partial,
                     dW_shard, nullptr, nullptr, nullptr, Cols{vocab_offset, vocab_total, lse},
                     stream);
}

flce_status_t flce_distill_fwd_bwd(flce_handle_t h, const void* X, const void* W,
                                   const void* X_teacher, const void* W_teacher,
                                   const int64_t* targets, int64_t T, int64_t ignore_index,
                                   float temperature, int32_t reduction, float* loss, void* dX,
                                   float* dW, int64_t* n_valid, void* stream) {
  if (!h || h->Ht <= 0) return FLCE_ERR_INVALID_ARGUMENT;
  if (T < 0) return FLCE_ERR_INVALID_ARGUMENT;
  if (!(temperature > 0.f) || !(temperature < 3.0e38f)) return FLCE_ERR_INVALID_ARGUMENT;
  if (reduction != FLCE_MEAN && reduction != FLCE_SUM) return FLCE_ERR_INVALID_ARGUMENT;
  if (!W || !W_teacher || !loss || !dW) return FLCE_ERR_INVALID_ARGUMENT;
  if (T > 0 && (!X || !X_teacher || !targets || !dX)) return FLCE_ERR_INVALID_ARGUMENT;
  if (!aligned16(W) || !aligned16(W_teacher) || !aligned16(dW) ||
      (T > 0 && (!aligned16(X) || !aligned16(X_teacher) || !aligned16(dX))))
    return FLCE_ERR_INVALID_ARGUMENT;
  if (misaligned(loss, 3) || misaligned(n_valid, 7) || misaligned(targets, 7))
    return FLCE_ERR_INVALID_ARGUMENT;
  const flce_status_t st = check_device(h, "flce_distill_fwd_bwd");
  if (st != FLCE_OK) return st;
  const Soft soft{X_teacher, W_teacher, 1.f / temperature};
  return run_fwd_bwd(h, X, W, targets, T, ignore_index, reduction, loss, dX, dW, nullptr, nullptr,
                     n_valid, Cols{0, h->V, nullptr}, stream, &soft);
}

}  // extern "C"

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
char* g_scratch_ptr[kMaxDevices];

// Address of this device's copy of `scratch`, looked up once per device with
// that device current.
flce_status_t scratch_for_device(int dev, char** out) {
  if (dev < 0 || dev >= kMaxDevices) {
    g_last_error = "flce_fwd_bwd_noalloc: device index beyond the library's table";
    return FLCE_ERR_UNSUPPORTED;
  }
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? (char*)p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev])
    return hip_fail(g_scratch_err[dev] != hipSuccess ? g_scratch_err[dev] : hipErrorInvalidSymbol,
                    "hipGetSymbolAddress(scratch)");
  *out = g_scratch_ptr[dev];
  return FLCE_OK;
}

}  // namespace

extern "C" {

flce_status_t flce_fwd_bwd_noalloc(const flce_config_t* cfg, const void* X, const void* W,
                                   const int64_t* targets, int64_t T, int64_t ignore_index,
                                   int32_t reduction, float* loss, void* dX, float* dW, float* lse,
                                   int32_t* argmax, int64_t* n_valid, void* stream) {
  flce_handle h;  // not heap-allocated; its buffers are bound to the scratch
  Layout L;
  flce_status_t st = configure(cfg, 0, &h, &L);
  if (st != FLCE_OK) return st;
  if (h.fwd_only) return FLCE_ERR_INVALID_ARGUMENT;
  st = check_fwd_bwd_args(X, W, targets, T, reduction, loss, dX, dW, lse, argmax, n_valid);
  if (st != FLCE_OK) return st;
  if (L.total > (size_t)FLCE_NOALLOC_SCRATCH_BYTES) {
    char buf[200];
    snprintf(buf, sizeof buf,
             "flce_fwd_bwd_noalloc: this configuration needs %zu bytes of workspace, more than "
             "the %zu-byte static scratch (smaller chunk_tokens or dw_chunks may fit)",
             L.total, (size_t)FLCE_NOALLOC_SCRATCH_BYTES);
    g_last_error = buf;
    return FLCE_ERR_UNSUPPORTED;
  }
  hipError_t e = hipGetDevice(&h.device);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if ((st = ensure_setup()) != FLCE_OK) return st;
  char* base = nullptr;
  if ((st = scratch_for_device(h.device, &base)) != FLCE_OK) return st;
  bind_workspace(&h, L, base);
  // Nothing in the workspace has to start at zero: every buffer a call reads
  // is written earlier in the same call (the target counts, the first
  // chunk's loss partials, the split-K partials).
  return run_fwd_bwd(&h, X, W, targets, T, ignore_index, reduction, loss, dX, dW, lse, argmax,
                     n_valid, Cols{0, h.V, nullptr}, stream);
}

flce_status_t flce_query_error(flce_handle_t h, void* stream, int64_t* bad_targets) {
  if (!h) return FLCE_ERR_INVALID_ARGUMENT;
  int64_t bad = 0;
  hipError_t e = hipMemcpyAsync(&bad, h->bad, sizeof bad, hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "flce_query_error");
  if (bad_targets) *bad_targets = bad;
  return bad > 0 ? FLCE_ERR_BAD_TARGET : FLCE_OK;
}

flce_status_t flce_timing_enable(flce_handle_t h, int32_t enable) {
  if (!h) return FLCE_ERR_INVALID_ARGUMENT;
  flce_status_t st = drain_timing(h);
  if (st != FLCE_OK) return st;
  h->timing = enable != 0;
  if (h->timing) {
    for (int k = 0; k < K_NUM; ++k) {
      h->total_ms[k] = 0.0;
      h->launches[k] = 0;
    }
  }
  return FLCE_OK;
}

flce_status_t flce_timing_read(flce_handle_t h, int32_t kind, double* total_ms, int64_t* launches) {
  if (!h || kind < 0 || kind >= K_NUM) return FLCE_ERR_INVALID_ARGUMENT;
  flce_status_t st = drain_timing(h);
  if (st != FLCE_OK) return st;
  if (total_ms) *total_ms = h->total_ms[kind];
  if (launches) *launches = h->launches[kind];
  return FLCE_OK;
}

}  // extern "C"
