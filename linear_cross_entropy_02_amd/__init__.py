"""Python binding of libflce (fused linear cross-entropy head for MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/flce.h.  PyTorch supplies device
memory and the current stream.  The binding refuses to work without the built
library -- there is no fallback path.

Entry points mirror the C names (flce_create, flce_fwd_bwd, flce_destroy,
flce_query_error, flce_workspace_bytes, flce_status_string, timing calls);
`FusedLinearCrossEntropy` wraps a handle and allocates the outputs.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libflce.so")

FLCE_OK = 0
FLCE_ERR_INVALID_ARGUMENT = 1
FLCE_ERR_UNSUPPORTED = 2
FLCE_ERR_HIP = 3
FLCE_ERR_OUT_OF_MEMORY = 4
FLCE_ERR_BAD_TARGET = 5

FLCE_F32 = 0
FLCE_BF16 = 1
FLCE_MEAN = 1
FLCE_SUM = 2

EXPORTED = (
    "flce_create", "flce_workspace_bytes", "flce_chunk_tokens", "flce_dw_chunks", "flce_fwd_bwd",
    "flce_fwd_bwd_noalloc", "flce_forward",
    "flce_vocab_shard_forward", "flce_vocab_shard_backward", "flce_distill_create",
    "flce_distill_fwd_bwd",
    "flce_query_error", "flce_timing_enable", "flce_timing_kinds", "flce_timing_kind_name",
    "flce_timing_read", "flce_destroy", "flce_status_string", "flce_last_error",
)


class flce_config_t(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int64), ("vocab", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("dw_chunks", ctypes.c_int32),
                ("chunk_tokens", ctypes.c_int64), ("flags", ctypes.c_int32)]


FLCE_FLAG_NO_WEIGHT_COPY = 1
FLCE_FLAG_DZ_IN_PLACE = 2
FLCE_FLAG_FORWARD_ONLY = 4


class FlceError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} {last_error()}".rstrip())


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libflce.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m linear_cross_entropy_02_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i64, i32, st = ctypes.c_int64, ctypes.c_int32, ctypes.c_int
    lib.flce_create.argtypes = [ctypes.POINTER(flce_config_t), ctypes.POINTER(P)]
    lib.flce_create.restype = st
    lib.flce_workspace_bytes.argtypes = [P]
    lib.flce_workspace_bytes.restype = ctypes.c_size_t
    lib.flce_chunk_tokens.argtypes = [P]
    lib.flce_chunk_tokens.restype = i64
    lib.flce_dw_chunks.argtypes = [P]
    lib.flce_dw_chunks.restype = i32
    lib.flce_fwd_bwd.argtypes = [P, P, P, P, i64, i64, i32, P, P, P, P, P, P, P]
    lib.flce_fwd_bwd.restype = st
    lib.flce_fwd_bwd_noalloc.argtypes = [ctypes.POINTER(flce_config_t), P, P, P, i64, i64, i32, P,
                                         P, P, P, P, P, P]
    lib.flce_fwd_bwd_noalloc.restype = st
    lib.flce_forward.argtypes = [P, P, P, P, i64, i64, i32, P, P, P, P, P, P]
    lib.flce_forward.restype = st
    lib.flce_vocab_shard_forward.argtypes = [P, P, P, P, i64, i64, i64, i64, P, P, P, P, P]
    lib.flce_vocab_shard_forward.restype = st
    lib.flce_vocab_shard_backward.argtypes = [P, P, P, P, i64, i64, i64, i64, i32, P, P, P, P]
    lib.flce_vocab_shard_backward.restype = st
    lib.flce_distill_create.argtypes = [ctypes.POINTER(flce_config_t), i64, ctypes.POINTER(P)]
    lib.flce_distill_create.restype = st
    lib.flce_distill_fwd_bwd.argtypes = [P, P, P, P, P, P, i64, i64, ctypes.c_float, i32, P, P, P,
                                         P, P]
    lib.flce_distill_fwd_bwd.restype = st
    lib.flce_query_error.argtypes = [P, P, ctypes.POINTER(i64)]
    lib.flce_query_error.restype = st
    lib.flce_timing_enable.argtypes = [P, i32]
    lib.flce_timing_enable.restype = st
    lib.flce_timing_kinds.argtypes = []
    lib.flce_timing_kinds.restype = i32
    lib.flce_timing_kind_name.argtypes = [i32]
    lib.flce_timing_kind_name.restype = ctypes.c_char_p
    lib.flce_timing_read.argtypes = [P, i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
    lib.flce_timing_read.restype = st
    lib.flce_destroy.argtypes = [P]
    lib.flce_destroy.restype = st
    lib.flce_status_string.argtypes = [st]
    lib.flce_status_string.restype = ctypes.c_char_p
    lib.flce_last_error.argtypes = []
    lib.flce_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().flce_status_string(status).decode()


def last_error() -> str:
    return load().flce_last_error().decode()


# ------------------------------------------------------------ C-name calls ---
def flce_create(hidden: int, vocab: int, dtype: int, chunk_tokens: int = 0, dw_chunks: int = 0,
                flags: int = 0):
    """Returns (status, handle)."""
    cfg = flce_config_t(hidden, vocab, dtype, dw_chunks, chunk_tokens, flags)
    h = ctypes.c_void_p()
    st = load().flce_create(ctypes.byref(cfg), ctypes.byref(h))
    return st, h


def flce_destroy(handle) -> int:
    return load().flce_destroy(handle)


def flce_workspace_bytes(handle) -> int:
    return load().flce_workspace_bytes(handle)


def flce_chunk_tokens(handle) -> int:
    return load().flce_chunk_tokens(handle)


def flce_dw_chunks(handle) -> int:
    return load().flce_dw_chunks(handle)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def flce_fwd_bwd(handle, X, W, targets, T: int, ignore_index: int, reduction: int,
                 loss, dX, dW, lse=None, argmax=None, n_valid=None, stream=None) -> int:
    """Direct call: tensors (or raw device addresses as ints) are passed as
    pointers; `stream` is a hipStream_t handle (int) or None for torch's
    current stream."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    return load().flce_fwd_bwd(handle, _ptr(X), _ptr(W), _ptr(targets), T, ignore_index,
                               reduction, _ptr(loss), _ptr(dX), _ptr(dW), _ptr(lse),
                               _ptr(argmax), _ptr(n_valid), stream)


# Bytes of the static device scratch flce_fwd_bwd_noalloc works in (one copy
# per GPU, held by the library until the process ends).
FLCE_NOALLOC_SCRATCH_BYTES = 128 << 20


def flce_fwd_bwd_noalloc(hidden: int, vocab: int, dtype: int, X, W, targets, T: int,
                         ignore_index: int, reduction: int, loss, dX, dW, lse=None, argmax=None,
                         n_valid=None, chunk_tokens: int = 0, dw_chunks: int = 0, flags: int = 0,
                         stream=None) -> int:
    """Direct call of the allocation-free entry point: the configuration is
    passed with the call instead of a handle (see flce_fwd_bwd for the
    tensors)."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    cfg = flce_config_t(hidden, vocab, dtype, dw_chunks, chunk_tokens, flags)
    return load().flce_fwd_bwd_noalloc(ctypes.byref(cfg), _ptr(X), _ptr(W), _ptr(targets), T,
                                       ignore_index, reduction, _ptr(loss), _ptr(dX), _ptr(dW),
                                       _ptr(lse), _ptr(argmax), _ptr(n_valid), stream)


def flce_forward(handle, X, W, targets, T: int, ignore_index: int, reduction: int,
                 loss=None, token_logprob=None, lse=None, argmax=None, n_valid=None,
                 stream=None) -> int:
    """Direct call of the forward-only entry point (see flce_fwd_bwd)."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    return load().flce_forward(handle, _ptr(X), _ptr(W), _ptr(targets), T, ignore_index,
                               reduction, _ptr(loss), _ptr(token_logprob), _ptr(lse),
                               _ptr(argmax), _ptr(n_valid), stream)


def flce_vocab_shard_forward(handle, X, W_shard, targets, T: int, ignore_index: int,
                             vocab_offset: int, vocab_total: int, m, sumexp, argmax, ztarget,
                             stream=None) -> int:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    return load().flce_vocab_shard_forward(handle, _ptr(X), _ptr(W_shard), _ptr(targets), T,
                                           ignore_index, vocab_offset, vocab_total, _ptr(m),
                                           _ptr(sumexp), _ptr(argmax), _ptr(ztarget), stream)


def flce_vocab_shard_backward(handle, X, W_shard, targets, T: int, ignore_index: int,
                              vocab_offset: int, vocab_total: int, reduction: int, lse,
                              dX_partial, dW_shard, stream=None) -> int:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    return load().flce_vocab_shard_backward(handle, _ptr(X), _ptr(W_shard), _ptr(targets), T,
                                            ignore_index, vocab_offset, vocab_total, reduction,
                                            _ptr(lse), _ptr(dX_partial), _ptr(dW_shard), stream)


def flce_distill_create(hidden: int, vocab: int, dtype: int, teacher_hidden: int,
                        chunk_tokens: int = 0, dw_chunks: int = 0, flags: int = 0):
    """Returns (status, handle) of a soft-target handle."""
    cfg = flce_config_t(hidden, vocab, dtype, dw_chunks, chunk_tokens, flags)
    h = ctypes.c_void_p()
    st = load().flce_distill_create(ctypes.byref(cfg), teacher_hidden, ctypes.byref(h))
    return st, h


def flce_distill_fwd_bwd(handle, X, W, X_teacher, W_teacher, targets, T: int, ignore_index: int,
                         temperature: float, reduction: int, loss, dX, dW, n_valid=None,
                         stream=None) -> int:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    return load().flce_distill_fwd_bwd(handle, _ptr(X), _ptr(W), _ptr(X_teacher), _ptr(W_teacher),
                                       _ptr(targets), T, ignore_index, temperature, reduction,
                                       _ptr(loss), _ptr(dX), _ptr(dW), _ptr(n_valid), stream)


def flce_query_error(handle, stream=None):
    """Synchronises the stream; returns (status, bad_targets)."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    bad = ctypes.c_int64(0)
    st = load().flce_query_error(handle, stream, ctypes.byref(bad))
    return st, bad.value


def flce_timing_enable(handle, enable: bool) -> int:
    return load().flce_timing_enable(handle, 1 if enable else 0)


def flce_timing_kinds() -> list:
    lib = load()
    return [lib.flce_timing_kind_name(k).decode() for k in range(lib.flce_timing_kinds())]


def flce_timing_read(handle, kind: int):
    """Returns (total_ms, launches) for one kernel class."""
    ms = ctypes.c_double(0)
    n = ctypes.c_int64(0)
    st = load().flce_timing_read(handle, kind, ctypes.byref(ms), ctypes.byref(n))
    if st != FLCE_OK:
        raise FlceError(st, "flce_timing_read")
    return ms.value, n.value


# ------------------------------------------------------------ torch facade ---
class FusedLinearCrossEntropy:
    """A handle for fixed (H, V, dtype, chunk, dW group) plus output allocation.

    fwd_bwd(X, W, y) returns a dict of device tensors: loss (float32 scalar),
    dX (X's dtype), dW (float32), lse (float32 [T]), argmax (int32 [T]) and
    n_valid (int64 scalar).  Gradients are for a loss gradient seed of 1.
    forward_only=True makes a handle for forward() and shard_forward() alone
    (FLCE_FLAG_FORWARD_ONLY: a workspace of the merge's partials only).
    """

    def __init__(self, hidden: int, vocab: int, dtype="bf16", chunk_tokens: int = 0,
                 dw_chunks: int = 0, weight_copy: bool = True, dz_in_place: bool = False,
                 forward_only: bool = False):
        import torch
        if not torch.cuda.is_available():
            raise RuntimeError("FusedLinearCrossEntropy needs a HIP device")
        self.torch_dtype = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
        self.dtype = FLCE_BF16 if dtype == "bf16" else FLCE_F32
        self.hidden, self.vocab = hidden, vocab
        flags = (0 if weight_copy else FLCE_FLAG_NO_WEIGHT_COPY) | \
            (FLCE_FLAG_DZ_IN_PLACE if dz_in_place else 0) | \
            (FLCE_FLAG_FORWARD_ONLY if forward_only else 0)
        st, h = flce_create(hidden, vocab, self.dtype, chunk_tokens, dw_chunks, flags)
        if st != FLCE_OK:
            raise FlceError(st, "flce_create")
        self.handle = h

    @property
    def workspace_bytes(self) -> int:
        return flce_workspace_bytes(self.handle)

    @property
    def chunk_tokens(self) -> int:
        return flce_chunk_tokens(self.handle)

    @property
    def dw_chunks(self) -> int:
        return flce_dw_chunks(self.handle)

    def close(self):
        if getattr(self, "handle", None):
            flce_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def alloc_outputs(self, T: int, device):
        import torch
        return dict(
            loss=torch.empty((), dtype=torch.float32, device=device),
            dX=torch.empty((T, self.hidden), dtype=self.torch_dtype, device=device),
            dW=torch.empty((self.vocab, self.hidden), dtype=torch.float32, device=device),
            lse=torch.empty((T,), dtype=torch.float32, device=device),
            argmax=torch.empty((T,), dtype=torch.int32, device=device),
            n_valid=torch.empty((), dtype=torch.int64, device=device),
        )

    def fwd_bwd(self, X, W, y, ignore_index: int = -100, reduction: str = "mean", out=None):
        T = X.shape[0] if X is not None else 0
        self._check(X, W, y, T)
        if out is None:
            out = self.alloc_outputs(T, W.device)
        else:
            for k in ("loss", "dX", "dW"):
                if out.get(k) is None:
                    raise ValueError(f"out[{k!r}] is required")
            self._check_out(out, self._out_spec(T), W.device)
        red = FLCE_MEAN if reduction == "mean" else FLCE_SUM if reduction == "sum" else -1
        st = flce_fwd_bwd(self.handle, X, W, y, T, ignore_index, red, out["loss"], out["dX"],
                          out["dW"], out.get("lse"), out.get("argmax"), out.get("n_valid"))
        if st != FLCE_OK:
            raise FlceError(st, "flce_fwd_bwd")
        return out

    def forward(self, X, W, y, ignore_index: int = -100, reduction: str = "mean", out=None):
        """Forward only: loss, per-token log-prob of the target (0 where
        ignored), lse, argmax and n_valid, without gradients."""
        import torch
        T = X.shape[0] if X is not None else 0
        self._check(X, W, y, T)
        if out is None:
            dev = W.device
            out = dict(
                loss=torch.empty((), dtype=torch.float32, device=dev),
                token_logprob=torch.empty((T,), dtype=torch.float32, device=dev),
                lse=torch.empty((T,), dtype=torch.float32, device=dev),
                argmax=torch.empty((T,), dtype=torch.int32, device=dev),
                n_valid=torch.empty((), dtype=torch.int64, device=dev),
            )
        else:
            self._check_out(out, self._out_spec(T), W.device)
        red = FLCE_MEAN if reduction == "mean" else FLCE_SUM if reduction == "sum" else -1
        st = flce_forward(self.handle, X, W, y, T, ignore_index, red, out.get("loss"),
                          out.get("token_logprob"), out.get("lse"), out.get("argmax"),
                          out.get("n_valid"))
        if st != FLCE_OK:
            raise FlceError(st, "flce_forward")
        return out

    def shard_forward(self, X, W_shard, y, vocab_offset: int, vocab_total: int,
                      ignore_index: int = -100):
        """Vocabulary shard, step 1: per-token (m, sumexp, global argmax,
        ztarget) of this shard's columns."""
        import torch
        T = X.shape[0]
        self._check(X, W_shard, y, T)
        dev = W_shard.device
        out = {k: torch.empty((T,), dtype=torch.float32, device=dev)
               for k in ("m", "sumexp", "ztarget")}
        out["argmax"] = torch.empty((T,), dtype=torch.int32, device=dev)
        st = flce_vocab_shard_forward(self.handle, X, W_shard, y, T, ignore_index, vocab_offset,
                                      vocab_total, out["m"], out["sumexp"], out["argmax"],
                                      out["ztarget"])
        if st != FLCE_OK:
            raise FlceError(st, "flce_vocab_shard_forward")
        return out

    def shard_backward(self, X, W_shard, y, lse, vocab_offset: int, vocab_total: int,
                       ignore_index: int = -100, reduction: str = "mean"):
        """Vocabulary shard, step 2: this shard's dX contribution and its rows
        of dW, given the whole vocabulary's lse."""
        import torch
        T = X.shape[0]
        self._check(X, W_shard, y, T)
        self._check_out({"lse": lse}, self._out_spec(T), W_shard.device)
        dX = torch.empty((T, self.hidden), dtype=self.torch_dtype, device=X.device)
        dW = torch.empty((self.vocab, self.hidden), dtype=torch.float32, device=X.device)
        red = FLCE_MEAN if reduction == "mean" else FLCE_SUM if reduction == "sum" else -1
        st = flce_vocab_shard_backward(self.handle, X, W_shard, y, T, ignore_index, vocab_offset,
                                       vocab_total, red, lse, dX, dW)
        if st != FLCE_OK:
            raise FlceError(st, "flce_vocab_shard_backward")
        return dX, dW

    def _check(self, X, W, y, T):
        if W.dtype != self.torch_dtype or tuple(W.shape) != (self.vocab, self.hidden):
            raise ValueError("W must be [V, H] in the handle's dtype")
        if not W.is_contiguous():
            raise ValueError("W must be contiguous")
        if T:
            if (X.dtype != self.torch_dtype or X.dim() != 2 or X.shape[1] != self.hidden
                    or not X.is_contiguous()):
                raise ValueError("X must be a contiguous [T, H] tensor in the handle's dtype")
            if (y.dtype.is_floating_point or y.element_size() != 8 or tuple(y.shape) != (T,)
                    or not y.is_contiguous()):
                raise ValueError("targets must be a contiguous int64 [T] tensor")
            if X.device != W.device or y.device != W.device:
                raise ValueError("X, W and the targets must be on one device")

    @staticmethod
    def _check_out(out, spec, device):
        """Caller-supplied output buffers: each present entry must have the
        shape and dtype the call writes, be contiguous and sit on `device`
        (the library writes the full extent without further checks)."""
        for name, (shape, dtype) in spec.items():
            t = out.get(name)
            if t is None:
                continue
            if (tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous()
                    or t.device != device):
                raise ValueError(f"out[{name!r}] must be a contiguous {dtype} tensor of shape "
                                 f"{tuple(shape)} on {device}")

    def _out_spec(self, T):
        import torch
        return dict(loss=((), torch.float32), dX=((T, self.hidden), self.torch_dtype),
                    dW=((self.vocab, self.hidden), torch.float32), lse=((T,), torch.float32),
                    argmax=((T,), torch.int32), n_valid=((), torch.int64),
                    token_logprob=((T,), torch.float32))


class FusedDistillationCrossEntropy(FusedLinearCrossEntropy):
    """Soft-target handle: the student head's tempered softmax against a
    teacher head's, both evaluated on the fly (see flce_distill_fwd_bwd)."""

    def __init__(self, hidden: int, vocab: int, teacher_hidden: int, dtype="bf16",
                 chunk_tokens: int = 0, dw_chunks: int = 0, weight_copy: bool = True):
        import torch
        if not torch.cuda.is_available():
            raise RuntimeError("FusedDistillationCrossEntropy needs a HIP device")
        self.torch_dtype = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
        self.dtype = FLCE_BF16 if dtype == "bf16" else FLCE_F32
        self.hidden, self.vocab, self.teacher_hidden = hidden, vocab, teacher_hidden
        flags = 0 if weight_copy else FLCE_FLAG_NO_WEIGHT_COPY
        st, h = flce_distill_create(hidden, vocab, self.dtype, teacher_hidden, chunk_tokens,
                                    dw_chunks, flags)
        if st != FLCE_OK:
            raise FlceError(st, "flce_distill_create")
        self.handle = h

    def distill(self, X, W, X_teacher, W_teacher, y, temperature: float = 1.0,
                ignore_index: int = -100, reduction: str = "mean", out=None):
        import torch
        T = X.shape[0]
        self._check(X, W, y, T)
        if (X_teacher.dtype != self.torch_dtype or tuple(X_teacher.shape) != (T, self.teacher_hidden)
                or tuple(W_teacher.shape) != (self.vocab, self.teacher_hidden)
                or W_teacher.dtype != self.torch_dtype or not X_teacher.is_contiguous()
                or not W_teacher.is_contiguous()):
            raise ValueError("teacher tensors must be contiguous [T, Ht] and [V, Ht] "
                             "in the handle's dtype")
        if out is None:
            dev = W.device
            out = dict(loss=torch.empty((), dtype=torch.float32, device=dev),
                       dX=torch.empty((T, self.hidden), dtype=self.torch_dtype, device=dev),
                       dW=torch.empty((self.vocab, self.hidden), dtype=torch.float32, device=dev),
                       n_valid=torch.empty((), dtype=torch.int64, device=dev))
        else:
            for k in ("loss", "dX", "dW"):
                if out.get(k) is None:
                    raise ValueError(f"out[{k!r}] is required")
            self._check_out(out, self._out_spec(T), W.device)
        if X_teacher.device != W.device or W_teacher.device != W.device:
            raise ValueError("teacher tensors must be on the student's device")
        red = FLCE_MEAN if reduction == "mean" else FLCE_SUM if reduction == "sum" else -1
        st = flce_distill_fwd_bwd(self.handle, X, W, X_teacher, W_teacher, y, T, ignore_index,
                                  float(temperature), red, out["loss"], out["dX"], out["dW"],
                                  out.get("n_valid"))
        if st != FLCE_OK:
            raise FlceError(st, "flce_distill_fwd_bwd")
        return out
