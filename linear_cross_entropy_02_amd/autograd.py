"""PyTorch autograd wrapper around the fused head.

The forward pass runs the whole fused computation (loss, dX and dW for a
loss gradient of 1) in one flce_fwd_bwd call and keeps dX and dW; the
backward pass only scales them by the incoming gradient of the scalar loss,
since the gradients are already finished when the loss is returned
(efficient-llm-anatomy README, Selected insights: fused cross-entropy
computes backward during forward).  Autograd then accumulates them into
`.grad`.

A custom Function is invisible to autocast unless it opts in (same README
and section: autocast does not see Function.apply()), so the forward is
decorated with custom_fwd and casts its floating inputs to bf16 when autocast
is on; dW, computed in fp32, is handed back in W's dtype.

A target that is neither ignore_index nor a vocabulary id is counted on the
device and treated as ignored (the C ABI never synchronises to raise).  With
check_targets=True the forward reads that count back (a stream
synchronisation) and raises ValueError when it is not zero, as PyTorch's own
cross-entropy would.
"""
from __future__ import annotations

import collections
import threading
from typing import Optional

import torch

from . import FLCE_OK, FlceError, FusedLinearCrossEntropy, flce_query_error
from .launch import suggest_launch

# Handles (each owning a workspace of up to a few GB) kept for reuse, the
# least recently used closed beyond this many.
MAX_CACHED_HANDLES = 4

_handles: "collections.OrderedDict" = collections.OrderedDict()
_lock = threading.Lock()


def _handle(device: torch.device, stream: torch.cuda.Stream, H: int, V: int, dtype: str,
            chunk_tokens: int, dw_chunks: int, weight_copy: bool = True,
            forward_only: bool = False) -> FusedLinearCrossEntropy:
    """One handle per (device, stream, shape, dtype, chunking, kind): a handle
    owns its workspace and must not be used by two streams at once."""
    key = (device.index, stream.cuda_stream, H, V, dtype, chunk_tokens, dw_chunks, weight_copy,
           forward_only)
    with _lock:
        op = _handles.get(key)
        if op is None:
            while len(_handles) >= MAX_CACHED_HANDLES:
                _, old = _handles.popitem(last=False)
                # the evicted handle's last call may still run on its stream
                torch.cuda.synchronize(device)
                old.close()
            with torch.cuda.device(device):
                op = FusedLinearCrossEntropy(H, V, dtype, chunk_tokens=chunk_tokens,
                                             dw_chunks=dw_chunks, weight_copy=weight_copy,
                                             forward_only=forward_only)
            _handles[key] = op
        else:
            _handles.move_to_end(key)
        return op


def clear_handle_cache():
    """Free every cached handle's workspace."""
    with _lock:
        if _handles:
            torch.cuda.synchronize()
        for op in _handles.values():
            op.close()
        _handles.clear()


class LinearCrossEntropyFunction(torch.autograd.Function):
    @staticmethod
    @torch.amp.custom_fwd(device_type="cuda", cast_inputs=torch.bfloat16)
    def forward(ctx, X, W, targets, ignore_index: int = -100, reduction: str = "mean",
                chunk_tokens: int = 0, dw_chunks: int = 0, weight_copy: Optional[bool] = None,
                check_targets: bool = False):
        if X.dim() != 2 or W.dim() != 2 or X.shape[1] != W.shape[1]:
            raise ValueError("X must be [T, H] and W [V, H]")
        if X.dtype != W.dtype or X.dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("X and W must share a dtype, bf16 or fp32")
        if reduction not in ("mean", "sum"):
            raise ValueError("reduction must be 'mean' or 'sum'")
        dtype = "bf16" if X.dtype == torch.bfloat16 else "f32"
        X = X.contiguous()
        W = W.contiguous()
        targets = targets.contiguous()
        stream = torch.cuda.current_stream(X.device)
        # unset launch settings: the ones measured fastest for this shape
        C, G, wc = suggest_launch(X.shape[0], X.shape[1], W.shape[0], dtype)
        chunk_tokens = chunk_tokens or C
        dw_chunks = dw_chunks or G
        weight_copy = wc if weight_copy is None else weight_copy
        op = _handle(X.device, stream, X.shape[1], W.shape[0], dtype, chunk_tokens, dw_chunks,
                     weight_copy)
        out = op.fwd_bwd(X, W, targets, ignore_index, reduction)
        if check_targets:
            st, bad = flce_query_error(op.handle, stream.cuda_stream)
            if bad > 0:
                raise ValueError(f"{bad} target(s) are neither ignore_index ({ignore_index}) nor "
                                 f"in [0, {W.shape[0]})")
            if st != FLCE_OK:
                raise FlceError(st, "flce_query_error")
        ctx.save_for_backward(out["dX"], out["dW"])
        ctx.w_dtype = W.dtype
        ctx.mark_non_differentiable(out["lse"])
        return out["loss"], out["lse"]

    @staticmethod
    @torch.amp.custom_bwd(device_type="cuda")
    def backward(ctx, grad_loss, grad_lse):
        dX, dW = ctx.saved_tensors
        g = grad_loss.to(torch.float32)
        gX = (dX.to(torch.float32) * g).to(dX.dtype) if ctx.needs_input_grad[0] else None
        gW = (dW * g).to(ctx.w_dtype) if ctx.needs_input_grad[1] else None
        return gX, gW, None, None, None, None, None, None, None


# Chunk of the forward-only handle that evaluation calls use: its workspace
# is the merge's partials alone, and 8192-token chunks measured fastest at
# the 16384 x 4096 x 128256 head.
FORWARD_CHUNK = 8192


def _forward_only(X, W, targets, ignore_index, reduction, chunk_tokens, check_targets):
    """Loss and lse without gradients: the forward-only call on a
    forward-only handle (a third of the work, no backward workspace)."""
    if torch.is_autocast_enabled("cuda"):
        X, W = X.to(torch.bfloat16), W.to(torch.bfloat16)
    if X.dim() != 2 or W.dim() != 2 or X.shape[1] != W.shape[1]:
        raise ValueError("X must be [T, H] and W [V, H]")
    if X.dtype != W.dtype or X.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("X and W must share a dtype, bf16 or fp32")
    if reduction not in ("mean", "sum"):
        raise ValueError("reduction must be 'mean' or 'sum'")
    dtype = "bf16" if X.dtype == torch.bfloat16 else "f32"
    X, W, targets = X.contiguous(), W.contiguous(), targets.contiguous()
    stream = torch.cuda.current_stream(X.device)
    tpad = max(256, -(-max(X.shape[0], 1) // 256) * 256)
    C = chunk_tokens or min(FORWARD_CHUNK, tpad)
    op = _handle(X.device, stream, X.shape[1], W.shape[0], dtype, C, 1, False, forward_only=True)
    out = op.forward(X, W, targets, ignore_index, reduction)
    if check_targets:
        st, bad = flce_query_error(op.handle, stream.cuda_stream)
        if bad > 0:
            raise ValueError(f"{bad} target(s) are neither ignore_index ({ignore_index}) nor "
                             f"in [0, {W.shape[0]})")
        if st != FLCE_OK:
            raise FlceError(st, "flce_query_error")
    return out["loss"], out["lse"]


def linear_cross_entropy(X: torch.Tensor, W: torch.Tensor, targets: torch.Tensor,
                         ignore_index: int = -100, reduction: str = "mean",
                         chunk_tokens: int = 0, dw_chunks: int = 0,
                         return_lse: bool = False, weight_copy: Optional[bool] = None,
                         check_targets: bool = False):
    """Cross-entropy of softmax(X W^T) against `targets`, fused: the T x V
    logits are never formed.  Returns the scalar loss (and the per-token
    log-sum-exp when `return_lse`); gradients reach X and W through
    autograd.  Launch settings left at 0 / None (chunk_tokens, dw_chunks,
    weight_copy) come from launch.suggest_launch for the shape: the fastest
    measured.  weight_copy=False (bf16) has the dX contraction read W as
    stored instead of a transposed copy made per call, for less memory.
    check_targets=True raises ValueError for a target outside [0, V) that
    is not ignore_index (one stream synchronisation per call); otherwise
    such tokens are ignored.  When no gradient is wanted (grad mode off, or
    neither X nor W requires one) only the forward runs, on a handle made
    for it (FLCE_FLAG_FORWARD_ONLY)."""
    if not (torch.is_grad_enabled() and (X.requires_grad or W.requires_grad)):
        loss, lse = _forward_only(X, W, targets, ignore_index, reduction, chunk_tokens,
                                  check_targets)
    else:
        loss, lse = LinearCrossEntropyFunction.apply(X, W, targets, ignore_index, reduction,
                                                     chunk_tokens, dw_chunks, weight_copy,
                                                     check_targets)
    return (loss, lse) if return_lse else loss


class LinearCrossEntropy(torch.nn.Module):
    """An lm_head with a fused cross-entropy loss: holds W ([V, H]) and maps
    hidden states and targets to the loss."""

    def __init__(self, hidden: int, vocab: int, dtype=torch.bfloat16, device="cuda",
                 ignore_index: int = -100, reduction: str = "mean", chunk_tokens: int = 0,
                 check_targets: bool = False):
        super().__init__()
        self.weight = torch.nn.Parameter(torch.empty(vocab, hidden, dtype=dtype, device=device))
        torch.nn.init.normal_(self.weight, std=hidden ** -0.5)
        self.ignore_index = ignore_index
        self.reduction = reduction
        self.chunk_tokens = chunk_tokens
        self.check_targets = check_targets

    def forward(self, hidden_states: torch.Tensor, targets: torch.Tensor) -> torch.Tensor:
        X = hidden_states.reshape(-1, hidden_states.shape[-1])
        return linear_cross_entropy(X, self.weight, targets.reshape(-1), self.ignore_index,
                                    self.reduction, self.chunk_tokens,
                                    check_targets=self.check_targets)
