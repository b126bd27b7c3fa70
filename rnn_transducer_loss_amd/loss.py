"""PyTorch front end of librnnt: ``rnnt_loss`` with autograd, and a low-level call.

Signature and semantics follow the rnnt-loss-ascend README (parameter table,
usage example): ``rnnt_loss(logits, targets, logit_lengths, target_lengths,
blank=-1, clamp=-1.0, reduction="mean", fused_log_softmax=True)`` on packed
``(sum_i T_i*(U_i+1), V)`` logits; ``loss.backward()`` fills ``logits.grad``.
Padded ``(B, max_T, max_U+1, V)`` logits (the layout of warp-transducer /
GPURNNT style pipelines) are accepted as well; their gradient is zero at the
padding positions.

This module only marshals arguments.  The loss, the gradient, the reduction
and the backward scaling all run in librnnt's kernels on the current HIP
stream; PyTorch provides the device buffers.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib

_DTYPES = {torch.float32: _lib.RNNT_F32, torch.float16: _lib.RNNT_F16}


def _dtype_code(dt: torch.dtype) -> int:
    if dt not in _DTYPES:
        raise ValueError(f"logits must be float32 or float16, got {dt}")
    return _DTYPES[dt]


# The current HIP stream of a device as a raw handle (torch's own accessor
# where it has one: it skips building a Stream object on every call).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(dev: torch.device) -> int:
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    if _raw_stream is not None:
        return _raw_stream(idx)
    return torch.cuda.current_stream(dev).cuda_stream


def _prepare(logits: torch.Tensor, targets: torch.Tensor):
    if not isinstance(logits, torch.Tensor) or logits.dim() not in (2, 4):
        raise ValueError("logits must be a packed 2-D (sum_i T_i*(U_i+1), V) or a padded 4-D "
                         "(B, max_T, max_U+1, V) tensor")
    if logits.device.type != "cuda":
        raise ValueError("logits must be on a GPU device")
    if not logits.is_contiguous():
        raise ValueError("logits must be contiguous")
    if targets.dim() == 1:
        targets = targets.unsqueeze(0)
    if targets.dim() != 2:
        raise ValueError("targets must be a 2-D (B, S) tensor")
    if targets.dtype == torch.int32 and targets.device == logits.device and targets.is_contiguous():
        return targets
    return targets.to(device=logits.device, dtype=torch.int32).contiguous()


class _on_device:
    """Makes ``dev`` the current device for the block, unless it already is (the common case costs nothing)."""
    __slots__ = ("ctx",)

    def __init__(self, dev: torch.device):
        idx = dev.index if dev.index is not None else torch.cuda.current_device()
        self.ctx = None if idx == torch.cuda.current_device() else torch.cuda.device(idx)

    def __enter__(self):
        if self.ctx is not None:
            self.ctx.__enter__()

    def __exit__(self, *exc):
        if self.ctx is not None:
            self.ctx.__exit__(*exc)
        return False


def workspace_bytes(logits: torch.Tensor, logit_lengths, target_lengths) -> int:
    T = _lib.host_i32(logit_lengths)
    U = _lib.host_i32(target_lengths)
    if logits.dim() == 4:
        return _lib.workspace_size_padded(len(T), logits.shape[3], logits.shape[1], logits.shape[2],
                                          _dtype_code(logits.dtype), T, U)
    return _lib.workspace_size(len(T), logits.shape[1], logits.shape[0], _dtype_code(logits.dtype), T, U)


def rnnt_loss_fused(logits: torch.Tensor, targets: torch.Tensor, logit_lengths, target_lengths, blank: int = -1,
                    clamp: float = -1.0, reduction: str = "mean", fused_log_softmax: bool = True,
                    compute_grad: bool = True, grad: Optional[torch.Tensor] = None, inplace: bool = False,
                    workspace: Optional[torch.Tensor] = None, loss: Optional[torch.Tensor] = None,
                    loss_reduced: Optional[torch.Tensor] = None, fastemit_lambda: float = 0.0):
    """One librnnt call.  Returns ``(loss, loss_reduced, grad, workspace)``.

    ``loss`` is the fp32 per-sample loss (B,), ``loss_reduced`` a (1,) fp32
    tensor for mean/sum (None for none).  ``grad`` is d(reduced loss)/d(logits)
    for a unit upstream gradient (clamped per sample, times 1/B for mean), in
    the logits dtype; with ``inplace=True`` it is written over ``logits``.
    ``fastemit_lambda >= 0`` weights the label-emission derivatives by
    (1 + lambda) (FastEmit); the loss value does not depend on it.
    Buffers may be passed in to avoid allocation (the bench does).
    """
    tg = _prepare(logits, targets)
    T = _lib.host_i32(logit_lengths)
    U = _lib.host_i32(target_lengths)
    B = len(T)
    if len(U) != B:
        raise ValueError("logit_lengths and target_lengths must have the same length")
    dev = logits.device
    code = _dtype_code(logits.dtype)
    padded = logits.dim() == 4
    if padded:
        if logits.shape[0] != B:
            raise ValueError("padded logits must have one (max_T, max_U+1, V) block per sample")
        max_T, max_U1, V = logits.shape[1], logits.shape[2], logits.shape[3]
    else:
        N, V = logits.shape
    if workspace is None:  # a caller's workspace is checked by the library itself
        need = (_lib.workspace_size_padded(B, V, max_T, max_U1, code, T, U) if padded
                else _lib.workspace_size(B, V, N, code, T, U))
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    if loss is None:
        loss = torch.empty(B, dtype=torch.float32, device=dev)
    if reduction != "none" and loss_reduced is None:
        loss_reduced = torch.empty(1, dtype=torch.float32, device=dev)
    if compute_grad:
        if inplace:
            grad = logits
        elif grad is None:
            grad = torch.empty_like(logits)
        elif grad.shape != logits.shape or grad.dtype != logits.dtype or not grad.is_contiguous():
            raise ValueError("grad must match logits in shape and dtype and be contiguous")
    else:
        grad = None
    with _on_device(dev):
        stream = _stream_handle(dev)
        tgp = tg.data_ptr() if tg.numel() else 0
        redp = loss_reduced.data_ptr() if reduction != "none" else 0
        gp = grad.data_ptr() if grad is not None else 0
        if padded:
            _lib.loss_padded(logits.data_ptr(), code, max_T, max_U1, V, tgp, tg.shape[1], T, U, blank, clamp,
                             fused_log_softmax, reduction, loss.data_ptr(), redp, gp, workspace.data_ptr(),
                             workspace.numel(), stream, fastemit_lambda)
        else:
            _lib.loss_fused(logits.data_ptr(), code, N, V, tgp, tg.shape[1], T, U, blank, clamp, fused_log_softmax,
                            reduction, loss.data_ptr(), redp, gp, workspace.data_ptr(), workspace.numel(), stream,
                            fastemit_lambda)
    return loss, (loss_reduced if reduction != "none" else None), grad, workspace


def device_flags(workspace: torch.Tensor) -> int:
    """RNNT_DEV_* bits of the last call on ``workspace`` (synchronises the current stream)."""
    with torch.cuda.device(workspace.device):
        return _lib.device_flags(workspace.data_ptr(), _stream_handle(workspace.device))


class _RNNTLossFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, logits, targets, logit_lengths, target_lengths, blank, clamp, reduction, fused_log_softmax,
                fastemit_lambda):
        T = _lib.host_i32(logit_lengths)
        U = _lib.host_i32(target_lengths)
        loss, loss_red, grad, ws = rnnt_loss_fused(logits, targets, T, U, blank, clamp, reduction, fused_log_softmax,
                                                   compute_grad=logits.requires_grad,
                                                   fastemit_lambda=fastemit_lambda)
        ctx.meta = (T, U, reduction, logits.shape, logits.dtype)
        ctx.used = False
        if grad is not None:
            ctx.save_for_backward(grad, ws)
        return loss if reduction == "none" else loss_red.reshape(())

    @staticmethod
    def backward(ctx, grad_out):
        T, U, reduction, shape, dtype = ctx.meta
        if not ctx.saved_tensors:
            return (None,) * 9
        if ctx.used:
            raise RuntimeError("rnnt_loss backward was already run for this forward call")
        ctx.used = True
        grad, ws = ctx.saved_tensors
        scale = grad_out.detach()
        if scale.dtype != torch.float32 or scale.device != grad.device or not scale.is_contiguous():
            scale = scale.to(device=grad.device, dtype=torch.float32).contiguous()
        scale = scale.reshape(-1)
        with _on_device(grad.device):
            stream = _stream_handle(grad.device)
            if len(shape) == 4:
                _lib.grad_scale_padded(grad.data_ptr(), _dtype_code(dtype), shape[1], shape[2], shape[3], T, U,
                                       scale.data_ptr(), reduction == "none", ws.data_ptr(), ws.numel(), stream)
            else:
                _lib.grad_scale(grad.data_ptr(), _dtype_code(dtype), shape[0], shape[1], T, U, scale.data_ptr(),
                                reduction == "none", ws.data_ptr(), ws.numel(), stream)
        return grad, None, None, None, None, None, None, None, None


def rnnt_loss(logits: torch.Tensor, targets: torch.Tensor, logit_lengths, target_lengths, blank: int = -1,
              clamp: float = -1.0, reduction: str = "mean", fused_log_softmax: bool = True,
              fastemit_lambda: float = 0.0) -> torch.Tensor:
    """RNN-T loss over packed (or padded 4-D) logits; differentiable with respect to ``logits``.

    ``blank`` in [-V, V-1] (negative counts from the end), ``clamp > 0`` clips
    each gradient element to [-clamp, clamp], ``reduction`` is none (per
    sample, fp32 (B,)), mean (over the batch) or sum.  With
    ``fused_log_softmax=False`` the inputs are taken as log-probabilities.
    ``fastemit_lambda >= 0`` is the FastEmit regularisation weight: the
    backward pass weights every label emission's derivative by
    (1 + fastemit_lambda); the returned loss is the plain one.
    """
    if reduction not in ("none", "mean", "sum"):
        raise ValueError(f"reduction must be none, mean or sum, got {reduction!r}")
    return _RNNTLossFunction.apply(logits, targets, logit_lengths, target_lengths, int(blank), float(clamp),
                                   reduction, bool(fused_log_softmax), float(fastemit_lambda))


class RNNTLoss(torch.nn.Module):
    """Module form of :func:`rnnt_loss` with the attributes fixed at construction."""

    def __init__(self, blank: int = -1, clamp: float = -1.0, reduction: str = "mean",
                 fused_log_softmax: bool = True, fastemit_lambda: float = 0.0):
        super().__init__()
        self.blank, self.clamp, self.reduction, self.fused_log_softmax = blank, clamp, reduction, fused_log_softmax
        self.fastemit_lambda = fastemit_lambda

    def forward(self, logits, targets, logit_lengths, target_lengths):
        return rnnt_loss(logits, targets, logit_lengths, target_lengths, self.blank, self.clamp, self.reduction,
                         self.fused_log_softmax, self.fastemit_lambda)


# ------------------------------------------------------ multi-blank transducer
def _big_blanks(big_blank_ids, big_blank_durations):
    """Validated lists of the big blanks' classes and durations (same length; ids distinct)."""
    ids = [int(v) for v in big_blank_ids]
    durs = [int(v) for v in big_blank_durations]
    if len(ids) != len(durs):
        raise ValueError("big_blank_ids and big_blank_durations must have the same length")
    if len(set(ids)) != len(ids):
        raise ValueError("big_blank_ids must be distinct classes")
    return ids, durs


def rnnt_multiblank_fused(logits: torch.Tensor, targets: torch.Tensor, logit_lengths, target_lengths, *,
                          big_blank_ids, big_blank_durations, blank: int = -1, sigma: float = 0.0,
                          clamp: float = -1.0, reduction: str = "mean", fused_log_softmax: bool = True,
                          fastemit_lambda: float = 0.0, compute_grad: bool = True,
                          grad: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                          loss: Optional[torch.Tensor] = None, loss_reduced: Optional[torch.Tensor] = None):
    """One multi-blank librnnt call.  Returns ``(loss, loss_reduced, grad, workspace)``.

    Big blank i is class ``big_blank_ids[i]`` and advances t by ``big_blank_durations[i]`` frames; ``sigma`` is
    subtracted from every emission's log-probability (logit under-normalisation).  Both lists are keyword-only
    (two integer lists in swapped order would otherwise be accepted silently); the classes must be distinct,
    in [0, V) and not the blank (the library refuses others).  Packed 2-D or padded 4-D logits, the rest as for
    :func:`rnnt_loss_fused`.
    """
    big_blank_ids, big_blank_durations = _big_blanks(big_blank_ids, big_blank_durations)
    tg = _prepare(logits, targets)
    T = _lib.host_i32(logit_lengths)
    U = _lib.host_i32(target_lengths)
    B = len(T)
    if len(U) != B:
        raise ValueError("logit_lengths and target_lengths must have the same length")
    dev = logits.device
    code = _dtype_code(logits.dtype)
    padded = logits.dim() == 4
    if padded:
        if logits.shape[0] != B:
            raise ValueError("padded logits must have one (max_T, max_U+1, V) block per sample")
        max_T, max_U1, V = logits.shape[1], logits.shape[2], logits.shape[3]
        need = _lib.workspace_size_multiblank_padded(B, V, max_T, max_U1, code, T, U, big_blank_durations)
    else:
        N, V = logits.shape
        need = _lib.workspace_size_multiblank(B, V, N, code, T, U, big_blank_durations)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    if loss is None:
        loss = torch.empty(B, dtype=torch.float32, device=dev)
    if reduction != "none" and loss_reduced is None:
        loss_reduced = torch.empty(1, dtype=torch.float32, device=dev)
    if compute_grad:
        if grad is None:
            grad = torch.empty_like(logits)
        elif grad.shape != logits.shape or grad.dtype != logits.dtype or not grad.is_contiguous():
            raise ValueError("grad must match logits in shape and dtype and be contiguous")
    else:
        grad = None
    with torch.cuda.device(dev):
        stream = _stream_handle(dev)
        tgp = tg.data_ptr() if tg.numel() else 0
        redp = loss_reduced.data_ptr() if reduction != "none" else 0
        gp = grad.data_ptr() if grad is not None else 0
        if padded:
            _lib.loss_multiblank_padded(logits.data_ptr(), code, max_T, max_U1, V, tgp, tg.shape[1], T, U, blank,
                                        big_blank_ids, big_blank_durations, sigma, clamp, fastemit_lambda,
                                        fused_log_softmax, reduction, loss.data_ptr(), redp, gp,
                                        workspace.data_ptr(), workspace.numel(), stream)
        else:
            _lib.loss_multiblank(logits.data_ptr(), code, N, V, tgp, tg.shape[1], T, U, blank, big_blank_ids,
                                 big_blank_durations, sigma, clamp, fastemit_lambda, fused_log_softmax, reduction,
                                 loss.data_ptr(), redp, gp, workspace.data_ptr(), workspace.numel(), stream)
    return loss, (loss_reduced if reduction != "none" else None), grad, workspace


class _MultiblankFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, logits, targets, logit_lengths, target_lengths, big_blank_ids, big_blank_durations, blank,
                sigma, clamp, reduction, fused_log_softmax, fastemit_lambda):
        T = _lib.host_i32(logit_lengths)
        U = _lib.host_i32(target_lengths)
        loss, loss_red, grad, ws = rnnt_multiblank_fused(
            logits, targets, T, U, big_blank_ids=big_blank_ids, big_blank_durations=big_blank_durations,
            blank=blank, sigma=sigma, clamp=clamp, reduction=reduction, fused_log_softmax=fused_log_softmax,
            fastemit_lambda=fastemit_lambda, compute_grad=logits.requires_grad)
        ctx.meta = (T, U, reduction, logits.shape, logits.dtype)
        ctx.used = False
        if grad is not None:
            ctx.save_for_backward(grad, ws)
        return loss if reduction == "none" else loss_red.reshape(())

    @staticmethod
    def backward(ctx, grad_out):
        none = (None,) * 11
        T, U, reduction, shape, dtype = ctx.meta
        if not ctx.saved_tensors:
            return (None,) + none
        if ctx.used:
            raise RuntimeError("rnnt_loss_multiblank backward was already run for this forward call")
        ctx.used = True
        grad, ws = ctx.saved_tensors
        scale = grad_out.detach()
        if scale.dtype != torch.float32 or scale.device != grad.device or not scale.is_contiguous():
            scale = scale.to(device=grad.device, dtype=torch.float32).contiguous()
        scale = scale.reshape(-1)
        with _on_device(grad.device):
            stream = _stream_handle(grad.device)
            if len(shape) == 4:
                _lib.grad_scale_multiblank_padded(grad.data_ptr(), _dtype_code(dtype), shape[1], shape[2], shape[3],
                                                  T, U, scale.data_ptr(), reduction == "none", ws.data_ptr(),
                                                  ws.numel(), stream)
            else:
                _lib.grad_scale_multiblank(grad.data_ptr(), _dtype_code(dtype), shape[0], shape[1], T, U,
                                           scale.data_ptr(), reduction == "none", ws.data_ptr(), ws.numel(), stream)
        return (grad,) + none


def rnnt_loss_multiblank(logits: torch.Tensor, targets: torch.Tensor, logit_lengths, target_lengths, *,
                         big_blank_ids, big_blank_durations, blank: int = -1, sigma: float = 0.0,
                         clamp: float = -1.0, reduction: str = "mean", fused_log_softmax: bool = True,
                         fastemit_lambda: float = 0.0) -> torch.Tensor:
    """Multi-blank transducer loss over packed (or padded 4-D) logits, differentiable with respect to ``logits``.

    ``big_blank_durations[i]`` is the number of frames big blank i (class ``big_blank_ids[i]``) advances;
    ``sigma`` lowers every emission's log-probability (logit under-normalisation).  With no big blank and
    ``sigma = 0`` this is :func:`rnnt_loss`.  The big-blank lists are keyword-only, as in
    :func:`rnnt_multiblank_fused`.
    """
    if reduction not in ("none", "mean", "sum"):
        raise ValueError(f"reduction must be none, mean or sum, got {reduction!r}")
    big_blank_ids, big_blank_durations = _big_blanks(big_blank_ids, big_blank_durations)
    return _MultiblankFunction.apply(logits, targets, logit_lengths, target_lengths, big_blank_ids,
                                     big_blank_durations, int(blank), float(sigma), float(clamp), reduction,
                                     bool(fused_log_softmax), float(fastemit_lambda))
