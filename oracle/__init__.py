"""Plain fp64 CPU oracle for the RNN-T loss (forward and backward).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``rnn_transducer_loss_amd``) never imports it, and the two share no code:
the only thing both sides use is the seeded input generator in
``workloads.py``, which holds none of the method's arithmetic.

The arithmetic lives in ``rnnt_oracle.c`` (fp64, row-major loops over the
lattice).  This module only builds/loads it and marshals numpy arrays.
Semantics follow the rnnt-loss-ascend README (parameter table and usage
example): ``blank`` in [-V, V-1] with negative values counted from the end,
``clamp <= 0`` disables clipping, and ``reduction`` is one of none / mean
(batch mean) / sum.  ``fastemit_lambda`` (the GPURNNT parameter of the ESPnet
multi-blank utilities page, defined by the FastEmit paper it refers to)
multiplies the loss's derivative with respect to every label-emission
log-probability by (1 + lambda); the loss value itself is unchanged.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rnnt_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()

ORACLE_OK = 0
ORACLE_BAD_ARGS = 1
ORACLE_BAD_TARGET = 2
ORACLE_NO_MEMORY = 3


def build(force: bool = True) -> str:
    """Compile rnnt_oracle.c into liboracle.so with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build(force=False)
            lib = ctypes.CDLL(_LIB_PATH)
            dp = ctypes.POINTER(ctypes.c_double)
            lib.rnnt_oracle_sample.argtypes = [
                dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                ctypes.c_int, ctypes.c_int, ctypes.c_double, dp, dp, dp, dp, dp]
            lib.rnnt_oracle_sample.restype = ctypes.c_int
            lib.rnnt_oracle_sample_ex.argtypes = [
                ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                ctypes.POINTER(ctypes.c_int), ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_double,
                ctypes.POINTER(ctypes.c_int64), ctypes.c_long, dp, dp, dp, dp, dp]
            lib.rnnt_oracle_sample_ex.restype = ctypes.c_int
            ip = ctypes.POINTER(ctypes.c_int)
            lib.rnnt_oracle_multiblank_sample.argtypes = [
                ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ip, ctypes.c_int,
                ctypes.c_int, ip, ip, ctypes.c_double, ctypes.c_int, ctypes.c_double, ctypes.c_double, dp, dp, dp]
            lib.rnnt_oracle_multiblank_sample.restype = ctypes.c_int
            lib.rnnt_oracle_half_to_double.argtypes = [ctypes.c_uint16]
            lib.rnnt_oracle_half_to_double.restype = ctypes.c_double
            _lib = lib
    return _lib


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def normalize_blank(blank: int, V: int) -> int:
    """Blank in [-V, V-1]; a negative value counts from the end (-1 -> V-1)."""
    if blank < -V or blank > V - 1:
        raise ValueError(f"blank {blank} outside [-{V}, {V - 1}]")
    return blank + V if blank < 0 else blank


class SampleResult:
    __slots__ = ("loss", "loss_alpha", "grad", "alpha", "beta", "bad_target")

    def __init__(self, loss, loss_alpha, grad, alpha, beta, bad_target=False):
        self.loss = loss
        self.loss_alpha = loss_alpha
        self.grad = grad
        self.alpha = alpha
        self.beta = beta
        self.bad_target = bad_target


_DT = {np.dtype(np.float64): 0, np.dtype(np.float32): 1, np.dtype(np.float16): 2}


def half_to_double(h: int) -> float:
    """The oracle's own exact binary16 -> binary64 conversion (pinned against numpy)."""
    return _load().rnnt_oracle_half_to_double(int(h))


def sample(x, T: int, U: int, y, blank: int, fused: bool = True, clamp: float = -1.0,
           want_grad: bool = True, want_tables: bool = False, rows=None,
           fastemit_lambda: float = 0.0, allow_bad_targets: bool = False) -> SampleResult:
    """Loss (and optionally gradient / alpha / beta tables) of one sample.

    ``x`` holds the sample's T*(U+1) rows of V values as float64, float32 or
    float16; the C code converts each value exactly to fp64 as it reads it.
    ``blank`` must already be in [0, V).  ``rows`` (sample-local row indices)
    restricts the gradient to those rows, returned in that order; by default
    every row.  The loss is the beta-path value -beta(0,0); ``loss_alpha`` is
    the alpha-path value kept for the cross-check.

    A label equal to blank or outside [0, V) (the build post's section 5.2
    rules blank out of the labels) leaves the sample without any alignment:
    loss +inf and a zero gradient.  Such a sample raises ValueError unless
    ``allow_bad_targets`` is set; then the result carries ``bad_target``.
    """
    lib = _load()
    x = np.asarray(x)
    if x.dtype not in _DT:
        x = x.astype(np.float64)
    x = np.ascontiguousarray(x)
    V = x.shape[1]
    if x.shape[0] != T * (U + 1):
        raise ValueError("row count does not match T*(U+1)")
    yy = np.ascontiguousarray(np.asarray(y[:U], dtype=np.int32)) if U > 0 else np.zeros(1, np.int32)
    if rows is None:
        rr, nr = None, -1
        n_out = T * (U + 1)
    else:
        rr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nr = len(rr)
        n_out = nr
    grad = np.empty((n_out, V), np.float64) if want_grad else None
    al = np.empty((T, U + 1), np.float64) if want_tables else None
    be = np.empty((T, U + 1), np.float64) if want_tables else None
    la = ctypes.c_double()
    lb = ctypes.c_double()
    rc = lib.rnnt_oracle_sample_ex(
        x.ctypes.data_as(ctypes.c_void_p), _DT[x.dtype], T, U, V, yy.ctypes.data_as(ctypes.POINTER(ctypes.c_int)),
        int(blank), int(bool(fused)), float(clamp), float(fastemit_lambda),
        rr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)) if rr is not None else None, nr,
        _ptr(grad), _ptr(al), _ptr(be), ctypes.byref(la), ctypes.byref(lb))
    if rc == ORACLE_BAD_TARGET and not allow_bad_targets:
        raise ValueError("target label equal to blank or outside [0, V)")
    if rc not in (ORACLE_OK, ORACLE_BAD_TARGET):
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return SampleResult(lb.value, la.value, grad, al, be, rc == ORACLE_BAD_TARGET)


def batch(logits, targets, logit_lengths, target_lengths, blank: int = -1, clamp: float = -1.0,
          reduction: str = "mean", fused: bool = True, want_grad: bool = True, fastemit_lambda: float = 0.0):
    """Whole-batch oracle over the packed (sum_i T_i*(U_i+1), V) layout.

    Returns ``(loss_per_sample, reduced_loss, grad_per_sample, grad_reduced)``.
    ``grad_per_sample`` is d loss_i / d logits for each sample's own rows
    (clamped, unscaled); ``grad_reduced`` is the gradient of the reduced loss
    with a unit upstream gradient: the same rows scaled by 1/B for mean and 1
    for sum and none.  Both are None when ``want_grad`` is False.
    """
    logits = np.asarray(logits)
    N, V = logits.shape
    B = len(logit_lengths)
    b = normalize_blank(int(blank), V)
    Ts = [int(v) for v in logit_lengths]
    Us = [int(v) for v in target_lengths]
    rows = [Ts[i] * (Us[i] + 1) for i in range(B)]
    if sum(rows) != N:
        raise ValueError("sum of T_i*(U_i+1) does not equal logits.shape[0]")
    if reduction not in ("none", "mean", "sum"):
        raise ValueError(f"unknown reduction {reduction!r}")
    losses = np.empty(B, np.float64)
    grad = np.empty((N, V), np.float64) if want_grad else None
    off = 0
    for i in range(B):
        res = sample(logits[off:off + rows[i]], Ts[i], Us[i], np.asarray(targets[i]), b, fused, clamp,
                     want_grad=want_grad, fastemit_lambda=fastemit_lambda)
        losses[i] = res.loss
        if want_grad:
            grad[off:off + rows[i]] = res.grad
        off += rows[i]
    if reduction == "none":
        reduced, scale = losses.copy(), 1.0
    elif reduction == "sum":
        reduced, scale = losses.sum(), 1.0
    else:
        reduced, scale = losses.sum() / B, 1.0 / B
    grad_reduced = grad * scale if want_grad else None
    return losses, reduced, grad, grad_reduced


def multiblank_sample(x, T: int, U: int, y, blank: int, big_blank_ids, big_blank_durations, sigma: float = 0.0,
                      fused: bool = True, clamp: float = -1.0, fastemit_lambda: float = 0.0,
                      want_grad: bool = True, allow_bad_targets: bool = False) -> SampleResult:
    """Multi-blank transducer loss (and gradient of every row) of one sample.

    Big blank i is class ``big_blank_ids[i]`` and moves t forward by
    ``big_blank_durations[i]``; every emission's log-probability is lowered
    by ``sigma`` (logit under-normalisation).  These follow the
    compute_multiblank_grad_kernel page's parameters; see rnnt_oracle.c for
    the reading of the alignment rules.  ``loss_alpha`` is the forward
    recursion's value, ``loss`` the backward one's.  A label that is a blank
    of either kind or outside [0, V) leaves no alignment (loss +inf, zero
    gradient); it raises ValueError unless ``allow_bad_targets`` is set.
    """
    lib = _load()
    x = np.asarray(x)
    if x.dtype not in _DT:
        x = x.astype(np.float64)
    x = np.ascontiguousarray(x)
    V = x.shape[1]
    if x.shape[0] != T * (U + 1):
        raise ValueError("row count does not match T*(U+1)")
    ids = np.ascontiguousarray(np.asarray(big_blank_ids, dtype=np.int32).reshape(-1))
    dur = np.ascontiguousarray(np.asarray(big_blank_durations, dtype=np.int32).reshape(-1))
    if ids.shape != dur.shape:
        raise ValueError("big_blank_ids and big_blank_durations must have the same length")
    nb = len(ids)
    yy = np.ascontiguousarray(np.asarray(y[:U], dtype=np.int32)) if U > 0 else np.zeros(1, np.int32)
    ip = ctypes.POINTER(ctypes.c_int)
    grad = np.empty((T * (U + 1), V), np.float64) if want_grad else None
    la = ctypes.c_double()
    lb = ctypes.c_double()
    rc = lib.rnnt_oracle_multiblank_sample(
        x.ctypes.data_as(ctypes.c_void_p), _DT[x.dtype], T, U, V, yy.ctypes.data_as(ip), int(blank), nb,
        (ids if nb else np.zeros(1, np.int32)).ctypes.data_as(ip),
        (dur if nb else np.zeros(1, np.int32)).ctypes.data_as(ip), float(sigma), int(bool(fused)), float(clamp),
        float(fastemit_lambda), _ptr(grad), ctypes.byref(la), ctypes.byref(lb))
    if rc == ORACLE_BAD_TARGET and not allow_bad_targets:
        raise ValueError("target label equal to a blank or outside [0, V)")
    if rc not in (ORACLE_OK, ORACLE_BAD_TARGET):
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return SampleResult(lb.value, la.value, grad, None, None, rc == ORACLE_BAD_TARGET)


def multiblank_batch(logits, targets, logit_lengths, target_lengths, big_blank_ids, big_blank_durations,
                     blank: int = -1, sigma: float = 0.0, clamp: float = -1.0, reduction: str = "mean",
                     fused: bool = True, fastemit_lambda: float = 0.0, want_grad: bool = True):
    """Whole-batch multi-blank oracle over the packed layout; returns as :func:`batch`."""
    logits = np.asarray(logits)
    N, V = logits.shape
    B = len(logit_lengths)
    b = normalize_blank(int(blank), V)
    Ts = [int(v) for v in logit_lengths]
    Us = [int(v) for v in target_lengths]
    rows = [Ts[i] * (Us[i] + 1) for i in range(B)]
    if sum(rows) != N:
        raise ValueError("sum of T_i*(U_i+1) does not equal logits.shape[0]")
    if reduction not in ("none", "mean", "sum"):
        raise ValueError(f"unknown reduction {reduction!r}")
    losses = np.empty(B, np.float64)
    grad = np.empty((N, V), np.float64) if want_grad else None
    off = 0
    for i in range(B):
        res = multiblank_sample(logits[off:off + rows[i]], Ts[i], Us[i], np.asarray(targets[i]), b, big_blank_ids,
                                big_blank_durations, sigma, fused, clamp, fastemit_lambda, want_grad)
        losses[i] = res.loss
        if want_grad:
            grad[off:off + rows[i]] = res.grad
        off += rows[i]
    if reduction == "none":
        reduced, scale = losses.copy(), 1.0
    elif reduction == "sum":
        reduced, scale = losses.sum(), 1.0
    else:
        reduced, scale = losses.sum() / B, 1.0 / B
    return losses, reduced, grad, (grad * scale if want_grad else None)
