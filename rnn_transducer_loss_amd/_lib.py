"""ctypes binding of librnnt (include/rnnt.h): argument marshalling only.

Every step of the loss runs in librnnt's HIP kernels.  PyTorch supplies
device memory and the current HIP stream.  If the built library is missing,
loading fails loudly: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librnnt.so")

RNNT_F32, RNNT_F16 = 0, 1
REDUCTIONS = {"none": 0, "mean": 1, "sum": 2}
RNNT_SUCCESS = 0
RNNT_INVALID_VALUE = 1
RNNT_WORKSPACE_TOO_SMALL = 2
RNNT_DEV_LOSS_MISMATCH = 1
RNNT_DEV_BAD_TARGET = 2

EXPORTS = ("rnnt_loss_fused_workspace_size", "rnnt_loss_fused", "rnnt_grad_scale", "rnnt_loss_fused_check",
           "rnnt_status_string", "rnnt_plan_describe", "rnnt_timing_enable", "rnnt_timing_read",
           "rnnt_loss_padded_workspace_size", "rnnt_loss_padded", "rnnt_grad_scale_padded",
           "rnnt_multiblank_workspace_size", "rnnt_multiblank_loss", "rnnt_multiblank_grad_scale",
           "rnnt_multiblank_padded_workspace_size", "rnnt_multiblank_loss_padded", "rnnt_multiblank_grad_scale_padded",
           "rnnt_loss_fused_noalloc")
NOALLOC_SCRATCH_BYTES = 128 << 20   # RNNT_NOALLOC_SCRATCH_BYTES
KERNELS = ("rowstats", "alpha_beta", "grad", "reduce")

_lib = None
_lock = threading.Lock()

_i32p = ctypes.POINTER(ctypes.c_int32)
_i32in = ctypes.c_char_p  # a host int32 input array, passed as the bytes of a contiguous copy
_vp = ctypes.c_void_p


class RNNTError(RuntimeError):
    pass


def load():
    """Load librnnt.so (built by ``python -m rnn_transducer_loss_amd.build``)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RNNTError(f"librnnt is not built ({LIB_PATH} missing); run python -m rnn_transducer_loss_amd.build")
        lib = ctypes.CDLL(LIB_PATH)
        lib.rnnt_status_string.argtypes = [ctypes.c_int]
        lib.rnnt_status_string.restype = ctypes.c_char_p
        lib.rnnt_loss_fused_workspace_size.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int,
                                                       _i32in, _i32in, ctypes.POINTER(ctypes.c_size_t)]
        lib.rnnt_loss_fused_workspace_size.restype = ctypes.c_int
        lib.rnnt_loss_fused.argtypes = [_vp, ctypes.c_int, ctypes.c_int64, ctypes.c_int32, _vp, ctypes.c_int32,
                                        _i32in, _i32in, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                        ctypes.c_float, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _vp,
                                        ctypes.c_size_t, _vp]
        lib.rnnt_loss_fused.restype = ctypes.c_int
        lib.rnnt_loss_fused_noalloc.argtypes = [_vp, ctypes.c_int, ctypes.c_int64, ctypes.c_int32, _vp,
                                                ctypes.c_int32, _i32in, _i32in, ctypes.c_int32, ctypes.c_int64,
                                                ctypes.c_float, ctypes.c_float, ctypes.c_int, ctypes.c_int, _vp, _vp,
                                                _vp, _vp, _vp]
        lib.rnnt_loss_fused_noalloc.restype = ctypes.c_int
        lib.rnnt_grad_scale.argtypes = [_vp, ctypes.c_int, ctypes.c_int64, ctypes.c_int32, _i32in, _i32in,
                                        ctypes.c_int32, _vp, ctypes.c_int, _vp, ctypes.c_size_t, _vp]
        lib.rnnt_grad_scale.restype = ctypes.c_int
        lib.rnnt_loss_padded_workspace_size.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                         ctypes.c_int32, ctypes.c_int, _i32in, _i32in,
                                                         ctypes.POINTER(ctypes.c_size_t)]
        lib.rnnt_loss_padded_workspace_size.restype = ctypes.c_int
        lib.rnnt_loss_padded.argtypes = [_vp, ctypes.c_int, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _vp,
                                         ctypes.c_int32, _i32in, _i32in, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                         ctypes.c_float, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _vp,
                                         ctypes.c_size_t, _vp]
        lib.rnnt_loss_padded.restype = ctypes.c_int
        lib.rnnt_grad_scale_padded.argtypes = [_vp, ctypes.c_int, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                               _i32in, _i32in, ctypes.c_int32, _vp, ctypes.c_int, _vp, ctypes.c_size_t,
                                               _vp]
        lib.rnnt_grad_scale_padded.restype = ctypes.c_int
        lib.rnnt_loss_fused_check.argtypes = [_vp, _vp, ctypes.POINTER(ctypes.c_uint32)]
        lib.rnnt_loss_fused_check.restype = ctypes.c_int
        lib.rnnt_plan_describe.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int, _i32in, _i32in, ctypes.c_int32,
                                           _i32p, _i32p, _i32p, _i32p, _i32p, _i32p, _i32p]
        lib.rnnt_plan_describe.restype = ctypes.c_int
        lib.rnnt_multiblank_workspace_size.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int,
                                                       _i32in, _i32in, ctypes.c_int32, _i32in,
                                                       ctypes.POINTER(ctypes.c_size_t)]
        lib.rnnt_multiblank_workspace_size.restype = ctypes.c_int
        lib.rnnt_multiblank_loss.argtypes = [_vp, ctypes.c_int, ctypes.c_int64, ctypes.c_int32, _vp, ctypes.c_int32,
                                             _i32in, _i32in, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, _i32in,
                                             _i32in, ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_int,
                                             ctypes.c_int, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        lib.rnnt_multiblank_loss.restype = ctypes.c_int
        lib.rnnt_multiblank_grad_scale.argtypes = [_vp, ctypes.c_int, ctypes.c_int64, ctypes.c_int32, _i32in, _i32in,
                                                   ctypes.c_int32, _vp, ctypes.c_int, _vp, ctypes.c_size_t, _vp]
        lib.rnnt_multiblank_grad_scale.restype = ctypes.c_int
        lib.rnnt_multiblank_padded_workspace_size.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                              ctypes.c_int32, ctypes.c_int, _i32in, _i32in,
                                                              ctypes.c_int32, _i32in, ctypes.POINTER(ctypes.c_size_t)]
        lib.rnnt_multiblank_padded_workspace_size.restype = ctypes.c_int
        lib.rnnt_multiblank_loss_padded.argtypes = [_vp, ctypes.c_int, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                    _vp, ctypes.c_int32, _i32in, _i32in, ctypes.c_int32,
                                                    ctypes.c_int64, ctypes.c_int32, _i32in, _i32in, ctypes.c_float,
                                                    ctypes.c_float, ctypes.c_float, ctypes.c_int, ctypes.c_int, _vp,
                                                    _vp, _vp, _vp, ctypes.c_size_t, _vp]
        lib.rnnt_multiblank_loss_padded.restype = ctypes.c_int
        lib.rnnt_multiblank_grad_scale_padded.argtypes = [_vp, ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                                          ctypes.c_int32, _i32in, _i32in, ctypes.c_int32, _vp,
                                                          ctypes.c_int, _vp, ctypes.c_size_t, _vp]
        lib.rnnt_multiblank_grad_scale_padded.restype = ctypes.c_int
        lib.rnnt_timing_enable.argtypes = [ctypes.c_int]
        lib.rnnt_timing_enable.restype = ctypes.c_int
        lib.rnnt_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), _i32p]
        lib.rnnt_timing_read.restype = ctypes.c_int
        _lib = lib
        return lib


def status_string(code: int) -> str:
    return load().rnnt_status_string(int(code)).decode()


def check(code: int, what: str):
    if code == RNNT_SUCCESS:
        return
    msg = f"{what}: {status_string(code)} (status {code})"
    if code == RNNT_INVALID_VALUE or code == RNNT_WORKSPACE_TOO_SMALL:
        raise ValueError(msg)
    raise RNNTError(msg)


def host_i32(a) -> np.ndarray:
    """A contiguous host int32 copy of a length vector (tensor on any device, list or array)."""
    if type(a) is np.ndarray and a.dtype == np.int32 and a.flags.c_contiguous:
        return a
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().to("cpu")
            return np.ascontiguousarray(a.numpy().astype(np.int32, copy=False))
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _p(a: np.ndarray):
    """Pointer to an int32 array the library writes (an output)."""
    return a.ctypes.data_as(_i32p)


def _b(a: np.ndarray) -> bytes:
    """An int32 input array for the library: the bytes of a contiguous host int32 array (read during the call
    only).  Faster to pass than an array pointer."""
    return a.tobytes()


def workspace_size(B: int, V: int, N: int, dtype_code: int, logit_lengths, target_lengths) -> int:
    T = host_i32(logit_lengths)
    U = host_i32(target_lengths)
    if len(T) != B or len(U) != B:
        raise ValueError("length vectors must have B entries")
    out = ctypes.c_size_t()
    check(load().rnnt_loss_fused_workspace_size(B, V, N, dtype_code, _b(T), _b(U), ctypes.byref(out)),
          "rnnt_loss_fused_workspace_size")
    return int(out.value)


def loss_fused(logits_ptr: int, dtype_code: int, N: int, V: int, targets_ptr: int, S: int, logit_lengths,
               target_lengths, blank: int, clamp: float, fused: bool, reduction: str, loss_ptr: int,
               loss_reduced_ptr: int, grad_ptr: int, ws_ptr: int, ws_bytes: int, stream: int,
               fastemit_lambda: float = 0.0):
    T = host_i32(logit_lengths)
    U = host_i32(target_lengths)
    B = len(T)
    if len(U) != B:
        raise ValueError("length vectors must have B entries")
    if reduction not in REDUCTIONS:
        raise ValueError(f"reduction must be one of {sorted(REDUCTIONS)}")
    rc = load().rnnt_loss_fused(logits_ptr or None, dtype_code, N, V, targets_ptr or None, S, _b(T), _b(U), B,
                                int(blank), float(clamp), float(fastemit_lambda), int(bool(fused)),
                                REDUCTIONS[reduction], loss_ptr or None,
                                loss_reduced_ptr or None, grad_ptr or None, ws_ptr or None, ws_bytes,
                                stream or None)
    check(rc, "rnnt_loss_fused")


def loss_fused_noalloc(logits_ptr: int, dtype_code: int, N: int, V: int, targets_ptr: int, S: int, logit_lengths,
                       target_lengths, blank: int, clamp: float, fused: bool, reduction: str, loss_ptr: int,
                       loss_reduced_ptr: int, grad_ptr: int, status_ptr: int, stream: int,
                       fastemit_lambda: float = 0.0):
    """rnnt_loss_fused_noalloc: the workspace is the library's fixed device scratch (no allocation)."""
    T = host_i32(logit_lengths)
    U = host_i32(target_lengths)
    B = len(T)
    if len(U) != B:
        raise ValueError("length vectors must have B entries")
    if reduction not in REDUCTIONS:
        raise ValueError(f"reduction must be one of {sorted(REDUCTIONS)}")
    rc = load().rnnt_loss_fused_noalloc(logits_ptr or None, dtype_code, N, V, targets_ptr or None, S, _b(T), _b(U),
                                        B, int(blank), float(clamp), float(fastemit_lambda), int(bool(fused)),
                                        REDUCTIONS[reduction], loss_ptr or None, loss_reduced_ptr or None,
                                        grad_ptr or None, status_ptr or None, stream or None)
    check(rc, "rnnt_loss_fused_noalloc")


def grad_scale(grad_ptr: int, dtype_code: int, N: int, V: int, logit_lengths, target_lengths, scale_ptr: int,
               per_sample: bool, ws_ptr: int, ws_bytes: int, stream: int):
    T = host_i32(logit_lengths)
    U = host_i32(target_lengths)
    rc = load().rnnt_grad_scale(grad_ptr or None, dtype_code, N, V, _b(T), _b(U), len(T), scale_ptr or None,
                                int(bool(per_sample)), ws_ptr or None, ws_bytes, stream or None)
    check(rc, "rnnt_grad_scale")


def workspace_size_padded(B: int, V: int, max_T: int, max_U1: int, dtype_code: int, logit_lengths,
                          target_lengths) -> int:
    T = host_i32(logit_lengths)
    U = host_i32(target_lengths)
    if len(T) != B or len(U) != B:
        raise ValueError("length vectors must have B entries")
    out = ctypes.c_size_t()
    check(load().rnnt_loss_padded_workspace_size(B, V, max_T, max_U1, dtype_code, _b(T), _b(U), ctypes.byref(out)),
          "rnnt_loss_padded_workspace_size")
    return int(out.value)


def loss_padded(logits_ptr: int, dtype_code: int, max_T: int, max_U1: int, V: int, targets_ptr: int, S: int,
                logit_lengths, target_lengths, blank: int, clamp: float, fused: bool, reduction: str, loss_ptr: int,
                loss_reduced_ptr: int, grad_ptr: int, ws_ptr: int, ws_bytes: int, stream: int,
                fastemit_lambda: float = 0.0):
    T = host_i32(logit_lengths)
    U = host_i32(target_lengths)
    B = len(T)
    if len(U) != B:
        raise ValueError("length vectors must have B entries")
    if reduction not in REDUCTIONS:
        raise ValueError(f"reduction must be one of {sorted(REDUCTIONS)}")
    rc = load().rnnt_loss_padded(logits_ptr or None, dtype_code, max_T, max_U1, V, targets_ptr or None, S, _b(T),
                                 _b(U), B, int(blank), float(clamp), float(fastemit_lambda), int(bool(fused)),
                                 REDUCTIONS[reduction],
                                 loss_ptr or None, loss_reduced_ptr or None, grad_ptr or None, ws_ptr or None,
                                 ws_bytes, stream or None)
    check(rc, "rnnt_loss_padded")


def grad_scale_padded(grad_ptr: int, dtype_code: int, max_T: int, max_U1: int, V: int, logit_lengths,
                      target_lengths, scale_ptr: int, per_sample: bool, ws_ptr: int, ws_bytes: int, stream: int):
    T = host_i32(logit_lengths)
    U = host_i32(target_lengths)
    rc = load().rnnt_grad_scale_padded(grad_ptr or None, dtype_code, max_T, max_U1, V, _b(T), _b(U), len(T),
                                       scale_ptr or None, int(bool(per_sample)), ws_ptr or None, ws_bytes,
                                       stream or None)
    check(rc, "rnnt_grad_scale_padded")


def device_flags(ws_ptr: int, stream: int) -> int:
    out = ctypes.c_uint32()
    check(load().rnnt_loss_fused_check(ws_ptr or None, stream or None, ctypes.byref(out)), "rnnt_loss_fused_check")
    return int(out.value)


def plan_describe(V: int, dtype_code: int, logit_lengths, target_lengths, diagonal: bool = False):
    """Host schedule; no GPU needed.

    Returns (sample_order, chunks) with chunks[k] = (sample, row_begin, row_count)
    (row order), or with diagonal=True chunks[k] = (sample, diag, col, count):
    the same runs walked in anti-diagonal order from node (diag, col).
    """
    T = host_i32(logit_lengths)
    U = host_i32(target_lengths)
    B = len(T)
    n = ctypes.c_int32()
    lib = load()
    check(lib.rnnt_plan_describe(B, V, dtype_code, _b(T), _b(U), 0, None, None, None, None, None, None,
                                 ctypes.byref(n)), "rnnt_plan_describe")
    cap = max(B, n.value)
    order = np.zeros(cap, np.int32)
    cs, cb, cc, cd, cu = (np.zeros(cap, np.int32) for _ in range(5))
    check(lib.rnnt_plan_describe(B, V, dtype_code, _b(T), _b(U), cap, _p(order), _p(cs), _p(cb), _p(cc), _p(cd),
                                 _p(cu), ctypes.byref(n)), "rnnt_plan_describe")
    k = n.value
    if diagonal:
        return order[:B].copy(), np.stack([cs[:k], cd[:k], cu[:k], cc[:k]], axis=1)
    return order[:B].copy(), np.stack([cs[:k], cb[:k], cc[:k]], axis=1)


def timing_enable(on: bool):
    check(load().rnnt_timing_enable(int(bool(on))), "rnnt_timing_enable")


def timing_read():
    """{kernel: (total_ms, launches)} recorded since timing was enabled."""
    ms = (ctypes.c_double * 4)()
    n = (ctypes.c_int32 * 4)()
    check(load().rnnt_timing_read(ms, n), "rnnt_timing_read")
    return {k: (float(ms[i]), int(n[i])) for i, k in enumerate(KERNELS)}


def _big_blanks(big_blank_ids, big_blank_durations):
    ids = host_i32(big_blank_ids).reshape(-1)
    dur = host_i32(big_blank_durations).reshape(-1)
    if ids.shape != dur.shape:
        raise ValueError("big_blank_ids and big_blank_durations must have the same length")
    # ctypes needs a valid pointer even for an empty list
    return len(ids), (ids if len(ids) else np.zeros(1, np.int32)), (dur if len(dur) else np.zeros(1, np.int32))


def workspace_size_multiblank(B: int, V: int, N: int, dtype_code: int, logit_lengths, target_lengths,
                              big_blank_durations) -> int:
    T = host_i32(logit_lengths)
    U = host_i32(target_lengths)
    if len(T) != B or len(U) != B:
        raise ValueError("length vectors must have B entries")
    nb, _, dur = _big_blanks(np.zeros(len(host_i32(big_blank_durations).reshape(-1)), np.int32), big_blank_durations)
    out = ctypes.c_size_t()
    check(load().rnnt_multiblank_workspace_size(B, V, N, dtype_code, _b(T), _b(U), nb, _b(dur), ctypes.byref(out)),
          "rnnt_multiblank_workspace_size")
    return int(out.value)


def loss_multiblank(logits_ptr: int, dtype_code: int, N: int, V: int, targets_ptr: int, S: int, logit_lengths,
                    target_lengths, blank: int, big_blank_ids, big_blank_durations, sigma: float, clamp: float,
                    fastemit_lambda: float, fused: bool, reduction: str, loss_ptr: int, loss_reduced_ptr: int,
                    grad_ptr: int, ws_ptr: int, ws_bytes: int, stream: int):
    T = host_i32(logit_lengths)
    U = host_i32(target_lengths)
    B = len(T)
    if len(U) != B:
        raise ValueError("length vectors must have B entries")
    if reduction not in REDUCTIONS:
        raise ValueError(f"reduction must be one of {sorted(REDUCTIONS)}")
    nb, ids, dur = _big_blanks(big_blank_ids, big_blank_durations)
    rc = load().rnnt_multiblank_loss(logits_ptr or None, dtype_code, N, V, targets_ptr or None, S, _b(T), _b(U), B,
                                     int(blank), nb, _b(ids), _b(dur), float(sigma), float(clamp),
                                     float(fastemit_lambda), int(bool(fused)), REDUCTIONS[reduction],
                                     loss_ptr or None, loss_reduced_ptr or None, grad_ptr or None, ws_ptr or None,
                                     ws_bytes, stream or None)
    check(rc, "rnnt_multiblank_loss")


def grad_scale_multiblank(grad_ptr: int, dtype_code: int, N: int, V: int, logit_lengths, target_lengths,
                          scale_ptr: int, per_sample: bool, ws_ptr: int, ws_bytes: int, stream: int):
    T = host_i32(logit_lengths)
    U = host_i32(target_lengths)
    rc = load().rnnt_multiblank_grad_scale(grad_ptr or None, dtype_code, N, V, _b(T), _b(U), len(T),
                                           scale_ptr or None, int(bool(per_sample)), ws_ptr or None, ws_bytes,
                                           stream or None)
    check(rc, "rnnt_multiblank_grad_scale")


def workspace_size_multiblank_padded(B: int, V: int, max_T: int, max_U1: int, dtype_code: int, logit_lengths,
                                     target_lengths, big_blank_durations) -> int:
    T = host_i32(logit_lengths)
    U = host_i32(target_lengths)
    if len(T) != B or len(U) != B:
        raise ValueError("length vectors must have B entries")
    dur = host_i32(big_blank_durations).reshape(-1)
    nb = len(dur)
    out = ctypes.c_size_t()
    check(load().rnnt_multiblank_padded_workspace_size(B, V, max_T, max_U1, dtype_code, _b(T), _b(U), nb,
                                                       _b(dur if nb else np.zeros(1, np.int32)), ctypes.byref(out)),
          "rnnt_multiblank_padded_workspace_size")
    return int(out.value)


def loss_multiblank_padded(logits_ptr: int, dtype_code: int, max_T: int, max_U1: int, V: int, targets_ptr: int,
                           S: int, logit_lengths, target_lengths, blank: int, big_blank_ids, big_blank_durations,
                           sigma: float, clamp: float, fastemit_lambda: float, fused: bool, reduction: str,
                           loss_ptr: int, loss_reduced_ptr: int, grad_ptr: int, ws_ptr: int, ws_bytes: int,
                           stream: int):
    T = host_i32(logit_lengths)
    U = host_i32(target_lengths)
    B = len(T)
    if len(U) != B:
        raise ValueError("length vectors must have B entries")
    if reduction not in REDUCTIONS:
        raise ValueError(f"reduction must be one of {sorted(REDUCTIONS)}")
    nb, ids, dur = _big_blanks(big_blank_ids, big_blank_durations)
    rc = load().rnnt_multiblank_loss_padded(logits_ptr or None, dtype_code, max_T, max_U1, V, targets_ptr or None, S,
                                            _b(T), _b(U), B, int(blank), nb, _b(ids), _b(dur), float(sigma),
                                            float(clamp), float(fastemit_lambda), int(bool(fused)),
                                            REDUCTIONS[reduction], loss_ptr or None, loss_reduced_ptr or None,
                                            grad_ptr or None, ws_ptr or None, ws_bytes, stream or None)
    check(rc, "rnnt_multiblank_loss_padded")


def grad_scale_multiblank_padded(grad_ptr: int, dtype_code: int, max_T: int, max_U1: int, V: int, logit_lengths,
                                 target_lengths, scale_ptr: int, per_sample: bool, ws_ptr: int, ws_bytes: int,
                                 stream: int):
    T = host_i32(logit_lengths)
    U = host_i32(target_lengths)
    rc = load().rnnt_multiblank_grad_scale_padded(grad_ptr or None, dtype_code, max_T, max_U1, V, _b(T), _b(U),
                                                  len(T), scale_ptr or None, int(bool(per_sample)), ws_ptr or None,
                                                  ws_bytes, stream or None)
    check(rc, "rnnt_multiblank_grad_scale_padded")
