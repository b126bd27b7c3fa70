"""Seeded synthetic RNN-T workloads shared by the tests, the smoke check and the bench.

This module holds input generation only and none of the method's arithmetic.
The five named workloads follow the shapes and value distributions of the
headline configurations (tiny / character vocabulary / BPE batch / half
precision / skewed long-form):

    name      B   T                         target length U              V     dtype  logits      blank  clamp  fused  reduction
    tiny      2   [12, 9]                   [4, 3]                      16     fp32   N(0,1)      -1     off    yes    none
    char      8   U{50..100}                U{10..30}                   29     fp32   N(0,1)       0     off    yes    sum
    bpe      32   U{200..400}               U{40..100}                1024     fp32   N(0,2^2)    -1     off    yes    mean
    half     16   U{300..600}               U{50..150}                4096     fp16   N(0,2^2)    -1     1.0    yes    mean
    skewed   64   lognormal(ln 300, 0.6)    round(T/5*U(0.6,1.0))     2048     fp16   log_softmax(N(0,1.5^2)) -1 off no sum
                  clipped to [50, 1600]
    vocab5k   4   U{800..1000}              U{150..200}               5000     fp32   N(0,2^2)    -1     off    yes    mean

(vocab5k: rows of 20000 bytes, wider than the 16 KiB a wave holds in registers; the rnnt-loss-ascend
README's "Performance data" shape B=16, T=1000, U=200, V=5000, with four samples so that the logits
and the gradient, 16 GB each, fit beside each other on one GPU)

plus one multi-blank workload, the bpe shapes with three big blanks (classes
1022, 1021, 1020 of durations 2, 4, 8 frames) beside the standard blank 1023
and sigma 0.05 (the logit under-normalisation):

    multiblank 32 U{200..400}               U{40..100}                1024     fp32   N(0,2^2)    -1     off    yes    mean

Draw order (numpy ``default_rng(seed)``): T[B], then U[B], then the padded
targets (B, max U) uniform over the non-blank ids (the big blanks excluded;
padding is 0 and never read), all on the host.  Logits are drawn per sample with torch's Philox
generator on the requested device, seeded with ``seed * 1000003 + i``, as
fp32 and rounded to fp16 (round-to-nearest-even) where the workload is fp16.
The skewed workload's inputs are log-probabilities: each sample's fp32 draw
is passed through a library log_softmax in fp64 and then rounded to fp16,
which is how that workload feeds pre-normalised inputs to the non-fused path.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch

NAMES = ("tiny", "char", "bpe", "half", "skewed", "multiblank", "vocab5k")
DEFAULT_SEEDS = {"tiny": 1, "char": 2, "bpe": 3, "half": 4, "skewed": 5, "multiblank": 6, "vocab5k": 7}
# big-blank classes, durations and sigma of the multi-blank workload
MULTIBLANK = {"big_blank_ids": (1022, 1021, 1020), "big_blank_durations": (2, 4, 8), "sigma": 0.05}


@dataclasses.dataclass
class Workload:
    name: str
    V: int
    blank: int                 # as passed by the caller (may be negative)
    clamp: float
    fused: bool
    reduction: str
    logit_lengths: np.ndarray  # int32 (B,)
    target_lengths: np.ndarray  # int32 (B,)
    targets: np.ndarray        # int32 (B, S), zero padded
    logits: torch.Tensor       # (N, V) fp32/fp16, packed t-major per sample
    offsets: np.ndarray        # int64 (B+1,), row offset of each sample
    big_blank_ids: tuple = ()  # multi-blank workloads only
    big_blank_durations: tuple = ()
    sigma: float = 0.0

    @property
    def B(self) -> int:
        return int(len(self.logit_lengths))

    @property
    def N(self) -> int:
        return int(self.offsets[-1])

    @property
    def dtype(self) -> torch.dtype:
        return self.logits.dtype

    def rows(self, i: int) -> slice:
        return slice(int(self.offsets[i]), int(self.offsets[i + 1]))


def _offsets(T: np.ndarray, U: np.ndarray) -> np.ndarray:
    off = np.zeros(len(T) + 1, np.int64)
    off[1:] = np.cumsum(T.astype(np.int64) * (U.astype(np.int64) + 1))
    return off


def _draw_targets(rng: np.random.Generator, U: np.ndarray, V: int, blank_norm: int, exclude=()) -> np.ndarray:
    S = max(1, int(U.max()) if len(U) else 1)
    ids = np.array([k for k in range(V) if k != blank_norm and k not in exclude], np.int64)
    tg = np.zeros((len(U), S), np.int32)
    for i, u in enumerate(U):
        if u > 0:
            tg[i, :u] = ids[rng.integers(0, len(ids), size=int(u))]
    return tg


def _draw_logits(T, U, V, std, dtype, seed, device, prenormalise=False) -> torch.Tensor:
    off = _offsets(T, U)
    out = torch.empty((int(off[-1]), V), dtype=dtype, device=device)
    gen = torch.Generator(device=device)
    chunk = 1 << 16
    for i in range(len(T)):
        gen.manual_seed(int(seed) * 1000003 + i)
        a, b = int(off[i]), int(off[i + 1])
        for r in range(a, b, chunk):
            e = min(b, r + chunk)
            x = torch.randn((e - r, V), generator=gen, device=device, dtype=torch.float32)
            if std != 1.0:
                x.mul_(std)
            if prenormalise:
                x = torch.log_softmax(x.double(), dim=1)
            out[r:e] = x.to(dtype)
    return out


def make_custom(T: List[int], U: List[int], V: int, *, dtype=torch.float32, std: float = 1.0,
                blank: int = -1, clamp: float = -1.0, fused: bool = True, reduction: str = "mean",
                seed: int = 0, device="cpu", prenormalise: bool = False, name: str = "custom",
                targets: Optional[np.ndarray] = None, big_blank_ids=(), big_blank_durations=(),
                sigma: float = 0.0) -> Workload:
    """A workload with explicit per-sample lengths (edge cases, small parity cases); targets avoid the blank
    and any big blank."""
    T = np.asarray(T, np.int32)
    U = np.asarray(U, np.int32)
    bn = blank + V if blank < 0 else blank
    rng = np.random.default_rng(seed)
    tg = (_draw_targets(rng, U, V, bn, tuple(big_blank_ids)) if targets is None
          else np.asarray(targets, np.int32))
    logits = _draw_logits(T, U, V, std, dtype, seed, device, prenormalise)
    return Workload(name, V, blank, clamp, fused, reduction, T, U, tg, logits, _offsets(T, U),
                    tuple(big_blank_ids), tuple(big_blank_durations), float(sigma))


def lengths(name: str, seed: Optional[int] = None, vocab: Optional[int] = None):
    """(T, U, targets, V, blank) of a named workload, without drawing logits; ``vocab`` replaces its V (the
    same lengths, targets drawn over the new classes)."""
    seed = DEFAULT_SEEDS[name] if seed is None else seed
    rng = np.random.default_rng(seed)
    if name == "tiny":
        T = np.array([12, 9], np.int32)
        U = np.array([4, 3], np.int32)
        V, blank = 16, -1
    elif name == "char":
        T = rng.integers(50, 101, size=8).astype(np.int32)
        U = rng.integers(10, 31, size=8).astype(np.int32)
        V, blank = 29, 0
    elif name in ("bpe", "multiblank"):
        T = rng.integers(200, 401, size=32).astype(np.int32)
        U = rng.integers(40, 101, size=32).astype(np.int32)
        V, blank = 1024, -1
    elif name == "half":
        T = rng.integers(300, 601, size=16).astype(np.int32)
        U = rng.integers(50, 151, size=16).astype(np.int32)
        V, blank = 4096, -1
    elif name == "vocab5k":
        T = rng.integers(800, 1001, size=4).astype(np.int32)
        U = rng.integers(150, 201, size=4).astype(np.int32)
        V, blank = 5000, -1
    elif name == "skewed":
        T = np.clip(np.round(np.exp(rng.normal(np.log(300.0), 0.6, size=64))), 50, 1600).astype(np.int32)
        U = np.round(T / 5.0 * rng.uniform(0.6, 1.0, size=64)).astype(np.int32)
        V, blank = 2048, -1
    else:
        raise KeyError(name)
    if vocab is not None:
        if name == "multiblank" or vocab < 2 or (blank >= 0 and blank >= vocab):
            raise ValueError(f"no vocabulary override {vocab} for workload {name}")
        V = int(vocab)
    bn = blank + V if blank < 0 else blank
    tg = _draw_targets(rng, U, V, bn, MULTIBLANK["big_blank_ids"] if name == "multiblank" else ())
    return T, U, tg, V, blank


_PARAMS = {
    #          dtype          std  clamp  fused  reduction prenormalise
    "tiny": (torch.float32, 1.0, -1.0, True, "none", False),
    "char": (torch.float32, 1.0, -1.0, True, "sum", False),
    "bpe": (torch.float32, 2.0, -1.0, True, "mean", False),
    "half": (torch.float16, 2.0, 1.0, True, "mean", False),
    "skewed": (torch.float16, 1.5, -1.0, False, "sum", True),
    "multiblank": (torch.float32, 2.0, -1.0, True, "mean", False),
    "vocab5k": (torch.float32, 2.0, -1.0, True, "mean", False),
}


def make(name: str, seed: Optional[int] = None, device="cpu", vocab: Optional[int] = None) -> Workload:
    """One of the named workloads, fully drawn on ``device`` (``vocab``: another V, as in :func:`lengths`)."""
    seed = DEFAULT_SEEDS[name] if seed is None else seed
    T, U, tg, V, blank = lengths(name, seed, vocab)
    dtype, std, clamp, fused, reduction, pre = _PARAMS[name]
    logits = _draw_logits(T, U, V, std, dtype, seed, device, pre)
    w = Workload(name, V, blank, clamp, fused, reduction, T, U, tg, logits, _offsets(T, U))
    if name == "multiblank":
        w.big_blank_ids = MULTIBLANK["big_blank_ids"]
        w.big_blank_durations = MULTIBLANK["big_blank_durations"]
        w.sigma = MULTIBLANK["sigma"]
    return w


def describe(name: str, seed: Optional[int] = None) -> dict:
    T, U, _, V, blank = lengths(name, seed)
    off = _offsets(T, U)
    dtype = _PARAMS[name][0]
    return {"workload": name, "B": int(len(T)), "V": int(V), "rows": int(off[-1]),
            "elements": int(off[-1]) * int(V), "dtype": "fp16" if dtype == torch.float16 else "fp32",
            "T_max": int(T.max()), "U_max": int(U.max()), "fused_log_softmax": _PARAMS[name][3],
            "reduction": _PARAMS[name][4], "clamp": _PARAMS[name][2], "blank": blank}
