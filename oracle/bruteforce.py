"""Brute-force RNN-T loss by enumerating every alignment path (tiny lattices only).

TEST INFRASTRUCTURE ONLY (imported by ``tests/`` alone).

The definition (warp-transducer build post, section 1.1): the loss is minus
the log of the summed probability of every legal alignment of the target over
the T x (U+1) grid.  An alignment is an ordering of T-1 blank moves (t -> t+1)
and U label moves (u -> u+1) starting at (0,0), followed by one final blank at
(T-1,U).  There are C(T-1+U, U) of them.  Pure Python, no recursion tables:
each path's probability is a product along the path.

The gradient is the expected number of times each (node, symbol) edge is used,
pushed through the log_softmax Jacobian written as an explicit V x V matrix.
With ``fastemit_lambda`` the label edges' expected uses count (1 + lambda)
times (the FastEmit gradient rule, read from the paper the GPURNNT parameter
list of the ESPnet multi-blank utilities page refers to).
"""
from __future__ import annotations

import itertools
import math

import numpy as np


def _paths(T: int, U: int):
    """Yield each alignment as the list of (t, u, emitted) triples it visits."""
    moves = T - 1 + U
    for label_slots in itertools.combinations(range(moves), U):
        chosen = set(label_slots)
        t = u = 0
        steps = []
        for m in range(moves):
            if m in chosen:
                steps.append((t, u, "label"))
                u += 1
            else:
                steps.append((t, u, "blank"))
                t += 1
        steps.append((T - 1, U, "blank"))
        yield steps


def _log_probs(x: np.ndarray, fused: bool) -> np.ndarray:
    if not fused:
        return x.astype(np.float64)
    out = np.empty_like(x, dtype=np.float64)
    for r in range(x.shape[0]):
        row = x[r].astype(np.float64)
        z = sum(math.exp(v) for v in row)
        out[r] = [v - math.log(z) for v in row]
    return out


def sample(x, T: int, U: int, y, blank: int, fused: bool = True, fastemit_lambda: float = 0.0):
    """Return (loss, grad) of one sample by full path enumeration."""
    x = np.asarray(x, dtype=np.float64)
    V = x.shape[1]
    U1 = U + 1
    lp = _log_probs(x, fused)

    path_logp = []
    path_steps = []
    for steps in _paths(T, U):
        s = 0.0
        for (t, u, e) in steps:
            k = blank if e == "blank" else int(y[u])
            s += lp[t * U1 + u, k]
        path_logp.append(s)
        path_steps.append(steps)
    m = max(path_logp)
    Z = sum(math.exp(p - m) for p in path_logp)
    loss = -(m + math.log(Z))

    # d loss / d lp(node, k) = - E[number of uses of edge (node, k)]; a label
    # edge's uses weigh (1 + fastemit_lambda).
    d_lp = np.zeros_like(lp)
    for p, steps in zip(path_logp, path_steps):
        w = math.exp(p - m) / Z
        for (t, u, e) in steps:
            k = blank if e == "blank" else int(y[u])
            d_lp[t * U1 + u, k] -= w if e == "blank" else w * (1.0 + fastemit_lambda)
    if not fused:
        return loss, d_lp
    grad = np.zeros_like(lp)
    for r in range(lp.shape[0]):
        p = np.exp(lp[r])
        # Jacobian of log_softmax: J[j, k] = d lp_j / d x_k = delta_jk - p_k.
        J = np.eye(V) - np.outer(np.ones(V), p)
        grad[r] = d_lp[r] @ J
    return loss, grad


def count_paths(T: int, U: int) -> int:
    return math.comb(T - 1 + U, U)


def _mb_paths(T: int, U: int, durations):
    """Yield each multi-blank alignment as (t, u, kind) steps; kind is "blank", "label" or a big-blank index.

    From a node (t, u) with t < T: the standard blank moves to t+1, big blank i to t+durations[i], the next label
    (u < U) to u+1.  An alignment is complete at exactly (T, U); moves past T or reaching T with u < U are
    dropped.
    """
    def walk(t, u, steps):
        if t == T:
            if u == U:
                yield list(steps)
            return
        moves = [("blank", 1)] + [(i, d) for i, d in enumerate(durations)]
        for kind, d in moves:
            nt = t + d
            if nt < T or (nt == T and u == U):
                steps.append((t, u, kind))
                yield from walk(nt, u, steps)
                steps.pop()
        if u < U:
            steps.append((t, u, "label"))
            yield from walk(t, u + 1, steps)
            steps.pop()

    yield from walk(0, 0, [])


def multiblank_sample(x, T: int, U: int, y, blank: int, big_blank_ids, big_blank_durations, sigma: float = 0.0,
                      fused: bool = True, fastemit_lambda: float = 0.0):
    """(loss, grad) of the multi-blank transducer by enumerating every alignment (tiny lattices only).

    Each emission's log-probability is lowered by sigma; a label edge's expected uses weigh (1 + lambda).
    """
    x = np.asarray(x, dtype=np.float64)
    V = x.shape[1]
    U1 = U + 1
    lp = _log_probs(x, fused) - sigma

    def cls(kind, u):
        if kind == "blank":
            return blank
        if kind == "label":
            return int(y[u])
        return int(big_blank_ids[kind])

    path_logp, path_steps = [], []
    for steps in _mb_paths(T, U, list(big_blank_durations)):
        path_logp.append(sum(lp[t * U1 + u, cls(k, u)] for (t, u, k) in steps))
        path_steps.append(steps)
    m = max(path_logp)
    Z = sum(math.exp(p - m) for p in path_logp)
    loss = -(m + math.log(Z))
    d_lp = np.zeros_like(lp)
    for p, steps in zip(path_logp, path_steps):
        w = math.exp(p - m) / Z
        for (t, u, k) in steps:
            d_lp[t * U1 + u, cls(k, u)] -= w * (1.0 + fastemit_lambda) if k == "label" else w
    if not fused:
        return loss, d_lp
    grad = np.zeros_like(lp)
    for r in range(lp.shape[0]):
        p = np.exp(lp[r] + sigma)
        J = np.eye(V) - np.outer(np.ones(V), p)
        grad[r] = d_lp[r] @ J
    return loss, grad


def count_multiblank_paths(T: int, U: int, durations) -> int:
    return sum(1 for _ in _mb_paths(T, U, list(durations)))
