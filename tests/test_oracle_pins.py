"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these checks retypes the oracle's recursion.  Each compares it with
an independent fact:

* brute-force enumeration of every alignment path (definition of the loss as
  a sum over alignments: warp-transducer build post, section 1.1);
* the all-zero-logit closed forms for the loss and, derived from path
  counting, for the whole gradient;
* invariants: alpha-path loss == beta-path loss (rnnt-loss-ascend README,
  "Value" section 3, dual-loss cross-check), fused-gradient rows sum to zero,
  each anti-diagonal carries total occupancy one, the non-fused gradient
  sums to -(T+U);
* the chain rule linking the fused and non-fused gradients via a library
  log_softmax; shift invariance of the fused path;
* central finite differences of the loss;
* single-path special cases (U = 0 and T = 1);
* clamp and reduction semantics of the README parameter table / usage example.
"""
import math

import numpy as np
import pytest
from scipy.special import log_softmax as sp_log_softmax

import oracle
from oracle import bruteforce


def _rand_case(rng, T, U, V, blank, std=1.0):
    x = rng.normal(0.0, std, size=(T * (U + 1), V))
    ids = [k for k in range(V) if k != blank]
    y = rng.choice(ids, size=U) if U > 0 else np.zeros(0, np.int64)
    return x, y


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("T,U", [(1, 0), (1, 1), (1, 3), (2, 0), (2, 1), (3, 2), (4, 3), (5, 2), (2, 5), (6, 4)])
def test_bruteforce_small_lattices(T, U, fused):
    rng = np.random.default_rng(100 * T + U + (7 if fused else 0))
    V, blank = 5, 2
    x, y = _rand_case(rng, T, U, V, blank)
    if not fused:
        x = sp_log_softmax(x, axis=1) + rng.normal(0, 0.1, size=x.shape)  # log-probs, not exactly normalised
    bf_loss, bf_grad = bruteforce.sample(x, T, U, y, blank, fused)
    r = oracle.sample(x, T, U, y, blank, fused)
    assert abs(r.loss - bf_loss) <= 1e-12 * max(1.0, abs(bf_loss))
    assert abs(r.loss_alpha - bf_loss) <= 1e-12 * max(1.0, abs(bf_loss))
    np.testing.assert_allclose(r.grad, bf_grad, atol=1e-12, rtol=0)


def test_bruteforce_tiny_workload():
    """Both samples of the tiny workload shape (T=[12,9], U=[4,3], V=16): 1365 and 165 paths."""
    rng = np.random.default_rng(11)
    V, blank = 16, 15
    for T, U in [(12, 4), (9, 3)]:
        x, y = _rand_case(rng, T, U, V, blank)
        assert bruteforce.count_paths(T, U) == {(12, 4): 1365, (9, 3): 165}[(T, U)]
        bf_loss, bf_grad = bruteforce.sample(x, T, U, y, blank, True)
        r = oracle.sample(x, T, U, y, blank, True)
        assert abs(r.loss - bf_loss) <= 1e-11 * abs(bf_loss)
        np.testing.assert_allclose(r.grad, bf_grad, atol=1e-12, rtol=0)


def _log_comb(n, k):
    return math.lgamma(n + 1) - math.lgamma(k + 1) - math.lgamma(n - k + 1)


@pytest.mark.parametrize("T,U,V", [(1, 0, 3), (1, 5, 7), (12, 4, 16), (9, 3, 16), (50, 10, 29), (300, 80, 1024),
                                   (600, 150, 4096)])
def test_zero_logits_loss_closed_form(T, U, V):
    """All-zero logits: every path has probability V^-(T+U), there are C(T-1+U, U) of them."""
    x = np.zeros((T * (U + 1), V))
    y = np.arange(U) % (V - 1)
    r = oracle.sample(x, T, U, y, V - 1, True, want_grad=False)
    expect = -_log_comb(T - 1 + U, U) + (T + U) * math.log(V)
    assert abs(r.loss - expect) <= 1e-12 * max(1.0, abs(expect))


@pytest.mark.parametrize("T,U,V,blank", [(1, 0, 4, 0), (3, 2, 5, 4), (7, 3, 6, 0), (12, 4, 16, 15), (20, 9, 11, 5)])
def test_zero_logits_gradient_closed_form(T, U, V, blank):
    """All-zero logits: occupancy and edge flows are ratios of path counts.

    occ(t,u)    = C(t+u,u) C(T-1-t+U-u, U-u) / C(T-1+U, U)
    flow_b(t,u) = C(t+u,u) C(T-2-t+U-u, U-u) / C(T-1+U, U)    (t < T-1); occ at (T-1,U); 0 at t=T-1, u<U
    flow_y(t,u) = C(t+u,u) C(T-1-t+U-u-1, U-u-1) / C(T-1+U, U)  (u < U)
    grad_k      = occ/V - [k=blank] flow_b - [k=y_{u+1}] flow_y
    """
    rng = np.random.default_rng(T * 31 + U)
    ids = [k for k in range(V) if k != blank]
    y = rng.choice(ids, size=U) if U else np.zeros(0, np.int64)
    x = np.zeros((T * (U + 1), V))
    r = oracle.sample(x, T, U, y, blank, True)
    C = math.comb
    total = C(T - 1 + U, U)
    expect = np.zeros_like(x)
    for t in range(T):
        for u in range(U + 1):
            row = t * (U + 1) + u
            occ = C(t + u, u) * C(T - 1 - t + U - u, U - u) / total
            if t < T - 1:
                fb = C(t + u, u) * C(T - 2 - t + U - u, U - u) / total
            elif u == U:
                fb = occ
            else:
                fb = 0.0
            fy = C(t + u, u) * C(T - 1 - t + U - u - 1, U - u - 1) / total if u < U else 0.0
            expect[row, :] = occ / V
            expect[row, blank] -= fb
            if u < U:
                expect[row, y[u]] -= fy
    np.testing.assert_allclose(r.grad, expect, atol=1e-14, rtol=0)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_alpha_beta_agree_and_occupancy(seed):
    rng = np.random.default_rng(seed)
    T, U, V, blank = 60 + 20 * seed, 15 + 5 * seed, 37, 0
    x, y = _rand_case(rng, T, U, V, blank, std=2.0)
    r = oracle.sample(x, T, U, y, blank, True, want_tables=True)
    assert abs(r.loss - r.loss_alpha) <= 1e-12 * abs(r.loss)
    logz = r.beta[0, 0]
    assert abs(-logz - r.loss) == 0.0
    occ = np.exp(r.alpha + r.beta - logz)
    for n in range(T + U):
        s = sum(occ[t, n - t] for t in range(max(0, n - U), min(T - 1, n) + 1))
        assert abs(s - 1.0) < 1e-11, (n, s)
    # Each fused gradient row sums to zero (softmax probabilities sum to one).
    assert np.abs(r.grad.sum(axis=1)).max() < 1e-13


def test_nonfused_gradient_counts_emissions():
    rng = np.random.default_rng(5)
    T, U, V, blank = 40, 12, 20, 19
    x, y = _rand_case(rng, T, U, V, blank)
    lp = sp_log_softmax(x, axis=1)
    r = oracle.sample(lp, T, U, y, blank, False)
    # Every path makes exactly T blank and U label emissions.
    assert abs(r.grad.sum() + (T + U)) < 1e-10
    assert abs(r.grad[:, blank].sum() + T) < 1e-10
    nnz = (r.grad != 0).sum(axis=1)
    assert nnz.max() <= 2


def test_fused_equals_chain_rule_of_nonfused():
    rng = np.random.default_rng(6)
    T, U, V, blank = 25, 7, 13, 3
    x, y = _rand_case(rng, T, U, V, blank, std=1.5)
    lp = sp_log_softmax(x, axis=1)
    rf = oracle.sample(x, T, U, y, blank, True)
    rn = oracle.sample(lp, T, U, y, blank, False)
    assert abs(rf.loss - rn.loss) <= 1e-12 * abs(rf.loss)
    p = np.exp(lp)
    expect = rn.grad - p * rn.grad.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(rf.grad, expect, atol=1e-13, rtol=0)


def test_fused_shift_invariance():
    rng = np.random.default_rng(7)
    T, U, V, blank = 15, 6, 9, 8
    x, y = _rand_case(rng, T, U, V, blank)
    shift = rng.normal(0, 5.0, size=(x.shape[0], 1))
    a = oracle.sample(x, T, U, y, blank, True)
    b = oracle.sample(x + shift, T, U, y, blank, True)
    assert abs(a.loss - b.loss) <= 1e-12 * abs(a.loss)
    np.testing.assert_allclose(a.grad, b.grad, atol=1e-13, rtol=0)


@pytest.mark.parametrize("fused", [True, False])
def test_central_finite_differences(fused):
    rng = np.random.default_rng(8 + fused)
    T, U, V, blank = 6, 4, 7, 0
    x, y = _rand_case(rng, T, U, V, blank)
    if not fused:
        x = sp_log_softmax(x, axis=1)
    g = oracle.sample(x, T, U, y, blank, fused).grad
    eps = 1e-6
    for _ in range(40):
        r = rng.integers(0, x.shape[0])
        k = rng.integers(0, V)
        xp = x.copy(); xp[r, k] += eps
        xm = x.copy(); xm[r, k] -= eps
        fd = (oracle.sample(xp, T, U, y, blank, fused, want_grad=False).loss
              - oracle.sample(xm, T, U, y, blank, fused, want_grad=False).loss) / (2 * eps)
        assert abs(fd - g[r, k]) < 1e-8, (r, k, fd, g[r, k])


def test_central_finite_differences_char_sized():
    """Random elements of a character-vocabulary-sized sample (T=70, U=20, V=29)."""
    rng = np.random.default_rng(9)
    T, U, V, blank = 70, 20, 29, 0
    x, y = _rand_case(rng, T, U, V, blank)
    g = oracle.sample(x, T, U, y, blank, True).grad
    eps = 1e-6
    for _ in range(12):
        r = rng.integers(0, x.shape[0])
        k = rng.integers(0, V)
        xp = x.copy(); xp[r, k] += eps
        xm = x.copy(); xm[r, k] -= eps
        fd = (oracle.sample(xp, T, U, y, blank, True, want_grad=False).loss
              - oracle.sample(xm, T, U, y, blank, True, want_grad=False).loss) / (2 * eps)
        assert abs(fd - g[r, k]) < 1e-7, (r, k, fd, g[r, k])


def test_single_path_special_cases():
    rng = np.random.default_rng(10)
    V, blank = 11, 4
    # U = 0: the only path emits blank at every frame.
    T = 9
    x, _ = _rand_case(rng, T, 0, V, blank)
    lp = sp_log_softmax(x, axis=1)
    r = oracle.sample(x, T, 0, [], blank, True)
    assert abs(r.loss + lp[:, blank].sum()) < 1e-12
    # T = 1: the only path emits all labels at t=0, then one blank.
    U = 6
    x, y = _rand_case(rng, 1, U, V, blank)
    lp = sp_log_softmax(x, axis=1)
    expect = -sum(lp[u, y[u]] for u in range(U)) - lp[U, blank]
    r = oracle.sample(x, 1, U, y, blank, True)
    assert abs(r.loss - expect) < 1e-12


def test_clamp_semantics():
    rng = np.random.default_rng(12)
    T, U, V, blank = 20, 5, 6, 5
    x, y = _rand_case(rng, T, U, V, blank, std=3.0)
    g = oracle.sample(x, T, U, y, blank, True).grad
    for c in (0.02, 0.1, 0.3):
        gc = oracle.sample(x, T, U, y, blank, True, clamp=c).grad
        np.testing.assert_array_equal(gc, np.clip(g, -c, c))
    for off in (0.0, -1.0):
        np.testing.assert_array_equal(oracle.sample(x, T, U, y, blank, True, clamp=off).grad, g)


def test_batch_reductions_and_permutation():
    rng = np.random.default_rng(13)
    V = 8
    Ts, Us = [4, 6, 3], [2, 1, 0]
    xs, ys = [], np.zeros((3, 2), np.int32)
    for i, (T, U) in enumerate(zip(Ts, Us)):
        x, y = _rand_case(rng, T, U, V, V - 1)
        xs.append(x)
        ys[i, :U] = y
    logits = np.concatenate(xs)
    loss, red, g, gr = oracle.batch(logits, ys, Ts, Us, blank=-1, reduction="mean")
    assert abs(red - loss.mean()) < 1e-14
    np.testing.assert_allclose(gr, g / 3, rtol=0, atol=1e-15)
    _, red_s, _, gr_s = oracle.batch(logits, ys, Ts, Us, blank=-1, reduction="sum")
    assert abs(red_s - loss.sum()) < 1e-13
    np.testing.assert_array_equal(gr_s, g)
    perm = [2, 0, 1]
    logits_p = np.concatenate([xs[i] for i in perm])
    loss_p, _, g_p, _ = oracle.batch(logits_p, ys[perm], [Ts[i] for i in perm], [Us[i] for i in perm],
                                     blank=V - 1, reduction="none")
    np.testing.assert_array_equal(loss_p, loss[perm])
    off = np.concatenate([[0], np.cumsum([T * (U + 1) for T, U in zip(Ts, Us)])])
    np.testing.assert_array_equal(g_p, np.concatenate([g[off[i]:off[i + 1]] for i in perm]))


def test_blank_normalisation_and_bad_targets():
    assert oracle.normalize_blank(-1, 10) == 9
    assert oracle.normalize_blank(-10, 10) == 0
    assert oracle.normalize_blank(9, 10) == 9
    with pytest.raises(ValueError):
        oracle.normalize_blank(10, 10)
    with pytest.raises(ValueError):
        oracle.normalize_blank(-11, 10)
    x = np.zeros((3 * 2, 5))
    with pytest.raises(ValueError):
        oracle.sample(x, 3, 1, [4], 4)   # label equal to blank
    with pytest.raises(ValueError):
        oracle.sample(x, 3, 1, [5], 4)   # label outside [0, V)


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("bad", [4, 5, -1])
def test_label_that_is_not_a_symbol_leaves_no_alignment(fused, bad):
    """The build post's section 5.2 rules blank out of the labels; a label equal to blank (4 here) or outside
    [0, V) is a symbol no alignment can emit.  Every alignment emits every label exactly once, so the set of
    alignments is empty: P(y|x) = 0, loss +inf, and the gradient of every row is exactly zero (also through the
    log_softmax chain rule).  The same sample with that label replaced by a valid one is finite, so the
    infinity comes from the label alone."""
    rng = np.random.default_rng(7)
    T, U, V = 4, 3, 5
    x = rng.normal(size=(T * (U + 1), V))
    if not fused:
        x = x - np.log(np.exp(x).sum(axis=1, keepdims=True))
    y = [1, bad, 2]
    r = oracle.sample(x, T, U, y, 4, fused=fused, allow_bad_targets=True)
    assert r.bad_target
    assert np.isinf(r.loss) and r.loss > 0 and np.isinf(r.loss_alpha)
    assert np.all(r.grad == 0.0)
    ok = oracle.sample(x, T, U, [1, 3, 2], 4, fused=fused)
    assert np.isfinite(ok.loss) and not ok.bad_target
    # the multi-blank oracle: a label equal to a big blank's class is no symbol either
    m = oracle.multiblank_sample(x, T, U, [1, 3, 2], 4, [3], [2], 0.1, fused=fused, allow_bad_targets=True)
    assert m.bad_target and np.isinf(m.loss) and np.all(m.grad == 0.0)
    m2 = oracle.multiblank_sample(x, T, U, y, 4, [0], [2], 0.1, fused=fused, allow_bad_targets=True)
    assert m2.bad_target and np.isinf(m2.loss) and np.all(m2.grad == 0.0)
    with pytest.raises(ValueError):
        oracle.multiblank_sample(x, T, U, [1, 3, 2], 4, [3], [2], 0.1, fused=fused)


def test_golden_readme_example():
    """The README usage-example layout (24 packed rows, V=8), values stored by tests/golden/make_golden.py."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "readme_example.json")
    with open(path) as f:
        gd = json.load(f)
    logits = np.array(gd["logits"])
    assert logits.shape == (24, 8)
    for case in gd["cases"]:
        loss, red, g, gr = oracle.batch(logits, np.array(gd["targets"], np.int32), gd["logit_lengths"],
                                        gd["target_lengths"], blank=gd["blank"], reduction=case["reduction"])
        np.testing.assert_allclose(np.atleast_1d(red), case["loss"], rtol=1e-13, atol=0)
        np.testing.assert_allclose(gr, np.array(case["grad"]), rtol=0, atol=1e-15)
        # Independent recomputation of each sample by path enumeration.
        off = 0
        for i, (T, U) in enumerate(zip(gd["logit_lengths"], gd["target_lengths"])):
            rows = T * (U + 1)
            bl, _ = bruteforce.sample(logits[off:off + rows], T, U, gd["targets"][i], 7, True)
            assert abs(bl - case["loss_per_sample"][i]) < 1e-12
            off += rows


def test_half_conversion_exact_for_every_half():
    """The oracle reads fp16 inputs through its own binary16 decoder: all 65536 encodings."""
    bits = np.arange(65536, dtype=np.uint16)
    expect = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    same = (got == expect) | (np.isnan(got) & np.isnan(expect))
    assert same.all()


def test_native_dtypes_and_row_subsets():
    """fp32 / fp16 inputs are read exactly; a row subset of the gradient equals those rows of the full one."""
    rng = np.random.default_rng(14)
    T, U, V, blank = 9, 4, 24, 0
    x, y = _rand_case(rng, T, U, V, blank, std=2.0)
    for dt in (np.float32, np.float16):
        xd = x.astype(dt)
        a = oracle.sample(xd, T, U, y, blank, True)
        b = oracle.sample(xd.astype(np.float64), T, U, y, blank, True)
        assert a.loss == b.loss
        np.testing.assert_array_equal(a.grad, b.grad)
        rows = [7, 0, T * (U + 1) - 1, 3]
        c = oracle.sample(xd, T, U, y, blank, True, rows=rows)
        np.testing.assert_array_equal(c.grad, a.grad[rows])


# FastEmit (fastemit_lambda of the GPURNNT parameter list on the ESPnet
# multi-blank utilities page, defined by the FastEmit paper it refers to):
# the derivative with respect to every label-emission log-probability is
# weighted by (1 + lambda); blank emissions and the loss value are unchanged.

@pytest.mark.parametrize("lam", [0.01, 0.5, 2.0])
@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("T,U", [(1, 3), (3, 2), (4, 3), (2, 5), (6, 4)])
def test_fastemit_bruteforce(T, U, fused, lam):
    rng = np.random.default_rng(1000 * T + 10 * U + int(fused))
    V, blank = 6, 0
    x, y = _rand_case(rng, T, U, V, blank, std=1.5)
    if not fused:
        x = sp_log_softmax(x, axis=1) + rng.normal(0, 0.1, size=x.shape)
    bf_loss, bf_grad = bruteforce.sample(x, T, U, y, blank, fused, fastemit_lambda=lam)
    r = oracle.sample(x, T, U, y, blank, fused, fastemit_lambda=lam)
    assert abs(r.loss - bf_loss) <= 1e-12 * max(1.0, abs(bf_loss))
    np.testing.assert_allclose(r.grad, bf_grad, atol=1e-12, rtol=0)


@pytest.mark.parametrize("T,U,V,blank,lam", [(3, 2, 5, 4, 0.3), (7, 3, 6, 0, 0.01), (12, 4, 16, 15, 1.5)])
def test_fastemit_zero_logits_closed_form(T, U, V, blank, lam):
    """All-zero logits, with the path-count flows of the plain closed form:
    grad_k = (occ + lam flow_y)/V - [k=blank] flow_b - [k=y_{u+1}] (1+lam) flow_y."""
    rng = np.random.default_rng(T * 17 + U)
    ids = [k for k in range(V) if k != blank]
    y = rng.choice(ids, size=U)
    x = np.zeros((T * (U + 1), V))
    r = oracle.sample(x, T, U, y, blank, True, fastemit_lambda=lam)
    C = math.comb
    total = C(T - 1 + U, U)
    expect = np.zeros_like(x)
    for t in range(T):
        for u in range(U + 1):
            row = t * (U + 1) + u
            occ = C(t + u, u) * C(T - 1 - t + U - u, U - u) / total
            fb = (C(t + u, u) * C(T - 2 - t + U - u, U - u) / total if t < T - 1
                  else (occ if u == U else 0.0))
            fy = C(t + u, u) * C(T - 2 - t + U - u, U - u - 1) / total if u < U else 0.0
            expect[row, :] = (occ + lam * fy) / V
            expect[row, blank] -= fb
            if u < U:
                expect[row, y[u]] -= (1.0 + lam) * fy
    np.testing.assert_allclose(r.grad, expect, atol=1e-14, rtol=0)


def test_fastemit_invariants():
    """Loss unchanged; fused rows still sum to zero; the non-fused gradient sums to -(T + (1+lam) U) with the
    blank column untouched."""
    rng = np.random.default_rng(21)
    T, U, V, blank, lam = 30, 9, 17, 16, 0.25
    x, y = _rand_case(rng, T, U, V, blank, std=2.0)
    a = oracle.sample(x, T, U, y, blank, True)
    b = oracle.sample(x, T, U, y, blank, True, fastemit_lambda=lam)
    assert a.loss == b.loss and a.loss_alpha == b.loss_alpha
    assert np.abs(b.grad.sum(axis=1)).max() < 1e-13
    lp = sp_log_softmax(x, axis=1)
    n0 = oracle.sample(lp, T, U, y, blank, False)
    n1 = oracle.sample(lp, T, U, y, blank, False, fastemit_lambda=lam)
    assert abs(n1.grad.sum() + (T + (1 + lam) * U)) < 1e-10
    np.testing.assert_array_equal(n1.grad[:, blank], n0.grad[:, blank])
    with pytest.raises(ValueError):
        oracle.sample(x, T, U, y, blank, True, fastemit_lambda=-0.1)
    with pytest.raises(ValueError):
        oracle.sample(x, T, U, y, blank, True, fastemit_lambda=float("inf"))


def test_fastemit_finite_differences():
    """Central differences split the fused gradient into its label-emission part: perturbing x only where it
    enters the label log-probabilities (the blank log-probabilities keep the unperturbed x).  FastEmit adds
    lam times that part to the full derivative."""
    rng = np.random.default_rng(22)
    T, U, V, blank, lam = 6, 4, 7, 0, 0.7
    x, y = _rand_case(rng, T, U, V, blank)
    g = oracle.sample(x, T, U, y, blank, True, fastemit_lambda=lam).grad
    lp0 = sp_log_softmax(x, axis=1)
    U1 = U + 1

    def loss_full(xx):
        return oracle.sample(xx, T, U, y, blank, True, want_grad=False).loss

    def loss_label_only(xx, r):
        lp = lp0.copy()
        u = r % U1
        if u < U:
            lp[r, y[u]] = sp_log_softmax(xx[r])[y[u]]
        return oracle.sample(lp, T, U, y, blank, False, want_grad=False).loss

    eps = 1e-6
    for _ in range(40):
        r = int(rng.integers(0, x.shape[0]))
        k = int(rng.integers(0, V))
        xp = x.copy(); xp[r, k] += eps
        xm = x.copy(); xm[r, k] -= eps
        fd_full = (loss_full(xp) - loss_full(xm)) / (2 * eps)
        fd_label = (loss_label_only(xp, r) - loss_label_only(xm, r)) / (2 * eps)
        assert abs(fd_full + lam * fd_label - g[r, k]) < 1e-8, (r, k)


# Multi-blank transducer (the compute_multiblank_grad_kernel page: big blanks with durations and sigma, the
# logit under-normalisation).  Reading: big blank i moves (t,u) -> (t+d_i,u); every emission's log-probability is
# lowered by sigma; an alignment ends when a blank of any kind lands exactly on t = T at u = U.

@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("T,U,ids,durs,sigma,lam", [
    (1, 2, [3], [2], 0.0, 0.0), (2, 1, [3], [2], 0.1, 0.0), (4, 2, [5, 4], [2, 3], 0.3, 0.0),
    (6, 1, [5, 4, 3], [2, 4, 6], 0.05, 0.2), (5, 3, [1], [1], 0.0, 0.0), (7, 2, [0, 2], [3, 8], -0.2, 0.5)])
def test_multiblank_bruteforce(T, U, ids, durs, sigma, lam, fused):
    rng = np.random.default_rng(T * 100 + U * 10 + len(ids) + int(fused))
    V, blank = 7, 6
    x = rng.normal(0.0, 1.5, size=(T * (U + 1), V))
    labels = [k for k in range(V) if k != blank and k not in ids]
    y = rng.choice(labels, size=U)
    if not fused:
        x = sp_log_softmax(x, axis=1) + rng.normal(0, 0.1, size=x.shape)
    bl, bg = bruteforce.multiblank_sample(x, T, U, y, blank, ids, durs, sigma, fused, lam)
    r = oracle.multiblank_sample(x, T, U, y, blank, ids, durs, sigma, fused, fastemit_lambda=lam)
    assert abs(r.loss - bl) <= 1e-12 * max(1.0, abs(bl))
    assert abs(r.loss_alpha - bl) <= 1e-12 * max(1.0, abs(bl))
    np.testing.assert_allclose(r.grad, bg, atol=1e-12, rtol=0)


def test_multiblank_path_counts():
    # no big blank: C(T-1+U, U) alignments; durations {2}: compositions of T into parts 1 and 2 (Fibonacci F(T+1))
    # interleaved with the U labels, which may only come before the last blank
    assert bruteforce.count_multiblank_paths(6, 0, []) == 1
    assert bruteforce.count_multiblank_paths(6, 0, [2]) == 13           # F(7)
    assert bruteforce.count_multiblank_paths(5, 2, []) == math.comb(6, 2)


def test_multiblank_reduces_to_the_plain_loss():
    rng = np.random.default_rng(31)
    T, U, V, blank = 23, 6, 11, 10
    x, y = _rand_case(rng, T, U, V, blank, std=2.0)
    p = oracle.sample(x, T, U, y, blank, True)
    m = oracle.multiblank_sample(x, T, U, y, blank, [], [], 0.0, True)
    assert abs(m.loss - p.loss) <= 1e-13 * abs(p.loss)
    np.testing.assert_allclose(m.grad, p.grad, atol=1e-15, rtol=0)
    # sigma alone: every alignment makes T + U emissions, so the loss moves by sigma (T + U), the gradient not at all
    s = oracle.multiblank_sample(x, T, U, y, blank, [], [], 0.37, True)
    assert abs(s.loss - (p.loss + 0.37 * (T + U))) <= 1e-12 * abs(p.loss)
    np.testing.assert_allclose(s.grad, p.grad, atol=1e-13, rtol=0)
    # a big blank longer than T can never be taken: the plain loss and gradient
    ids = [k for k in range(V) if k != blank and k not in y][:1]
    z = oracle.multiblank_sample(x, T, U, y, blank, ids, [T + 1], 0.0, True)
    assert abs(z.loss - p.loss) <= 1e-13 * abs(p.loss)
    np.testing.assert_allclose(z.grad, p.grad, atol=1e-15, rtol=0)


def test_multiblank_invariants():
    """Fused rows sum to zero; non-fused flows: the blanks of all kinds advance t by exactly T in total, the
    labels are emitted U times; alpha and beta agree."""
    rng = np.random.default_rng(32)
    T, U, V, blank = 40, 9, 13, 0
    ids, durs = [12, 11], [2, 4]
    labels = [k for k in range(V) if k not in (blank, 12, 11)]
    x = rng.normal(0.0, 2.0, size=(T * (U + 1), V))
    y = rng.choice(labels, size=U)
    f = oracle.multiblank_sample(x, T, U, y, blank, ids, durs, 0.25, True)
    assert abs(f.loss - f.loss_alpha) <= 1e-12 * abs(f.loss)
    assert np.abs(f.grad.sum(axis=1)).max() < 1e-13
    lp = sp_log_softmax(x, axis=1)
    n = oracle.multiblank_sample(lp, T, U, y, blank, ids, durs, 0.25, False)
    advance = -(n.grad[:, blank].sum() + 2 * n.grad[:, 12].sum() + 4 * n.grad[:, 11].sum())
    assert abs(advance - T) < 1e-10
    assert abs(-n.grad[:, labels].sum() - U) < 1e-10
    with pytest.raises(ValueError):
        oracle.multiblank_sample(x, T, U, y, blank, [blank], [2], 0.0, True)       # big blank equal to blank
    with pytest.raises(ValueError):
        oracle.multiblank_sample(x, T, U, [12] * U, blank, ids, durs, 0.0, True)  # label equal to a big blank


def test_multiblank_finite_differences():
    rng = np.random.default_rng(33)
    T, U, V, blank = 9, 3, 8, 7
    ids, durs = [6, 5], [2, 3]
    x = rng.normal(0.0, 1.0, size=(T * (U + 1), V))
    y = rng.choice([0, 1, 2, 3, 4], size=U)
    g = oracle.multiblank_sample(x, T, U, y, blank, ids, durs, 0.2, True).grad
    eps = 1e-6
    for _ in range(40):
        r = int(rng.integers(0, x.shape[0]))
        k = int(rng.integers(0, V))
        xp = x.copy(); xp[r, k] += eps
        xm = x.copy(); xm[r, k] -= eps
        fd = (oracle.multiblank_sample(xp, T, U, y, blank, ids, durs, 0.2, True, want_grad=False).loss
              - oracle.multiblank_sample(xm, T, U, y, blank, ids, durs, 0.2, True, want_grad=False).loss) / (2 * eps)
        assert abs(fd - g[r, k]) < 1e-8, (r, k)
