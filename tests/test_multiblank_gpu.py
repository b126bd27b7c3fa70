"""GPU parity of the multi-blank transducer path against the fp64 oracle (run on an MI355X).

The path (the ESPnet compute_multiblank_grad_kernel page: big blanks with durations and sigma, the logit
under-normalisation) runs through the C ABI (``rnnt_multiblank_loss``) on seeded inputs and is compared element
by element with ``oracle.multiblank_sample`` on the same inputs, to the same gates as the plain path:

    fp32 inputs: loss relative error <= 1e-5, gradient absolute error <= 1e-5
    fp16 inputs: loss relative error <= 2e-3, gradient absolute error <= 3e-3

The per-sample gradient (the output divided by the reduction scale) is held to the gate.
"""
import concurrent.futures as cf
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = {torch.float32: (1e-5, 1e-5), torch.float16: (2e-3, 3e-3)}


@pytest.fixture(scope="module")
def rl():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rnn_transducer_loss_amd as rl
    rl._lib.load()
    return rl


def _threads():
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return 4


def run_mb(rl, w, reduction=None, clamp=None, fastemit=0.0, compute_grad=True):
    reduction = w.reduction if reduction is None else reduction
    clamp = w.clamp if clamp is None else clamp
    tg = torch.from_numpy(w.targets).to("cuda")
    loss, red, grad, ws = rl.rnnt_multiblank_fused(w.logits, tg, w.logit_lengths, w.target_lengths,
                                                   big_blank_ids=w.big_blank_ids,
                                                   big_blank_durations=w.big_blank_durations, blank=w.blank,
                                                   sigma=w.sigma, clamp=clamp, reduction=reduction,
                                                   fused_log_softmax=w.fused, fastemit_lambda=fastemit,
                                                   compute_grad=compute_grad)
    flags = rl.device_flags(ws)
    torch.cuda.synchronize()
    return loss, red, grad, flags


def check_mb(w, loss, grad, reduction, clamp=None, fastemit=0.0, grad_samples=None):
    clamp = w.clamp if clamp is None else clamp
    ltol, gtol = TOL[w.dtype]
    b = w.blank + w.V if w.blank < 0 else w.blank
    scale = 1.0 / w.B if reduction == "mean" else 1.0
    loss_h = loss.detach().cpu().numpy().astype(np.float64)
    want = set(range(w.B) if grad_samples is None else grad_samples) if grad is not None else set()

    def one(i):
        T, U = int(w.logit_lengths[i]), int(w.target_lengths[i])
        x = w.logits[w.rows(i)].detach().cpu().numpy()
        r = oracle.multiblank_sample(x, T, U, w.targets[i], b, w.big_blank_ids, w.big_blank_durations, w.sigma,
                                     w.fused, clamp, fastemit, want_grad=(i in want))
        return i, r

    worst_l, worst_g = 0.0, 0.0
    with cf.ThreadPoolExecutor(_threads()) as ex:
        for i, r in ex.map(one, range(w.B)):
            rel = abs(loss_h[i] - r.loss) / max(1.0, abs(r.loss))
            worst_l = max(worst_l, rel)
            assert rel <= ltol, f"sample {i}: loss {loss_h[i]} vs oracle {r.loss} (rel {rel:.3g})"
            if r.grad is not None:
                g = grad[w.rows(i)].detach().double().cpu().numpy() / scale
                err = np.abs(g - r.grad).max()
                worst_g = max(worst_g, err)
                assert err <= gtol, f"sample {i}: grad max abs err {err:.3g}"
    return worst_l, worst_g


def _mb(Ts, Us, V, ids, durs, sigma=0.0, **kw):
    return workloads.make_custom(Ts, Us, V, device="cuda", big_blank_ids=ids, big_blank_durations=durs, sigma=sigma,
                                 **kw)


@pytest.mark.parametrize("V,dtype,fused,ids,durs,sigma,lam,clamp", [
    (16, torch.float32, True, [14, 13], [2, 3], 0.1, 0.0, -1.0),
    (50, torch.float32, True, [46, 47, 48], [2, 4, 8], 0.05, 0.3, 0.2),
    (1024, torch.float32, True, [1022, 1021, 1020], [2, 4, 8], 0.05, 0.0, -1.0),
    (300, torch.float16, True, [1, 2], [3, 6], 0.0, 0.0, -1.0),
    (64, torch.float32, False, [62], [5], 0.2, 0.0, -1.0),
    (2048, torch.float16, False, [2046, 2045], [2, 4], 0.0, 0.1, -1.0),
    (33, torch.float32, True, [0, 5, 9, 31], [1, 16, 7, 2], -0.1, 0.0, 0.05),
])
def test_multiblank_against_oracle(rl, V, dtype, fused, ids, durs, sigma, lam, clamp):
    # samples shorter than some durations, U = 0, T = 1 and ordinary ones in one batch
    blank = 0 if 0 not in ids and V == 300 else -1
    w = _mb([40, 12, 3, 1, 25], [9, 4, 2, 3, 0], V, ids, durs, sigma, dtype=dtype, std=2.0 if fused else 1.5,
            blank=blank, clamp=clamp, fused=fused, prenormalise=not fused, reduction="mean", seed=V + len(ids))
    loss, red, grad, flags = run_mb(rl, w, fastemit=lam)
    assert flags == 0
    check_mb(w, loss, grad, "mean", fastemit=lam)
    assert abs(red.item() - loss.double().mean().item()) <= 1e-6 * max(1.0, abs(red.item()))


@pytest.mark.parametrize("U,durs", [(63, [2, 8]), (64, [2, 8]), (127, [3]), (128, [3]), (255, [2, 16]),
                                    (256, [2, 15]), (511, [4]), (512, [7]), (700, [2, 6]), (1023, [2, 7])])
def test_multiblank_lattice_widths(rl, U, durs):
    # U+1 across every column width of the sweep (64, 128, 256, 512, 1024 columns) and ring depths up to the
    # 64 KiB limit: R * columns * 8 bytes, R the power of two above the longest duration
    ids = [7, 6][:len(durs)]
    w = _mb([3, 30], [U, min(U, 20)], 9, ids, durs, 0.05, std=1.0, blank=0, reduction="none", seed=U)
    loss, red, grad, flags = run_mb(rl, w)
    assert flags == 0
    check_mb(w, loss, grad, "none")


def test_multiblank_without_big_blanks(rl):
    """No big blank and sigma = 0: the plain loss and gradient; sigma alone shifts each loss by sigma (T+U)."""
    w = _mb([30, 17, 8], [7, 5, 0], 40, [], [], 0.0, std=2.0, blank=-1, reduction="none", seed=3)
    loss, _, grad, flags = run_mb(rl, w)
    assert flags == 0
    check_mb(w, loss, grad, "none")
    tg = torch.from_numpy(w.targets).to("cuda")
    ploss, _, pgrad, _ = rl.rnnt_loss_fused(w.logits, tg, w.logit_lengths, w.target_lengths, blank=-1,
                                            reduction="none")
    torch.cuda.synchronize()
    assert torch.allclose(loss, ploss, rtol=2e-6, atol=0)
    assert (grad - pgrad).abs().max().item() <= 2e-6
    w.sigma = 0.4
    sloss, _, sgrad, _ = run_mb(rl, w)
    shift = torch.tensor([0.4 * float(T + U) for T, U in zip(w.logit_lengths, w.target_lengths)],
                         dtype=torch.float32, device="cuda")
    assert torch.allclose(sloss, loss + shift, rtol=2e-6, atol=0)
    assert (sgrad - grad).abs().max().item() <= 2e-6


@pytest.mark.parametrize("reduction", ["none", "mean", "sum"])
def test_multiblank_autograd(rl, reduction):
    w = _mb([26, 19, 11], [6, 8, 3], 48, [45, 46], [2, 4], 0.1, std=2.0, blank=-1, reduction=reduction, seed=21)
    x = w.logits.clone().requires_grad_(True)
    tg = torch.from_numpy(w.targets).cuda()
    out = rl.rnnt_loss_multiblank(x, tg, torch.from_numpy(w.logit_lengths).cuda(),
                                  torch.from_numpy(w.target_lengths).cuda(), big_blank_ids=w.big_blank_ids,
                                  big_blank_durations=w.big_blank_durations,
                                  blank=-1, sigma=w.sigma, reduction=reduction)
    if reduction == "none":
        up = torch.tensor([0.5, 2.0, -1.0], device="cuda")
        (out * up).sum().backward()
        fac = np.repeat(up.cpu().numpy(), [w.rows(i).stop - w.rows(i).start for i in range(3)])[:, None]
    else:
        (out * 3.5).backward()
        fac = 3.5 / w.B if reduction == "mean" else 3.5
    _, red, gref, _ = oracle.multiblank_batch(x.detach().cpu().numpy(), w.targets, w.logit_lengths,
                                              w.target_lengths, w.big_blank_ids, w.big_blank_durations, blank=-1,
                                              sigma=w.sigma, reduction="none")
    err = np.abs(x.grad.double().cpu().numpy() - gref * fac).max()
    assert err <= 1e-5 * 3.5
    if reduction != "none":
        expect = red.sum() / (w.B if reduction == "mean" else 1)
        assert abs(out.item() - expect) <= 1e-5 * abs(expect)


@pytest.mark.parametrize("fused", [True, False])
def test_multiblank_bad_targets_are_flagged(rl, fused):
    """Labels equal to a big blank's class, to the standard blank or outside [0, V) are no symbols: those samples
    have no alignment (loss +inf, zero gradient) on both sides, the status word is flagged, and the other
    samples match the oracle."""
    w = _mb([8, 6, 7, 9], [3, 2, 3, 4], 12, [10, 9], [2, 3], 0.05, std=1.0, blank=-1, fused=fused,
            prenormalise=not fused, reduction="none", seed=8)
    tg = w.targets.copy()
    tg[0, 1] = 10         # a big blank's class
    tg[2, 0] = 11         # the standard blank
    tg[3, 3] = 12         # outside [0, V)
    w.targets = tg
    loss, red, grad, flags = run_mb(rl, w)
    assert flags & 2
    x = w.logits.float().cpu().numpy()
    for i in range(w.B):
        T, U = int(w.logit_lengths[i]), int(w.target_lengths[i])
        r = oracle.multiblank_sample(x[w.rows(i)], T, U, w.targets[i], w.V - 1, w.big_blank_ids,
                                     w.big_blank_durations, w.sigma, fused=fused, allow_bad_targets=True)
        g = grad[w.rows(i)].double().cpu().numpy()
        if i == 1:
            assert not r.bad_target
            assert abs(loss[i].item() - r.loss) <= 1e-5 * max(1.0, abs(r.loss))
            assert np.abs(g - r.grad).max() <= 1e-5
        else:
            assert r.bad_target and np.isinf(r.loss) and np.all(r.grad == 0)
            assert math.isinf(loss[i].item()) and loss[i].item() > 0 and np.all(g == 0), i


def test_multiblank_score_only_and_deterministic(rl):
    """grad = NULL: every loss against the oracle and bit for bit equal to the full call's; repeated calls
    are bitwise identical."""
    w = _mb([50, 31], [12, 7], 200, [198, 197], [2, 4], 0.05, std=2.0, blank=-1, reduction="sum", seed=4)
    a = run_mb(rl, w)
    b = run_mb(rl, w)
    c = run_mb(rl, w, compute_grad=False)
    assert torch.equal(a[0], b[0]) and torch.equal(a[2], b[2]) and torch.equal(a[0], c[0])
    assert c[2] is None
    check_mb(w, c[0], None, "sum")


def test_multiblank_workload_full_size(rl):
    """The multi-blank workload (bpe shapes, big blanks of 2, 4 and 8 frames, sigma 0.05): every loss, and
    every gradient row of the smallest and the largest sample; fused rows sum to zero."""
    w = workloads.make("multiblank", device="cuda")
    loss, red, grad, flags = run_mb(rl, w)
    assert flags == 0
    area = w.logit_lengths.astype(np.int64) * (w.target_lengths + 1)
    check_mb(w, loss, grad, w.reduction, grad_samples=[int(np.argmin(area)), int(np.argmax(area))])
    assert grad.double().sum(dim=1).abs().max().item() < 1e-6


def test_multiblank_extreme_fused_logits(rl):
    """Fused logits of spread N(0, 40^2): edge log-probabilities reach about -300, far outside fp32's exponent
    range, inside fp64's (the sweep works in fp64 probabilities).  The fp32 row steps work on x - max, so the
    fp32 gate holds: loss 1e-5 relative, gradient 1e-5."""
    w = _mb([25, 11, 7], [5, 4, 0], 64, [60, 61], [2, 3], 0.1, std=40.0, blank=-1, reduction="sum", seed=43)
    loss, red, grad, flags = run_mb(rl, w)
    assert flags == 0
    check_mb(w, loss, grad, "sum")


@pytest.mark.parametrize("offset", [100.0, 1000.0, "random"])
@pytest.mark.parametrize("V,dtype", [(1024, torch.float32), (50, torch.float32), (4096, torch.float16)])
def test_multiblank_fused_logit_offsets(rl, V, dtype, offset):
    """A constant added to each row's logits (100, 1000, or a per-row constant from [-1000, 1000]) leaves the
    multi-blank loss and gradient at the gates (log_softmax is shift-invariant)."""
    ids = [V - 2, V - 3, V - 4]
    w = _mb([40, 23, 31], [12, 7, 0], V, ids, [2, 4, 8], 0.05, dtype=dtype, std=2.0, blank=-1, reduction="mean",
            seed=V)
    if offset == "random":
        g = torch.Generator(device="cuda").manual_seed(V)
        c = torch.rand(w.N, 1, generator=g, device="cuda", dtype=torch.float64) * 2000.0 - 1000.0
    else:
        c = torch.full((w.N, 1), float(offset), device="cuda", dtype=torch.float64)
    w.logits = (w.logits.double() + c).to(dtype)
    loss, red, grad, flags = run_mb(rl, w)
    assert flags == 0
    check_mb(w, loss, grad, "mean")


def test_multiblank_very_long_lattices(rl):
    """T = 20000 frames with big blanks of 2 and 8 frames: ~20000 diagonal steps through the LDS ring, every loss
    and the whole gradient."""
    w = _mb([20000, 9000], [3, 0], 16, [14, 13], [2, 8], 0.05, std=1.0, blank=-1, reduction="none", seed=18)
    loss, red, grad, flags = run_mb(rl, w)
    assert flags == 0
    check_mb(w, loss, grad, "none")


def test_multiblank_wide_alpha_range(rl):
    """A big blank of 12 frames on a lattice with twice as many labels as frames (T=116, U=238): advancing in t
    is so cheap that on late anti-diagonals the nodes with more frames done lie ~e^745 above those with more labels
    done, which carry alignment mass because they finish cheaply.  The probability-domain sweep loses them; the
    label-count check catches it and the sample is rerun in the log domain.  Every loss and the whole gradient."""
    w = _mb([116, 8], [238, 119], 1024, [352], [12], 0.05, dtype=torch.float32, std=2.0, blank=675, clamp=-1.0,
            fused=True, prenormalise=False, reduction="mean", seed=3001)
    loss, red, grad, flags = run_mb(rl, w, fastemit=0.2)
    assert flags == 0
    check_mb(w, loss, grad, "mean", fastemit=0.2)


@pytest.mark.parametrize("gap", [15.0, 25.0])
def test_multiblank_peaked_blank(rl, gap):
    """The blank logit `gap` nats above every other class (labels and the big blanks alike): alpha falls by ~gap
    per label along an anti-diagonal, so the probability-domain sweep loses the nodes that carry the mass and the
    sample is rerun in the log domain.  Every loss and the whole gradient."""
    w = _mb([300, 60], [100, 50], 8, [7, 6], [4, 8], 0.0, std=1.0, blank=0, reduction="none", seed=int(gap))
    x = np.zeros(tuple(w.logits.shape), np.float32)
    x[:, 0] = gap
    w.logits = torch.from_numpy(x).to("cuda")
    loss, red, grad, flags = run_mb(rl, w)
    assert flags == 0
    check_mb(w, loss, grad, "none")


def test_multiblank_cheap_big_blank_expensive_blank(rl):
    """Logits of 0 for a 16-frame big blank, -80 for the standard blank, small for the labels: with five labels, ten
    of every sixteen diagonals are reached only through standard blanks, so the diagonal where the next big blank
    lands sits ~e^800 above the one before it, past fp64's range in the probability-domain sweep; the check sends
    the sample to the log domain.  Every loss and the whole gradient."""
    w = _mb([100, 33], [5, 3], 12, [11], [16], 0.0, std=1.0, blank=0, reduction="none", seed=77)
    rng = np.random.default_rng(77)
    x = (0.5 * rng.standard_normal(tuple(w.logits.shape))).astype(np.float32)
    x[:, 0] = -80.0
    x[:, 11] = 0.0
    w.logits = torch.from_numpy(x).to("cuda")
    loss, red, grad, flags = run_mb(rl, w)
    assert flags == 0
    check_mb(w, loss, grad, "none")


@pytest.mark.parametrize("fused,frac", [(True, 0.3), (False, 0.7)])
def test_multiblank_masked_vocabulary(rl, fused, frac):
    """-inf logits (or log-probs) on a random share of the classes other than the standard blank, big blanks
    included: exactly impossible edges, and samples with no possible alignment (loss +inf, zero gradient)."""
    Ts, Us, V = [40, 25, 60, 9], [30, 12, 45, 0], 29
    ids, durs = [28, 27], [2, 5]
    w = _mb(Ts, Us, V, ids, durs, 0.0, std=2.0 if fused else 1.5, blank=0, fused=fused, prenormalise=not fused,
            reduction="none", seed=int(frac * 100))
    rng = np.random.default_rng(int(frac * 100) + 1)
    x = w.logits.float().cpu().numpy()
    m = rng.random(x.shape) < frac
    m[:, 0] = False
    x[m] = -np.inf
    w.logits = torch.from_numpy(x).to("cuda")
    loss, red, grad, flags = run_mb(rl, w, fastemit=0.1)
    for i in range(w.B):
        T, U = int(w.logit_lengths[i]), int(w.target_lengths[i])
        r = oracle.multiblank_sample(x[w.rows(i)], T, U, w.targets[i], 0, ids, durs, 0.0, fused, -1.0, 0.1,
                                     want_grad=True)
        g = grad[w.rows(i)].detach().double().cpu().numpy()
        lg = float(loss[i].item())
        if np.isinf(r.loss):
            assert np.isinf(lg) and lg > 0 and np.all(g == 0), f"sample {i}"
        else:
            assert abs(lg - r.loss) <= 1e-5 * max(1.0, abs(r.loss)), f"sample {i}: loss {lg} vs oracle {r.loss}"
            assert np.isfinite(g).all() and np.abs(g - r.grad).max() <= 1e-5, f"sample {i}: gradient"


@pytest.mark.parametrize("seed", range(2000, 2016))
def test_multiblank_random_option_sweep(rl, seed):
    """Seeded draws over the multi-blank option space: batch shape, vocabulary, dtype, fused or not, the big
    blanks (count, classes, durations), sigma, clamp, FastEmit and reduction."""
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 10))
    V = int(rng.choice([8, 16, 33, 64, 200, 1024]))
    nb = int(rng.integers(0, 5))
    blank = int(rng.integers(-V, V))
    bn = blank + V if blank < 0 else blank
    ids = [int(k) for k in rng.choice([k for k in range(V) if k != bn], size=nb, replace=False)]
    durs = [int(d) for d in rng.integers(1, 17, size=nb)]
    Ts = rng.integers(1, 60, size=B).tolist()
    Us = rng.integers(0, 25, size=B).tolist()
    fused = bool(rng.random() < 0.7)
    dtype = torch.float16 if rng.random() < 0.3 else torch.float32
    reduction = str(rng.choice(["none", "mean", "sum"]))
    clamp = float(rng.choice([-1.0, -1.0, 0.1]))
    lam = float(rng.choice([0.0, 0.0, 0.2]))
    sigma = float(rng.choice([0.0, 0.05, -0.1]))
    w = _mb(Ts, Us, V, ids, durs, sigma, dtype=dtype, std=2.0 if fused else 1.5, blank=blank, clamp=clamp,
            fused=fused, prenormalise=not fused, reduction=reduction, seed=seed)
    loss, red, grad, flags = run_mb(rl, w, fastemit=lam)
    assert flags == 0
    check_mb(w, loss, grad, reduction, fastemit=lam)


def _padded(w, max_T, max_U1, fill=float("nan")):
    x = torch.full((w.B, max_T, max_U1, w.V), fill, dtype=w.logits.dtype, device=w.logits.device)
    for i in range(w.B):
        T, U = int(w.logit_lengths[i]), int(w.target_lengths[i])
        x[i, :T, :U + 1] = w.logits[w.rows(i)].reshape(T, U + 1, w.V)
    return x


def _unpad(w, g, max_T, max_U1):
    valid = torch.zeros((w.B, max_T, max_U1), dtype=torch.bool, device=g.device)
    parts = []
    for i in range(w.B):
        T, U = int(w.logit_lengths[i]), int(w.target_lengths[i])
        valid[i, :T, :U + 1] = True
        parts.append(g[i, :T, :U + 1].reshape(-1, w.V))
    return torch.cat(parts), g[~valid]


@pytest.mark.parametrize("V,dtype,fused", [(64, torch.float32, True), (33, torch.float32, True),
                                           (256, torch.float16, False)])
def test_multiblank_padded_matches_packed(rl, V, dtype, fused):
    # padded (B, max_T, max_U+1, V) logits (NaN padding, never used): the packed call's losses and, row for row,
    # its gradient bits; the padding rows get a zero gradient
    Ts, Us = [30, 12, 1, 19], [6, 0, 4, 9]
    w = _mb(Ts, Us, V, [V - 2, V - 3], [2, 5], 0.05, dtype=dtype, std=2.0 if fused else 1.5, blank=-1, fused=fused,
            prenormalise=not fused, reduction="sum", seed=V + 7)
    max_T, max_U1 = max(Ts) + 2, max(Us) + 3
    xp = _padded(w, max_T, max_U1)
    tg = torch.from_numpy(w.targets).to("cuda")
    loss_p, red_p, grad_p, ws = rl.rnnt_multiblank_fused(xp, tg, w.logit_lengths, w.target_lengths,
                                                         big_blank_ids=w.big_blank_ids,
                                                         big_blank_durations=w.big_blank_durations, blank=w.blank, sigma=w.sigma,
                                                         reduction="sum", fused_log_softmax=fused)
    assert rl.device_flags(ws) == 0
    loss, red, grad, _ = run_mb(rl, w)
    torch.cuda.synchronize()
    assert torch.equal(loss_p, loss) and torch.equal(red_p, red)
    rows, pad = _unpad(w, grad_p, max_T, max_U1)
    assert torch.equal(rows, grad)
    assert pad.numel() > 0 and bool((pad == 0).all())
    check_mb(w, loss, grad, "sum")


def test_multiblank_padded_autograd(rl):
    Ts, Us = [22, 9, 15], [5, 2, 7]
    w = _mb(Ts, Us, 48, [45, 46], [3, 2], 0.1, std=2.0, blank=-1, reduction="none", seed=47)
    tg = torch.from_numpy(w.targets).to("cuda")
    xp = _padded(w, 24, 9, fill=0.0)
    ref_loss, _, ref_grad, _ = rl.rnnt_multiblank_fused(xp, tg, w.logit_lengths, w.target_lengths,
                                                        big_blank_ids=w.big_blank_ids,
                                                        big_blank_durations=w.big_blank_durations, blank=-1, sigma=w.sigma,
                                                        reduction="none")
    x = xp.clone().requires_grad_(True)
    out = rl.rnnt_loss_multiblank(x, tg, w.logit_lengths, w.target_lengths, big_blank_ids=w.big_blank_ids,
                                  big_blank_durations=w.big_blank_durations,
                                  blank=-1, sigma=w.sigma, reduction="none")
    up = torch.tensor([0.5, -2.0, 3.0], device="cuda")
    out.backward(up)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), ref_loss)
    assert torch.allclose(x.grad, ref_grad * up.view(-1, 1, 1, 1), rtol=1e-6, atol=0)


@pytest.mark.parametrize("V,dtype,fused", [(1029, torch.float32, True), (2053, torch.float16, True),
                                           (1029, torch.float32, False), (1537, torch.float16, True)])
def test_multiblank_rows_off_16_byte_boundaries(rl, V, dtype, fused):
    """Row lengths that are no multiple of 16 bytes (1024 labels, the blank and four big blanks: 1029 classes):
    the vector row passes read each row in the 16-byte vectors that cover it and store the row's first and last
    vectors element by element.  Packed against the oracle (every loss and gradient row), the padded layout
    against the oracle with zero padding, and logits and gradient at matching and at different offsets from a
    16-byte boundary (the latter on the scalar kernels) against the oracle."""
    Ts, Us = [14, 9, 21], [6, 0, 11]
    ids = [V - 2, V - 3, V - 4, V - 5]
    w = _mb(Ts, Us, V, ids, [2, 3, 5, 8], 0.05, dtype=dtype, std=2.0 if fused else 1.5, blank=-1, fused=fused,
            prenormalise=not fused, reduction="sum", seed=V + 11)
    loss, red, grad, flags = run_mb(rl, w)
    assert flags == 0
    check_mb(w, loss, grad, "sum")
    tg = torch.from_numpy(w.targets).to("cuda")
    max_T, max_U1 = max(Ts) + 1, max(Us) + 1
    xp = _padded(w, max_T, max_U1, fill=0.0)
    loss_p, _, grad_p, _ = rl.rnnt_multiblank_fused(xp, tg, w.logit_lengths, w.target_lengths,
                                                    big_blank_ids=w.big_blank_ids,
                                                    big_blank_durations=w.big_blank_durations, blank=w.blank,
                                                    sigma=w.sigma, reduction="sum", fused_log_softmax=fused)
    torch.cuda.synchronize()
    rows, pad = _unpad(w, grad_p, max_T, max_U1)
    assert pad.numel() > 0 and bool((pad == 0).all())
    check_mb(w, loss_p, rows, "sum")
    n = w.logits.numel()
    for xo, go in ((1, 1), (1, 2)):
        xs = torch.empty(n + 16, dtype=dtype, device="cuda")
        gs = torch.empty(n + 16, dtype=dtype, device="cuda")
        x = xs[xo:xo + n].view(w.N, w.V)
        x.copy_(w.logits)
        g = gs[go:go + n].view(w.N, w.V)
        loss1, _, grad1, _ = rl.rnnt_multiblank_fused(x, tg, w.logit_lengths, w.target_lengths,
                                                      big_blank_ids=w.big_blank_ids,
                                                      big_blank_durations=w.big_blank_durations, blank=w.blank,
                                                      sigma=w.sigma, reduction="sum", fused_log_softmax=fused,
                                                      grad=g)
        torch.cuda.synchronize()
        assert grad1.data_ptr() == g.data_ptr()
        check_mb(w, loss1, grad1, "sum")
