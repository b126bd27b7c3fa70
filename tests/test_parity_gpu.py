"""GPU parity of librnnt against the fp64 oracle (run on an MI355X).

Every case draws seeded inputs with ``workloads``, runs the HIP path through
the C ABI (via the ctypes binding) and compares element by element with the
oracle on the same inputs:

    fp32 inputs: loss relative error <= 1e-5, gradient absolute error <= 1e-5
    fp16 inputs: loss relative error <= 2e-3, gradient absolute error <= 3e-3
                 (the oracle reads the fp16-rounded inputs exactly)

The per-sample gradient (the library's output divided by the reduction scale)
is held to the gate, which is stricter than comparing the scaled output.
At the full workload sizes the oracle computes every sample's loss and the
gradient of selected rows (the first and last rows of every sample, and
random rows); properties that hold at any size are checked on the whole
output.
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


def _blank(w):
    return w.blank + w.V if w.blank < 0 else w.blank


def _np_rows(t: torch.Tensor) -> np.ndarray:
    a = t.detach().cpu()
    if a.dtype == torch.float16:
        return a.numpy()
    return a.numpy()


def run(rl, w, reduction=None, inplace=False, compute_grad=True, clamp=None, fastemit=0.0):
    reduction = w.reduction if reduction is None else reduction
    clamp = w.clamp if clamp is None else clamp
    logits = w.logits.clone() if inplace else w.logits
    tg = torch.from_numpy(w.targets).to("cuda")
    loss, red, grad, ws = rl.rnnt_loss_fused(logits, tg, w.logit_lengths, w.target_lengths, blank=w.blank,
                                             clamp=clamp, reduction=reduction, fused_log_softmax=w.fused,
                                             compute_grad=compute_grad, inplace=inplace, fastemit_lambda=fastemit)
    flags = rl.device_flags(ws)
    torch.cuda.synchronize()
    return loss, red, grad, flags


def check_against_oracle(w, loss, grad, reduction, clamp=None, grad_rows="all", samples=None, seed=0,
                         fastemit=0.0):
    """Compare per-sample loss (all samples) and gradients of selected rows with the oracle."""
    clamp = w.clamp if clamp is None else clamp
    ltol, gtol = TOL[w.dtype]
    B = w.B
    b = _blank(w)
    scale = 1.0 / B if reduction == "mean" else 1.0
    loss_h = loss.detach().cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(seed)
    samples = range(B) if samples is None else samples
    want_grad = set(samples) if grad is not None else set()

    def one(i):
        sl = w.rows(i)
        x = _np_rows(w.logits[sl])
        T, U = int(w.logit_lengths[i]), int(w.target_lengths[i])
        n = T * (U + 1)
        rows = None
        if i in want_grad and grad_rows != "all":
            pick = set([0, 1, U, n - 1, n - 2, max(0, n - U - 1)])
            pick |= set(rng.integers(0, n, size=min(n, grad_rows)).tolist())
            rows = np.array(sorted(r for r in pick if 0 <= r < n), np.int64)
        r = oracle.sample(x, T, U, w.targets[i], b, w.fused, clamp, want_grad=(i in want_grad), rows=rows,
                          fastemit_lambda=fastemit)
        return i, r, rows

    errs_loss, errs_grad = [], []
    with cf.ThreadPoolExecutor(_threads()) as ex:
        for i, r, rows in ex.map(one, range(B)):
            ref = r.loss
            rel = abs(loss_h[i] - ref) / max(1.0, abs(ref))
            errs_loss.append(rel)
            assert rel <= ltol, f"sample {i}: loss {loss_h[i]} vs oracle {ref} (rel {rel:.3g})"
            assert abs(r.loss_alpha - r.loss) <= 1e-9 * max(1.0, abs(r.loss))
            if r.grad is not None:
                sl = w.rows(i)
                g = grad[sl] if rows is None else grad[sl][torch.from_numpy(rows).to(grad.device)]
                g = g.detach().double().cpu().numpy() / scale
                err = np.abs(g - r.grad).max()
                errs_grad.append(err)
                assert err <= gtol, f"sample {i}: grad max abs err {err:.3g}"
    return max(errs_loss), (max(errs_grad) if errs_grad else 0.0)


def _reduced_ok(w, loss, red, reduction):
    if reduction == "none":
        assert red is None
        return
    s = loss.double().sum().item()
    expect = s / w.B if reduction == "mean" else s
    assert abs(red.item() - expect) <= 1e-6 * max(1.0, abs(expect))


# ------------------------------------------------------------- named workloads
@pytest.mark.parametrize("reduction", ["none", "mean", "sum"])
def test_tiny_workload(rl, reduction):
    w = workloads.make("tiny", device="cuda")
    assert w.N == 96 and w.logits.shape == (96, 16)
    loss, red, grad, flags = run(rl, w, reduction=reduction)
    assert flags == 0
    check_against_oracle(w, loss, grad, reduction)
    _reduced_ok(w, loss, red, reduction)


@pytest.mark.parametrize("seed", [2, 101, 102, 103])
def test_char_workload(rl, seed):
    w = workloads.make("char", seed=seed, device="cuda")
    loss, red, grad, flags = run(rl, w)
    assert flags == 0
    check_against_oracle(w, loss, grad, w.reduction)
    _reduced_ok(w, loss, red, w.reduction)


def test_bpe_workload_full_size(rl):
    w = workloads.make("bpe", device="cuda")
    loss, red, grad, flags = run(rl, w)
    assert flags == 0
    order = np.argsort(w.logit_lengths.astype(np.int64) * (w.target_lengths + 1))
    picks = [int(order[0]), int(order[-1]), int(order[len(order) // 2])]
    check_against_oracle(w, loss, grad, w.reduction, grad_rows="all", samples=picks)
    _reduced_ok(w, loss, red, w.reduction)
    # any-size property: each fused gradient row sums to zero (fp32 rounding only)
    rs = grad.double().sum(dim=1).abs().max().item()
    assert rs < 1e-6


def test_half_workload_full_size(rl):
    """The fp16 workload at full size (16 samples, V = 4096): every loss, and in every sample the gradient of
    rows (0,0), (0,1), (0,U), (T-1,U), the two rows before it and 200 random rows."""
    w = workloads.make("half", device="cuda")
    loss, red, grad, flags = run(rl, w)
    assert flags == 0
    check_against_oracle(w, loss, grad, w.reduction, grad_rows=200)
    _reduced_ok(w, loss, red, w.reduction)
    assert torch.isfinite(grad).all()


def test_skewed_workload_full_size(rl):
    """The skewed log-prob workload at full size (64 samples): every loss, and in every sample the gradient of
    the corner rows and 200 random rows."""
    w = workloads.make("skewed", device="cuda")
    loss, red, grad, flags = run(rl, w)
    assert flags == 0
    order = np.argsort(w.logit_lengths.astype(np.int64) * (w.target_lengths + 1))
    check_against_oracle(w, loss, grad, w.reduction, grad_rows=200)
    _reduced_ok(w, loss, red, w.reduction)
    # non-fused: at most two non-zeros per row; per sample the entries sum to -(T+U)
    nnz = (grad != 0).sum(dim=1)
    assert int(nnz.max().item()) <= 2
    big = int(order[-1])
    s = grad[w.rows(big)].double().sum().item()
    T, U = int(w.logit_lengths[big]), int(w.target_lengths[big])
    assert abs(s + (T + U)) <= 3e-3 * (T + U)


# ------------------------------------------------------------------ edge cases
def _custom(Ts, Us, V, **kw):
    return workloads.make_custom(Ts, Us, V, device="cuda", **kw)


def _to_padded(w, max_T, max_U1, fill=float("nan")):
    """The packed logits of w scattered into a (B, max_T, max_U1, V) tensor; padding holds `fill`."""
    x = torch.full((w.B, max_T, max_U1, w.V), fill, dtype=w.logits.dtype, device=w.logits.device)
    for i in range(w.B):
        T, U = int(w.logit_lengths[i]), int(w.target_lengths[i])
        x[i, :T, :U + 1] = w.logits[w.rows(i)].reshape(T, U + 1, w.V)
    return x


def _padded_rows(w, g, max_T, max_U1):
    """(valid rows of a padded gradient in packed order, its padding entries)."""
    valid = torch.zeros((w.B, max_T, max_U1), dtype=torch.bool, device=g.device)
    parts = []
    for i in range(w.B):
        T, U = int(w.logit_lengths[i]), int(w.target_lengths[i])
        valid[i, :T, :U + 1] = True
        parts.append(g[i, :T, :U + 1].reshape(-1, w.V))
    return torch.cat(parts), g[~valid]


@pytest.mark.parametrize("V,dtype,fused", [(300, torch.float32, True), (29, torch.float32, True),
                                           (512, torch.float16, True), (256, torch.float16, False)])
@pytest.mark.parametrize("size", ["small", "large"])
def test_padded_layout_matches_packed(rl, V, dtype, fused, size):
    # padded (B, max_T, max_U+1, V) input: same losses and, row for row, the
    # same gradient bits as the packed call on the same values; the padding
    # (NaN here, never used) gets a zero gradient.  "large": above the
    # 64512-row line below which a batch takes three launches
    Ts, Us = ([40, 17, 33, 1, 25], [9, 0, 14, 6, 3]) if size == "small" else \
        ([500, 170, 330, 1, 250], [90, 0, 44, 6, 30])
    assert (sum(t * (u + 1) for t, u in zip(Ts, Us)) < 64512) == (size == "small")
    w = workloads.make_custom(Ts, Us, V, dtype=dtype, std=2.0 if fused else 1.5, fused=fused, reduction="sum",
                              seed=77, device="cuda", prenormalise=not fused)
    max_T, max_U1 = max(Ts) + 3, max(Us) + 4
    xp = _to_padded(w, max_T, max_U1)
    tg = torch.from_numpy(w.targets).to("cuda")
    loss_p, red_p, grad_p, ws = rl.rnnt_loss_fused(xp, tg, w.logit_lengths, w.target_lengths, blank=w.blank,
                                                   reduction="sum", fused_log_softmax=fused)
    assert rl.device_flags(ws) == 0
    loss, red, grad, _ = run(rl, w)
    torch.cuda.synchronize()
    assert torch.equal(loss_p, loss) and torch.equal(red_p, red)
    rows, pad = _padded_rows(w, grad_p, max_T, max_U1)
    assert torch.equal(rows, grad)
    assert pad.numel() > 0 and bool((pad == 0).all())
    check_against_oracle(w, loss, grad, "sum", grad_rows=("all" if fused else 64) if size == "small" else 300)


@pytest.mark.parametrize("V,dtype,fused", [(1000, torch.float32, True), (2504, torch.float16, True),
                                           (1000, torch.float32, False)])
def test_padded_rows_sharing_lines(rl, V, dtype, fused):
    """Rows whose boundaries fall inside 128-byte lines (4000- and 5008-byte rows), in the padded layout with
    max_U1 = max(U)+1: in the widest sample the time steps follow each other in memory, so its line shared by
    (t, U) and (t+1, 0) goes whole to the later row's wave, while the other samples' time steps end at padding.
    Bitwise equal to the packed call, the padding zero, in place equal to out of place, and the packed call
    against the oracle."""
    Ts, Us = [23, 9, 30, 1], [11, 4, 11, 0]
    w = workloads.make_custom(Ts, Us, V, dtype=dtype, std=2.0 if fused else 1.5, fused=fused, reduction="sum",
                              seed=83, device="cuda", prenormalise=not fused)
    max_T, max_U1 = max(Ts) + 2, max(Us) + 1
    xp = _to_padded(w, max_T, max_U1, fill=0.0)
    tg = torch.from_numpy(w.targets).to("cuda")
    loss_p, red_p, grad_p, ws = rl.rnnt_loss_fused(xp, tg, w.logit_lengths, w.target_lengths, blank=w.blank,
                                                   reduction="sum", fused_log_softmax=fused)
    assert rl.device_flags(ws) == 0
    loss, red, grad, _ = run(rl, w)
    y = xp.clone()
    loss_i, _, grad_i, _ = rl.rnnt_loss_fused(y, tg, w.logit_lengths, w.target_lengths, blank=w.blank,
                                              reduction="sum", fused_log_softmax=fused, inplace=True)
    torch.cuda.synchronize()
    assert torch.equal(loss_p, loss) and torch.equal(red_p, red)
    rows, pad = _padded_rows(w, grad_p, max_T, max_U1)
    assert torch.equal(rows, grad)
    assert pad.numel() > 0 and bool((pad == 0).all())
    assert grad_i.data_ptr() == y.data_ptr() and torch.equal(loss_i, loss_p) and torch.equal(y, grad_p)
    check_against_oracle(w, loss, grad, "sum", grad_rows="all")


def test_padded_inplace_and_autograd(rl):
    Ts, Us = [30, 12, 21], [7, 3, 10]
    w = workloads.make_custom(Ts, Us, 320, std=2.0, reduction="none", seed=78, device="cuda")
    max_T, max_U1 = 32, 12
    tg = torch.from_numpy(w.targets).to("cuda")
    xp = _to_padded(w, max_T, max_U1, fill=0.0)
    ref_loss, _, ref_grad, _ = rl.rnnt_loss_fused(xp, tg, w.logit_lengths, w.target_lengths, blank=w.blank,
                                                  reduction="none")
    y = xp.clone()
    loss_i, _, grad_i, _ = rl.rnnt_loss_fused(y, tg, w.logit_lengths, w.target_lengths, blank=w.blank,
                                              reduction="none", inplace=True)
    torch.cuda.synchronize()
    assert grad_i.data_ptr() == y.data_ptr()
    assert torch.equal(loss_i, ref_loss) and torch.equal(y, ref_grad)
    # autograd with a per-sample upstream gradient (reduction none)
    x = xp.clone().requires_grad_(True)
    out = rl.rnnt_loss(x, tg, w.logit_lengths, w.target_lengths, blank=w.blank, reduction="none")
    up = torch.tensor([0.5, -2.0, 3.0], device="cuda")
    out.backward(up)
    torch.cuda.synchronize()
    want = ref_grad * up.view(-1, 1, 1, 1).to(ref_grad.dtype)
    assert torch.allclose(x.grad, want, rtol=1e-6, atol=0)
    assert torch.equal(out.detach(), ref_loss)


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16])
def test_single_path_and_degenerate_lattices(rl, dtype):
    # U = 0 (all-blank lattice), T = 1 (single path), 1x1, and ordinary samples mixed
    w = _custom([7, 1, 1, 5, 33], [0, 6, 0, 3, 0], 19, dtype=dtype, std=2.0, blank=4, reduction="sum", seed=11)
    loss, red, grad, flags = run(rl, w)
    assert flags == 0
    check_against_oracle(w, loss, grad, "sum")


@pytest.mark.parametrize("V", [1, 2, 3, 5, 31, 64, 65, 100, 257, 1000, 1023, 2049, 5001])
def test_vocab_sizes(rl, V):
    # V = 1 only admits U = 0; odd V exercises the scalar (unvectorised) row path
    Us = [0, 0] if V == 1 else [3, min(9, 5)]
    w = _custom([6, 11], Us, V, std=1.5, blank=-1, reduction="mean", seed=V)
    loss, red, grad, flags = run(rl, w)
    assert flags == 0
    check_against_oracle(w, loss, grad, "mean")


@pytest.mark.parametrize("V,dtype,clamp", [(2048, torch.float32, -1.0), (4096, torch.float32, 0.5),
                                           (8192, torch.float16, -1.0), (3000, torch.float16, 0.05)])
def test_wide_rows_split_over_waves(rl, V, dtype, clamp):
    # rows of 8-16 KiB: the gradient pass splits each row over two or four waves (the flows land in
    # whichever part holds the blank / label), the row pass holds the whole row in one wave
    w = _custom([7, 5], [6, 9], V, dtype=dtype, std=2.0, blank=-1, clamp=clamp, reduction="mean", seed=V)
    loss, red, grad, flags = run(rl, w)
    assert flags == 0
    check_against_oracle(w, loss, grad, "mean")


@pytest.mark.parametrize("V,dtype,clamp,fused", [
    (1028, torch.float32, -1.0, True),    # 4112-byte rows: shared lines, one part of five vectors per lane
    (1088, torch.float32, 0.3, True),     # 4352-byte rows on line boundaries, clamp
    (2056, torch.float16, -1.0, True),    # fp16 rows of 4112 bytes
    (2112, torch.float16, -1.0, False),   # log-prob inputs, 4224-byte rows
    (1280, torch.float32, -1.0, False),   # 5120-byte rows: the part exactly full
])
def test_rows_of_4_to_5_kib(rl, V, dtype, clamp, fused):
    """Rows a little over 4 KiB: the row pass takes each in one step of five vectors per lane and the gradient
    in one wave of five vectors per lane (where four would leave a second, nearly empty part); every gradient
    row against the oracle."""
    w = _custom([9, 6], [7, 10], V, dtype=dtype, std=2.0 if fused else 1.5, blank=-1, clamp=clamp, fused=fused,
                prenormalise=not fused, reduction="mean", seed=V + 1)
    loss, red, grad, flags = run(rl, w)
    assert flags == 0
    check_against_oracle(w, loss, grad, "mean")


@pytest.mark.parametrize("V,dtype,clamp,fused", [
    (4104, torch.float16, -1.0, True),    # 8208-byte rows: the last block of 64 vectors joins the part before
    (2056, torch.float32, 0.3, True),     # 8224-byte fp32 rows, clamp
    (2049, torch.float32, -1.0, False),   # 8196-byte log-prob rows off 16-byte boundaries
    (6152, torch.float16, -1.0, True),    # 12304-byte rows: three parts, the last of five blocks
])
def test_rows_a_block_over_4_kib_parts(rl, V, dtype, clamp, fused):
    """Rows that would end in a part (gradient) or segment (row pass) of at most one block of 64 vectors: that
    block is taken as a fifth block of the part or segment before it.  Every gradient row against the oracle."""
    w = _custom([8, 5], [6, 9], V, dtype=dtype, std=2.0 if fused else 1.5, blank=-1, clamp=clamp, fused=fused,
                prenormalise=not fused, reduction="mean", seed=V + 2)
    loss, red, grad, flags = run(rl, w)
    assert flags == 0
    check_against_oracle(w, loss, grad, "mean")


@pytest.mark.parametrize("V,dtype,clamp,fused,size", [
    (1025, torch.float32, -1.0, True, "small"),   # 4100-byte rows: a BPE vocabulary of 1024 and the blank
    (1025, torch.float32, -1.0, True, "large"),
    (2049, torch.float16, -1.0, True, "small"),   # fp16, 4098-byte rows
    (4097, torch.float16, 0.5, True, "large"),    # 8194-byte rows, clamp
    (5001, torch.float32, -1.0, True, "small"),   # 20004-byte rows over five parts
    (257, torch.float32, -1.0, True, "small"),    # 1028-byte rows, just over the narrow kernels' 1 KiB
    (1537, torch.float32, -1.0, False, "small"),  # log-prob inputs, 6148-byte rows
    (3001, torch.float16, -1.0, False, "large"),
])
def test_rows_off_16_byte_boundaries(rl, V, dtype, clamp, fused, size):
    """Row lengths that are no multiple of 16 bytes: the row pass reads each row in the 16-byte vectors that cover
    it (slots outside the row masked), the gradient pass owns whole lines and computes the elements of two rows
    that meet inside a vector each with its own row's terms.  "large": above the 64512-row line below which a
    batch takes three launches.  Every loss, and every gradient row (small) or corner and random rows (large),
    against the oracle."""
    Ts, Us = ([9, 6, 1], [7, 10, 0]) if size == "small" else ([400, 300], [130, 100])
    assert (sum(t * (u + 1) for t, u in zip(Ts, Us)) < 64512) == (size == "small")
    w = _custom(Ts, Us, V, dtype=dtype, std=2.0 if fused else 1.5, blank=-1, clamp=clamp, fused=fused,
                prenormalise=not fused, reduction="sum", seed=V + 3)
    loss, red, grad, flags = run(rl, w)
    assert flags == 0
    check_against_oracle(w, loss, grad, "sum", grad_rows="all" if size == "small" else 300)


@pytest.mark.parametrize("V,dtype", [(1025, torch.float32), (2049, torch.float16)])
def test_odd_rows_padded_inplace_and_offsets(rl, V, dtype):
    """Rows off 16-byte boundaries in the padded layout (max_U1 = max(U)+1, so one sample's time steps are adjacent
    in memory; padding zero), in place (bitwise equal to out of place at the same addresses), and with logits and
    gradient one element past a 16-byte boundary (the same vectors) or at different offsets (the narrow gradient
    kernels): each against the oracle.  The row pass's lanes take a row's elements by their place in 16-byte
    blocks, so calls at other addresses agree to rounding, not bit for bit."""
    Ts, Us = [13, 7, 20], [9, 4, 9]
    w = _custom(Ts, Us, V, dtype=dtype, std=2.0, blank=-1, reduction="sum", seed=V + 5)
    tg = torch.from_numpy(w.targets).to("cuda")
    loss0, red0, grad0, flags = run(rl, w)
    assert flags == 0
    check_against_oracle(w, loss0, grad0, "sum")
    max_T, max_U1 = max(Ts) + 1, max(Us) + 1
    xp = _to_padded(w, max_T, max_U1, fill=0.0)
    loss_p, red_p, grad_p, _ = rl.rnnt_loss_fused(xp, tg, w.logit_lengths, w.target_lengths, blank=w.blank,
                                                  reduction="sum")
    y = xp.clone()
    loss_i, _, grad_i, _ = rl.rnnt_loss_fused(y, tg, w.logit_lengths, w.target_lengths, blank=w.blank,
                                              reduction="sum", inplace=True)
    torch.cuda.synchronize()
    rows, pad = _padded_rows(w, grad_p, max_T, max_U1)
    check_against_oracle(w, loss_p, rows, "sum")
    assert bool((pad == 0).all())
    assert grad_i.data_ptr() == y.data_ptr() and torch.equal(loss_i, loss_p) and torch.equal(y, grad_p)
    n = w.logits.numel()
    for xo, go in ((1, 1), (1, 3)):
        xs = torch.empty(n + 16, dtype=dtype, device="cuda")
        gs = torch.empty(n + 16, dtype=dtype, device="cuda")
        x = xs[xo:xo + n].view(w.N, w.V)
        x.copy_(w.logits)
        g = gs[go:go + n].view(w.N, w.V)
        loss1, red1, grad1, _ = rl.rnnt_loss_fused(x, tg, w.logit_lengths, w.target_lengths, blank=w.blank,
                                                   reduction="sum", grad=g)
        torch.cuda.synchronize()
        assert grad1.data_ptr() == g.data_ptr()
        check_against_oracle(w, loss1, grad1, "sum")


@pytest.mark.parametrize("V,dtype,clamp,fused,lam", [
    (5000, torch.float32, -1.0, True, 0.0),      # 20000-byte rows: five 4 KiB segments, the last partial
    (8192, torch.float32, 0.05, True, 0.3),      # 32 KiB rows, clamp, FastEmit
    (50000, torch.float32, -1.0, True, 0.0),     # 200 KB rows (the README's largest vocabulary)
    (16384, torch.float16, -1.0, True, 0.0),     # fp16 rows of 32 KiB
    (20000, torch.float16, 1.0, True, 0.1),
    (12000, torch.float32, -1.0, False, 0.2),    # log-prob inputs: flows only
])
def test_rows_wider_than_16k(rl, V, dtype, clamp, fused, lam):
    """Rows wider than the 16 KiB a wave holds in registers: the row pass streams each row in 4 KiB segments
    (running maximum and rescaled sum per lane), the gradient pass splits it over one wave per 4 KiB."""
    w = _custom([7, 5, 1], [6, 9, 3], V, dtype=dtype, std=2.0 if fused else 1.5, blank=-1, clamp=clamp,
                fused=fused, prenormalise=not fused, reduction="mean", seed=V % 1000)
    loss, red, grad, flags = run(rl, w, fastemit=lam)
    assert flags == 0
    check_against_oracle(w, loss, grad, "mean", fastemit=lam)
    if fused and clamp <= 0:  # unclamped fused rows sum to zero
        assert grad.double().sum(dim=1).abs().max().item() < (1e-6 if dtype == torch.float32 else 2e-2)


def test_vocab5k_workload_full_size(rl):
    """The vocab5k workload (4 samples, V = 5000: 20000-byte rows, the README's V = 5000 shape): every loss and,
    in every sample, the corner rows and 200 random rows of the gradient."""
    w = workloads.make("vocab5k", device="cuda")
    loss, red, grad, flags = run(rl, w)
    assert flags == 0
    check_against_oracle(w, loss, grad, w.reduction, grad_rows=200)
    _reduced_ok(w, loss, red, w.reduction)


@pytest.mark.parametrize("U", [0, 1, 62, 63, 64, 127, 128, 255, 256, 511, 512, 700, 767, 768, 1023, 1024, 1279,
                               1280, 1535, 1536, 1791, 1792, 2047])
def test_lattice_widths_across_register_tiles(rl, U):
    # U+1 crosses each width of the alpha/beta sweeps' lane tiles: 64 columns (one per lane), 128 (two per
    # lane), then groups of 256 (four per lane), up to eight groups
    w = _custom([3, 40], [U, min(U, 20)], 8, std=1.0, blank=0, reduction="none", seed=U)
    loss, red, grad, flags = run(rl, w)
    assert flags == 0
    check_against_oracle(w, loss, grad, "none")


@pytest.mark.parametrize("U", [512, 743, 744, 991, 992, 1023, 1500, 1983, 1984])
@pytest.mark.parametrize("domain", ["prob", "log"])
def test_wide_sweep_widths_in_a_large_batch(rl, U, domain):
    """Lattices of 513 to 1985 columns in a batch above 64 K rows, so the recursions run on the six-launch path:
    the one-wave tiles of two to four column groups up to 1024 columns, the multi-wave sweep above; in the
    probability domain and in the log domain (log-probs down to -200, as in
    test_log_domain_across_register_tiles)."""
    Ts, Us, V = [9, 300], [U, 250], 8
    log = domain == "log"
    w = _custom(Ts, Us, V, std=1.0, blank=0, fused=not log, prenormalise=log, reduction="none", seed=U + 7)
    if log:
        rng = np.random.default_rng(U)
        x = np.round(rng.uniform(-200.0, -0.25, size=(w.N, V)) * 4) / 4
        x[::5, 0] = -0.5
        w.logits = torch.tensor(x, dtype=torch.float32, device="cuda")
    assert w.N > 64512
    loss, red, grad, flags = run(rl, w)
    assert flags == 0
    check_against_oracle(w, loss, grad, "none", grad_rows=300)


@pytest.mark.parametrize("fused", [True, False])
def test_wide_lattices_in_a_large_batch(rl, fused):
    """Lattices of 2001 and 1501 columns (eight and six column groups per lane) in a batch above 64 K rows, so
    the recursions run on the six-launch path; with log-prob inputs, mildly peaked, for the probability domain."""
    w = _custom([40, 44, 30], [2000, 1500, 700], 8, std=1.0, blank=0, fused=fused, prenormalise=not fused,
                reduction="mean", seed=71)
    assert w.N > 64 * 1024
    loss, red, grad, flags = run(rl, w)
    assert flags == 0
    check_against_oracle(w, loss, grad, "mean", grad_rows=300)
    _reduced_ok(w, loss, red, "mean")


def test_wide_lattices_with_options(rl):
    """A 1700-column lattice (the multi-wave recursion) in fp16 with clamp and FastEmit, against the oracle; the
    same batch in the padded layout bitwise equal to it, and score-only returning the same losses."""
    w = _custom([30, 12, 25], [1699, 400, 1300], 24, dtype=torch.float16, std=2.0, blank=-1, clamp=0.3,
                reduction="sum", seed=73)
    assert w.N > 64 * 1024 or max(w.target_lengths) + 1 > 1024
    loss, red, grad, flags = run(rl, w, fastemit=0.02)
    assert flags == 0
    check_against_oracle(w, loss, grad, "sum", grad_rows=300, fastemit=0.02)
    _reduced_ok(w, loss, red, "sum")
    max_T, max_U1 = max(w.logit_lengths) + 1, max(w.target_lengths) + 2
    xp = _to_padded(w, max_T, max_U1)
    tg = torch.from_numpy(w.targets).to("cuda")
    lp_, _, gp_, _ = rl.rnnt_loss_fused(xp, tg, w.logit_lengths, w.target_lengths, blank=w.blank, clamp=0.3,
                                        reduction="sum", fused_log_softmax=True, fastemit_lambda=0.02)
    torch.cuda.synchronize()
    rows, pad = _padded_rows(w, gp_, max_T, max_U1)
    assert torch.equal(lp_, loss) and torch.equal(rows, grad) and bool((pad == 0).all())
    ls, _, _, _ = rl.rnnt_loss_fused(w.logits, tg, w.logit_lengths, w.target_lengths, blank=w.blank, clamp=0.3,
                                     reduction="sum", fused_log_softmax=True, compute_grad=False,
                                     fastemit_lambda=0.02)
    torch.cuda.synchronize()
    assert torch.equal(ls, loss)


def test_ragged_batch_many_samples(rl):
    rng = np.random.default_rng(77)
    B = 150
    Ts = rng.integers(1, 90, size=B).tolist()
    Us = rng.integers(0, 40, size=B).tolist()
    w = _custom(Ts, Us, 40, std=2.0, blank=-40, reduction="mean", seed=77)
    loss, red, grad, flags = run(rl, w)
    assert flags == 0
    check_against_oracle(w, loss, grad, "mean")


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16])
@pytest.mark.parametrize("clamp", [0.02, 0.1, 0.3])
def test_clamp(rl, dtype, clamp):
    w = _custom([30, 17], [8, 5], 12, dtype=dtype, std=3.0, blank=-1, reduction="mean", seed=5)
    loss, red, grad, flags = run(rl, w, clamp=clamp)
    check_against_oracle(w, loss, grad, "mean", clamp=clamp)
    assert grad.abs().max().item() <= clamp / w.B * (1 + 1e-3)


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16])
def test_nonfused_inputs(rl, dtype):
    w = _custom([25, 40, 9], [6, 12, 0], 50, dtype=dtype, std=1.5, blank=0, fused=False, prenormalise=True,
                reduction="sum", seed=9)
    loss, red, grad, flags = run(rl, w)
    check_against_oracle(w, loss, grad, "sum")


def test_inplace_gradient_over_logits(rl):
    w = _custom([40, 20], [10, 7], 256, std=2.0, blank=-1, reduction="none", seed=3)
    ref_loss, _, ref_grad, _ = run(rl, w)
    loss, _, grad, _ = run(rl, w, inplace=True)
    assert torch.equal(loss, ref_loss)
    assert torch.equal(grad, ref_grad)


@pytest.mark.parametrize("V,dtype,fused", [(64, torch.float32, True), (1024, torch.float32, True),
                                           (29, torch.float32, True), (2048, torch.float16, False)])
@pytest.mark.parametrize("size", ["small", "large"])
def test_score_only(rl, V, dtype, fused, size):
    """grad = NULL (the GPURNNT page's score_forward: costs without gradients): every loss against the oracle,
    and bit for bit equal to the loss of the full call; on both sides of the 64512-row line."""
    Ts, Us = ([40, 20, 33], [10, 7, 0]) if size == "small" else ([500, 200, 330], [100, 70, 0])
    assert (sum(t * (u + 1) for t, u in zip(Ts, Us)) < 64512) == (size == "small")
    w = _custom(Ts, Us, V, dtype=dtype, std=2.0 if fused else 1.5, blank=-1, fused=fused,
                prenormalise=not fused, reduction="sum", seed=4)
    loss, red, grad, flags = run(rl, w, compute_grad=False)
    assert grad is None and flags == 0
    check_against_oracle(w, loss, None, "sum")
    _reduced_ok(w, loss, red, "sum")
    ref, _, _, _ = run(rl, w)
    assert torch.equal(loss, ref)


def test_unaligned_logits_pointer(rl):
    # logits starting 4 bytes past a 16-byte boundary force the scalar access path
    w = _custom([20, 13], [5, 9], 32, std=2.0, blank=3, reduction="mean", seed=6)
    buf = torch.empty(w.logits.numel() + 1, dtype=w.logits.dtype, device="cuda")
    buf[1:].copy_(w.logits.reshape(-1))
    w.logits = buf[1:].view(w.N, w.V)
    assert w.logits.data_ptr() % 16 != 0
    loss, red, grad, flags = run(rl, w)
    check_against_oracle(w, loss, grad, "mean")


@pytest.mark.parametrize("V,dtype,fused", [(1024, torch.float32, True), (2048, torch.float16, False),
                                           (5000, torch.float32, True), (300, torch.float32, True),
                                           (2504, torch.float16, True), (1000, torch.float32, False)])
def test_rows_off_128_byte_lines(rl, V, dtype, fused):
    """Logits and gradient 16 bytes past a 128-byte boundary: every row starts inside a line, so the gradient
    pass gives each line shared by two adjacent rows to the later row's wave, which computes the earlier row's
    last vectors too (as it does for 20000- and 1200-byte rows anywhere); with 4 KiB rows that takes a second,
    nearly empty part per row.  The row pass reads the same rows in the same lane order, and the gradient is
    elementwise, so everything is bitwise equal to the aligned call; the aligned call is checked against the
    oracle."""
    w = _custom([37, 22], [9, 14], V, dtype=dtype, std=2.0 if fused else 1.5, blank=-1, fused=fused,
                prenormalise=not fused, reduction="sum", seed=61)
    tg = torch.from_numpy(w.targets).to("cuda")
    shift = 16 // w.logits.element_size()
    xs = torch.empty(w.logits.numel() + 64, dtype=w.logits.dtype, device="cuda")
    gs = torch.empty_like(xs)
    assert xs.data_ptr() % 128 == 0 and gs.data_ptr() % 128 == 0
    x = xs[shift:shift + w.logits.numel()].view(w.N, w.V)
    x.copy_(w.logits)
    g = gs[shift:shift + w.logits.numel()].view(w.N, w.V)
    loss0, red0, grad0, flags = run(rl, w)
    assert flags == 0
    check_against_oracle(w, loss0, grad0, "sum", grad_rows=64)
    loss1, red1, grad1, _ = rl.rnnt_loss_fused(x, tg, w.logit_lengths, w.target_lengths, blank=w.blank,
                                               reduction="sum", fused_log_softmax=fused, grad=g)
    torch.cuda.synchronize()
    assert grad1.data_ptr() == g.data_ptr()
    assert torch.equal(loss1, loss0) and torch.equal(red1, red0) and torch.equal(grad1, grad0)


def test_deterministic_bitwise(rl):
    w = workloads.make("char", seed=7, device="cuda")
    a = run(rl, w)
    b = run(rl, w)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])


@pytest.mark.parametrize("fused", [True, False])
def test_bad_targets_are_flagged(rl, fused):
    """A label equal to blank or outside [0, V) is no symbol an alignment can emit (the build post's section 5.2
    rules blank out of the labels): that sample has no alignment, loss +inf and a zero gradient, on both sides;
    the status word is flagged and the other samples are unaffected."""
    w = _custom([6, 5, 9], [3, 2, 4], 10, std=1.0, blank=-1, fused=fused, prenormalise=not fused,
                reduction="none", seed=8)
    tg = w.targets.copy()
    tg[0, 1] = 9          # equals blank (V-1)
    tg[1, 0] = 12         # outside [0, V)
    w.targets = tg
    loss, red, grad, flags = run(rl, w)
    assert flags & 2
    x = w.logits.float().cpu().numpy()

    def ref(i):
        T, U = int(w.logit_lengths[i]), int(w.target_lengths[i])
        return oracle.sample(x[w.rows(i)], T, U, w.targets[i], 9, fused, -1.0, allow_bad_targets=True)
    check_masked(w, loss, grad, ref)
    assert math.isinf(loss[0].item()) and math.isinf(loss[1].item()) and math.isfinite(loss[2].item())


# ------------------------------------------------------------------- autograd
@pytest.mark.parametrize("reduction", ["none", "mean", "sum"])
def test_autograd_backward(rl, reduction):
    w = _custom([30, 22, 15], [7, 4, 9], 48, std=2.0, blank=-1, reduction=reduction, seed=21)
    x = w.logits.clone().requires_grad_(True)
    tg = torch.from_numpy(w.targets).cuda()
    Tl = torch.from_numpy(w.logit_lengths).cuda()
    Ul = torch.from_numpy(w.target_lengths).cuda()
    out = rl.rnnt_loss(x, tg, Tl, Ul, blank=-1, reduction=reduction)
    if reduction == "none":
        weights = torch.tensor([0.5, 2.0, -1.0], device="cuda")
        (out * weights).sum().backward()
    else:
        (out * 3.5).backward()
    # oracle: per-sample gradient times the upstream factor of each sample
    _, _, gref, _ = oracle.batch(x.detach().cpu().numpy(), w.targets, w.logit_lengths, w.target_lengths,
                                 blank=-1, reduction="none")
    if reduction == "none":
        fac = np.repeat([0.5, 2.0, -1.0], [w.rows(i).stop - w.rows(i).start for i in range(3)])[:, None]
    else:
        fac = 3.5 / w.B if reduction == "mean" else 3.5
    err = np.abs(x.grad.double().cpu().numpy() - gref * fac).max()
    assert err <= 1e-5 * (3.5 if reduction != "none" else 2.0)


def test_readme_example_golden(rl):
    """The README usage layout (24 rows, V=8) against the stored oracle values."""
    import json
    gd = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "readme_example.json")))
    logits = torch.tensor(gd["logits"], dtype=torch.float32, device="cuda")
    tg = torch.tensor(gd["targets"], dtype=torch.int32, device="cuda")
    for case in gd["cases"]:
        loss, red, grad, _ = rl.rnnt_loss_fused(logits, tg, gd["logit_lengths"], gd["target_lengths"], blank=-1,
                                                reduction=case["reduction"])
        out = (loss if case["reduction"] == "none" else red).double().cpu().numpy()
        np.testing.assert_allclose(out, case["loss"], rtol=1e-5, atol=0)
        np.testing.assert_allclose(grad.double().cpu().numpy(), np.array(case["grad"]), rtol=0, atol=1e-5)


# ------------------------------------------------ log-domain recursion fallback
def test_extreme_log_probs_take_the_log_domain_path(rl):
    """Non-fused inputs with log-probs far outside [-80, 80]: the log-domain sweep must match the oracle.

    Values are multiples of 1/4, exact in fp32 and fp16, so no input rounding enters.
    """
    rng = np.random.default_rng(41)
    Ts, Us, V = [20, 9, 14], [6, 3, 0], 24
    w = _custom(Ts, Us, V, std=1.0, blank=0, fused=False, reduction="sum", seed=41)
    x = np.round(rng.uniform(-300.0, -0.25, size=(w.N, V)) * 4) / 4
    x[::7, 0] = -0.5          # some likely blanks keep the total probability away from underflow
    w.logits = torch.tensor(x, dtype=torch.float32, device="cuda")
    loss, red, grad, flags = run(rl, w)
    assert flags == 0
    check_against_oracle(w, loss, grad, "sum")


@pytest.mark.parametrize("U", [40, 63, 100, 130, 300, 600, 900, 1100, 1700, 2047])
def test_log_domain_across_register_tiles(rl, U):
    """The log-domain sweep on lattices wide enough for one to four column groups per lane.

    Values are multiples of 1/4 (exact in fp32); one in five blank log-probs is -0.5 so the total
    probability stays away from underflow in fp64.
    """
    rng = np.random.default_rng(U)
    Ts, Us, V = [4, 3], [U, U // 2], 12
    w = _custom(Ts, Us, V, std=1.0, blank=0, fused=False, reduction="none", seed=U)
    x = np.round(rng.uniform(-200.0, -0.25, size=(w.N, V)) * 4) / 4
    x[::5, 0] = -0.5
    w.logits = torch.tensor(x, dtype=torch.float32, device="cuda")
    loss, red, grad, flags = run(rl, w)
    assert flags == 0
    check_against_oracle(w, loss, grad, "none")


def test_extreme_fused_logits(rl):
    """Fused logits of spread ~N(0, 40^2): log-probs reach -300, the sample takes the log-domain sweep.  The
    fp32 steps work on x - max, never on x, so the fp32 gate holds: loss 1e-5 relative, gradient 1e-5."""
    w = _custom([25, 11], [5, 4], 64, std=40.0, blank=-1, reduction="sum", seed=42)
    loss, red, grad, flags = run(rl, w)
    assert flags == 0
    check_against_oracle(w, loss, grad, "sum")


def _offset_rows(w, offset, seed):
    """The logits of w with a constant added to every row: `offset` itself, or (offset "random") a per-row
    constant drawn uniformly from [-1000, 1000].  The sum is rounded to the logits' dtype; the oracle reads the
    rounded values."""
    if offset == "random":
        g = torch.Generator(device="cuda").manual_seed(seed)
        c = (torch.rand(w.N, 1, generator=g, device="cuda", dtype=torch.float64) * 2000.0 - 1000.0)
    else:
        c = torch.full((w.N, 1), float(offset), device="cuda", dtype=torch.float64)
    return (w.logits.double() + c).to(w.logits.dtype)


@pytest.mark.parametrize("offset", [50.0, 100.0, 300.0, 1000.0, -1000.0, "random"])
@pytest.mark.parametrize("case", ["tiny", "char", "bpe_shaped", "wide_fp32", "half_fp16", "stream_fp32"])
def test_fused_logit_offsets(rl, case, offset):
    """log_softmax is shift-invariant (README parameter table, fused_log_softmax; "Value" section 3), so a
    constant added to a row's logits must leave the fused path within the parity gates: fp32 loss 1e-5
    relative and gradient 1e-5 absolute (fp16: 2e-3 / 3e-3).  Offsets of 50 to 1000 (and random per-row
    ones) on the tiny and char workloads, a bpe-shaped batch (V = 1024, one 4 KiB row per wave), rows of
    16 KiB split over four gradient waves, and fp16 rows of V = 4096."""
    if case in ("tiny", "char"):
        w = workloads.make(case, device="cuda")
    elif case == "bpe_shaped":
        w = _custom([60, 37, 81], [20, 9, 31], 1024, std=2.0, blank=-1, reduction="mean", seed=31)
    elif case == "wide_fp32":
        w = _custom([9, 14], [6, 3], 4096, std=2.0, blank=-1, reduction="sum", seed=32)
    elif case == "stream_fp32":
        w = _custom([8, 11], [5, 4], 5000, std=2.0, blank=-1, reduction="sum", seed=34)
    else:
        w = _custom([30, 21], [8, 12], 4096, dtype=torch.float16, std=2.0, blank=-1, clamp=1.0,
                    reduction="mean", seed=33)
    w.logits = _offset_rows(w, offset, seed=len(case))
    loss, red, grad, flags = run(rl, w)
    assert flags == 0
    check_against_oracle(w, loss, grad, w.reduction)


def test_bpe_workload_random_row_offsets(rl):
    """The full bpe batch with a per-row offset drawn from [-1000, 1000]: every loss at 1e-5, every gradient
    row of the smallest and the largest sample at 1e-5, 200 rows of every other sample; fused rows sum to 0."""
    w = workloads.make("bpe", device="cuda")
    w.logits = _offset_rows(w, "random", seed=3)
    loss, red, grad, flags = run(rl, w)
    assert flags == 0
    order = np.argsort(w.logit_lengths.astype(np.int64) * (w.target_lengths + 1))
    check_against_oracle(w, loss, grad, w.reduction, grad_rows="all", samples=[int(order[0]), int(order[-1])])
    check_against_oracle(w, loss, grad, w.reduction, grad_rows=200, samples=[int(i) for i in order[1:-1]], seed=1)
    assert grad.double().sum(dim=1).abs().max().item() < 1e-6


def test_mixed_domains_in_one_batch(rl):
    """One sample with ordinary log-probs, one with extreme ones: each takes its own sweep."""
    rng = np.random.default_rng(43)
    w = _custom([30, 30], [8, 8], 16, std=1.0, blank=-1, fused=False, prenormalise=True, reduction="none", seed=43)
    x = w.logits.cpu().numpy().astype(np.float64)
    sl = w.rows(1)
    x[sl] = np.round(rng.uniform(-200.0, -1.0, size=x[sl].shape) * 4) / 4
    w.logits = torch.tensor(x, dtype=torch.float32, device="cuda")
    loss, red, grad, flags = run(rl, w)
    check_against_oracle(w, loss, grad, "none")


# ------------------------------------------------------------------- FastEmit
@pytest.mark.parametrize("V,dtype,fused,lam,clamp", [
    (29, torch.float32, True, 0.01, -1.0),       # narrow rows (several rows per wave)
    (1024, torch.float32, True, 0.5, -1.0),      # one 4 KiB row per wave
    (1000, torch.float32, True, 2.0, 0.1),       # unaligned row length (scalar tail), clamp
    (4096, torch.float16, True, 0.5, -1.0),      # half rows of 8 KiB
    (8192, torch.float32, True, 0.3, 0.05),      # rows split over several waves, clamp
    (2048, torch.float16, False, 0.3, -1.0),     # log-prob inputs: flows only
    (50, torch.float32, False, 1.0, 0.2),
])
def test_fastemit_gradient(rl, V, dtype, fused, lam, clamp):
    w = _custom([31, 12, 1, 20], [7, 4, 5, 0], V, dtype=dtype, std=2.0, blank=-1, fused=fused,
                prenormalise=not fused, clamp=clamp, reduction="mean", seed=V + 3)
    loss, red, grad, flags = run(rl, w, fastemit=lam)
    assert flags == 0
    check_against_oracle(w, loss, grad, "mean", fastemit=lam)
    plain, _, _, _ = run(rl, w)
    assert torch.equal(loss, plain)   # the loss value does not depend on the FastEmit weight


def test_fastemit_log_domain(rl):
    """Extreme log-prob inputs (the log-domain sweep) with a FastEmit weight."""
    rng = np.random.default_rng(44)
    w = _custom([18, 7], [5, 3], 20, std=1.0, blank=0, fused=False, reduction="sum", seed=44)
    x = np.round(rng.uniform(-250.0, -0.25, size=(w.N, w.V)) * 4) / 4
    x[::6, 0] = -0.5
    w.logits = torch.tensor(x, dtype=torch.float32, device="cuda")
    loss, red, grad, flags = run(rl, w, fastemit=0.7)
    assert flags == 0
    check_against_oracle(w, loss, grad, "sum", fastemit=0.7)


def test_fastemit_bpe_full_size(rl):
    """The full bpe batch with lambda = 0.01: every loss, every row of the smallest and largest samples, and
    rows of a middle one; each fused gradient row still sums to zero."""
    w = workloads.make("bpe", device="cuda")
    loss, red, grad, flags = run(rl, w, fastemit=0.01)
    assert flags == 0
    order = np.argsort(w.logit_lengths.astype(np.int64) * (w.target_lengths + 1))
    check_against_oracle(w, loss, grad, w.reduction, grad_rows="all", samples=[int(order[0]), int(order[-1])],
                         fastemit=0.01)
    assert grad.double().sum(dim=1).abs().max().item() < 1e-6


def test_fastemit_padded_and_autograd(rl):
    Ts, Us = [26, 9, 14], [6, 2, 11]
    w = workloads.make_custom(Ts, Us, 96, std=2.0, reduction="none", seed=45, device="cuda")
    lam = 0.25
    tg = torch.from_numpy(w.targets).to("cuda")
    ref_loss, _, ref_grad, _ = run(rl, w, fastemit=lam)
    check_against_oracle(w, ref_loss, ref_grad, "none", fastemit=lam)
    max_T, max_U1 = 28, 13
    xp = _to_padded(w, max_T, max_U1)
    loss_p, _, grad_p, _ = rl.rnnt_loss_fused(xp, tg, w.logit_lengths, w.target_lengths, blank=w.blank,
                                              reduction="none", fastemit_lambda=lam)
    torch.cuda.synchronize()
    rows, pad = _padded_rows(w, grad_p, max_T, max_U1)
    assert torch.equal(loss_p, ref_loss) and torch.equal(rows, ref_grad) and bool((pad == 0).all())
    x = w.logits.clone().requires_grad_(True)
    out = rl.rnnt_loss(x, tg, w.logit_lengths, w.target_lengths, blank=w.blank, reduction="none",
                       fastemit_lambda=lam)
    up = torch.tensor([1.5, -0.5, 2.0], device="cuda")
    out.backward(up)
    torch.cuda.synchronize()
    fac = torch.cat([torch.full((w.rows(i).stop - w.rows(i).start, 1), float(up[i])) for i in range(3)]).cuda()
    assert torch.allclose(x.grad, ref_grad * fac, rtol=1e-6, atol=0)


# ------------------------------------------------------------ HIP graph capture
def test_graph_capture_and_replay(rl):
    """A batch of up to 64 samples enqueues kernels only: capture one call, replay it several times with eager
    calls and synchronisations in between, and check every replay bit for bit against the eager result."""
    w = workloads.make("char", seed=2, device="cuda")
    tg = torch.from_numpy(w.targets).to("cuda")
    T, U = w.logit_lengths, w.target_lengths
    loss = torch.empty(w.B, dtype=torch.float32, device="cuda")
    red = torch.empty(1, dtype=torch.float32, device="cuda")
    grad = torch.empty_like(w.logits)
    ws = torch.empty(rl.workspace_bytes(w.logits, T, U), dtype=torch.uint8, device="cuda")

    def call():
        rl.rnnt_loss_fused(w.logits, tg, T, U, blank=w.blank, reduction=w.reduction, fused_log_softmax=w.fused,
                           grad=grad, workspace=ws, loss=loss, loss_reduced=red)

    call()
    torch.cuda.synchronize()
    ref = (loss.clone(), red.clone(), grad.clone())
    check_against_oracle(w, ref[0], ref[2], w.reduction)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    other = workloads.make_custom([30, 12], [6, 3], 40, std=2.0, seed=9, device="cuda")
    for k in range(3):
        loss.zero_()
        red.zero_()
        grad.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(loss, ref[0]) and torch.equal(red, ref[1]) and torch.equal(grad, ref[2]), k
        run(rl, other)              # eager work of another batch in between
        torch.cuda.synchronize()


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")  # nothing is captured: both calls are refused
def test_graph_capture_refuses_host_copies(rl):
    """More than 64 samples (and the multi-blank path) copy their schedule from the host: refused under capture."""
    Ts, Us = [5] * 70, [2] * 70
    w = workloads.make_custom(Ts, Us, 16, std=1.0, seed=10, device="cuda")
    tg = torch.from_numpy(w.targets).to("cuda")
    loss = torch.empty(w.B, dtype=torch.float32, device="cuda")
    ws = torch.empty(rl.workspace_bytes(w.logits, w.logit_lengths, w.target_lengths), dtype=torch.uint8,
                     device="cuda")
    grad = torch.empty_like(w.logits)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        with pytest.raises(ValueError):
            rl.rnnt_loss_fused(w.logits, tg, w.logit_lengths, w.target_lengths, reduction="none", grad=grad,
                               workspace=ws, loss=loss)
        with pytest.raises(ValueError):
            rl.rnnt_multiblank_fused(w.logits, tg, w.logit_lengths, w.target_lengths, big_blank_ids=[13],
                                     big_blank_durations=[2], reduction="none",
                                     grad=grad, loss=loss)
    torch.cuda.synchronize()
    loss2, _, _, _ = rl.rnnt_loss_fused(w.logits, tg, w.logit_lengths, w.target_lengths, reduction="none")
    torch.cuda.synchronize()
    assert torch.isfinite(loss2).all()


def test_concurrent_calls_from_two_threads(rl):
    """Two host threads, each on its own stream with its own batch and buffers, alternate calls: one batch of
    more than 64 samples (schedule through the pinned staging ring), one of 8 (schedule as kernel arguments),
    so the plan cache is replaced on nearly every call.  Every result equals its sequential reference."""
    import threading
    rng = np.random.default_rng(91)
    big = workloads.make_custom(rng.integers(5, 40, size=80).tolist(), rng.integers(0, 12, size=80).tolist(), 64,
                                std=2.0, seed=91, reduction="sum", device="cuda")
    small = workloads.make("char", seed=101, device="cuda")

    def buffers(w):
        return dict(loss=torch.empty(w.B, dtype=torch.float32, device="cuda"),
                    loss_reduced=torch.empty(1, dtype=torch.float32, device="cuda"),
                    grad=torch.empty_like(w.logits),
                    workspace=torch.empty(rl.workspace_bytes(w.logits, w.logit_lengths, w.target_lengths),
                                          dtype=torch.uint8, device="cuda"))

    def call(w, buf):
        tg = torch.from_numpy(w.targets).to("cuda")
        rl.rnnt_loss_fused(w.logits, tg, w.logit_lengths, w.target_lengths, blank=w.blank, reduction=w.reduction,
                           fused_log_softmax=w.fused, **buf)

    refs = {}
    for name, w in (("big", big), ("small", small)):
        b = buffers(w)
        call(w, b)
        torch.cuda.synchronize()
        refs[name] = (b["loss"].clone(), b["loss_reduced"].clone(), b["grad"].clone())
    check_against_oracle(big, refs["big"][0], refs["big"][2], "sum")
    errors = []

    def worker(name, w):
        try:
            stream = torch.cuda.Stream()
            b = buffers(w)
            with torch.cuda.stream(stream):
                for _ in range(25):
                    call(w, b)
                    stream.synchronize()
                    ok = (torch.equal(b["loss"], refs[name][0]) and torch.equal(b["loss_reduced"], refs[name][1])
                          and torch.equal(b["grad"], refs[name][2]))
                    if not ok:
                        errors.append(name)
                        return
        except Exception as e:  # pragma: no cover - reported below
            errors.append(f"{name}: {e!r}")

    threads = [threading.Thread(target=worker, args=(n, w)) for n, w in (("big", big), ("small", small))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors


def test_very_long_lattices(rl):
    """T = 20000 frames (about 20000 dependent diagonal steps, total probabilities near e^-55000, far below fp64's
    range, carried by the sweeps' exponents), with U = 3 and U = 0, fused fp32: every loss and the whole gradient."""
    w = _custom([20000, 12000], [3, 0], 16, std=1.0, blank=-1, reduction="none", seed=17)
    loss, red, grad, flags = run(rl, w)
    assert flags == 0
    check_against_oracle(w, loss, grad, "none")


@pytest.mark.parametrize("gap,jitter", [(15.0, 0.0), (20.0, 0.0), (15.0, 1.0), (25.0, 2.0)])
def test_peaked_blank_lattices(rl, gap, jitter):
    """The blank logit `gap` nats above every label on every row (a model that favours blank everywhere): each
    label costs ~gap nats, so along an anti-diagonal alpha falls by ~gap per label while the nodes that carry the
    alignment mass sit hundreds of nats below the diagonal's largest value.  The probability-domain sweeps lose
    them (fp64 range); the forward-backward check catches it and reruns the sample in the log domain.  Every loss
    and the whole gradient against the oracle."""
    Ts, Us, V = [300, 40, 120], [100, 39, 30], 8
    w = _custom(Ts, Us, V, std=1.0, blank=0, reduction="none", seed=int(gap * 10 + jitter))
    rng = np.random.default_rng(int(gap))
    x = np.zeros(tuple(w.logits.shape), np.float32)
    x[:, 0] = gap
    x += (jitter * rng.standard_normal(x.shape)).astype(np.float32)
    w.logits = torch.from_numpy(x).to("cuda")
    loss, red, grad, flags = run(rl, w)
    assert flags == 0
    check_against_oracle(w, loss, grad, "none")


@pytest.mark.parametrize("size", ["small", "large"])
@pytest.mark.parametrize("reduction", ["none", "sum"])
def test_launch_paths_on_mixed_batches(rl, size, reduction):
    """Batches below 64512 lattice rows take three launches (the row pass finds its chunks from descriptors passed
    as kernel arguments and reports its flags per chunk; one workgroup per sample runs both recursions, their
    check and the rerun), larger ones six.  On both sides of that line, one batch mixes an ordinary sample, one
    whose blank logit is 20 nats above every label (its probability-domain sweeps lose the alignment mass, the
    check sends it to the log domain), one with logits of spread 40 (log-probs beyond -80: the row pass sends it
    to the log domain) and one with a label outside [0, V) (no alignment, the status word flagged).  Every loss,
    the whole gradient and the reduction against the oracle."""
    scale = 1 if size == "small" else 6
    Ts = [120 * scale, 100 * scale, 80 * scale, 60 * scale]
    Us, V = [30, 60, 20, 10], 16
    w = _custom(Ts, Us, V, std=1.0, blank=0, reduction=reduction, seed=77 + scale)
    rows = sum(t * (u + 1) for t, u in zip(Ts, Us))
    assert (rows < 64512) == (size == "small")
    x = w.logits.float().cpu().numpy()
    peaked = x[w.rows(1)]
    peaked[:] = 0.25 * np.random.default_rng(5).standard_normal(peaked.shape).astype(np.float32)
    peaked[:, 0] += 30.0
    x[w.rows(2)] *= 40.0
    w.logits = torch.from_numpy(x).to("cuda")
    tg = w.targets.copy()
    tg[3, 4] = V + 3
    w.targets = tg
    loss, red, grad, ws = rl.rnnt_loss_fused(w.logits, torch.from_numpy(tg).to("cuda"), w.logit_lengths,
                                             w.target_lengths, blank=0, reduction=reduction)
    flags = rl.device_flags(ws)
    assert flags == 2
    # the per-sample mode words (int32 at byte 256 of the workspace): 0 probability domain, 1 log domain from the
    # row pass, 2 rerun after a failed check (the peaked sample, and the one without an alignment)
    mode = ws[256:256 + 4 * w.B].view(torch.int32).tolist()
    assert mode == [0, 2, 1, 2], mode

    def ref(i):
        T, U = int(w.logit_lengths[i]), int(w.target_lengths[i])
        return oracle.sample(x[w.rows(i)], T, U, w.targets[i], 0, True, -1.0, allow_bad_targets=True)
    check_masked(w, loss, grad, ref)
    assert math.isinf(loss[3].item()) and all(math.isfinite(loss[i].item()) for i in range(3))
    if reduction == "sum":
        assert math.isinf(red.item())


@pytest.mark.parametrize("Ts,Us,V,blank,std,clamp,reduction,seed", [
    ([131], [537], 2, 1, 8.0, -1.0, "none", 5091),
    ([299, 247, 131], [152, 121, 472], 8, 7, 2.0, 0.1, "sum", 5113),
])
def test_fastemit_on_lattices_with_underflowing_corners(rl, Ts, Us, V, blank, std, clamp, reduction, seed):
    """Wide lattices (U up to 537) whose far corners underflow in the probability domain while carrying no
    alignment mass: the FastEmit term must leave those nodes' zero occupancy alone (it produced NaN gradients
    there).  Every loss and the whole gradient against the oracle."""
    w = _custom(Ts, Us, V, std=std, blank=blank, clamp=clamp, reduction=reduction, seed=seed)
    loss, red, grad, flags = run(rl, w, fastemit=0.3)
    assert flags == 0
    check_against_oracle(w, loss, grad, reduction, fastemit=0.3)


def check_masked(w, loss, grad, oracle_fn, gtol=1e-5):
    """Per-sample comparison that admits impossible alignments: an infinite oracle loss must come back as +inf
    with a zero gradient, a finite one to the fp32 tolerances."""
    for i in range(w.B):
        r = oracle_fn(i)
        g = grad[w.rows(i)].detach().double().cpu().numpy()
        lg = float(loss[i].item())
        if np.isinf(r.loss):
            assert np.isinf(lg) and lg > 0, f"sample {i}: loss {lg}, oracle +inf"
            assert np.all(g == 0), f"sample {i}: impossible alignment with a non-zero gradient"
        else:
            assert abs(lg - r.loss) <= 1e-5 * max(1.0, abs(r.loss)), f"sample {i}: loss {lg} vs oracle {r.loss}"
            assert np.isfinite(g).all() and np.abs(g - r.grad).max() <= gtol, f"sample {i}: gradient"


@pytest.mark.parametrize("fused,frac,lam", [(True, 0.3, 0.0), (True, 0.7, 0.2), (False, 0.3, 0.2), (False, 0.7, 0.0)])
def test_masked_vocabulary(rl, fused, frac, lam, oracle_mod):
    """-inf logits (or log-probs) on a random share of the non-blank classes of every row: edges that are exactly
    impossible, and samples whose every alignment is (loss +inf, zero gradient).  Every loss and gradient."""
    Ts, Us, V = [40, 25, 60, 7, 33], [30, 12, 45, 6, 0], 29
    w = _custom(Ts, Us, V, std=2.0 if fused else 1.5, blank=0, fused=fused, prenormalise=not fused,
                reduction="none", seed=int(frac * 100) + fused)
    rng = np.random.default_rng(int(frac * 100))
    x = w.logits.float().cpu().numpy()
    m = rng.random(x.shape) < frac
    m[:, 0] = False
    x[m] = -np.inf
    w.logits = torch.from_numpy(x).to("cuda")
    loss, red, grad, flags = run(rl, w, fastemit=lam)

    def ref(i):
        T, U = int(w.logit_lengths[i]), int(w.target_lengths[i])
        return oracle_mod.sample(x[w.rows(i)], T, U, w.targets[i], 0, fused, -1.0, want_grad=True,
                                 fastemit_lambda=lam)
    check_masked(w, loss, grad, ref)


# ------------------------------------------------------ randomized option sweep
def _random_case(seed):
    """One seeded draw over the option space: batch shape, vocabulary, dtype, fused or not, blank position,
    clamp, FastEmit, reduction and logits alignment."""
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 12))
    V = int(rng.choice([1, 2, 7, 16, 29, 64, 100, 257, 512, 1000, 1024, 1025, 1028, 2048, 2049, 4097]))
    Ts = rng.integers(1, 70, size=B).tolist()
    Us = (rng.integers(0, 30, size=B) if V > 1 else np.zeros(B, np.int64)).tolist()
    dtype = torch.float16 if rng.random() < 0.4 else torch.float32
    fused = bool(rng.random() < 0.7)
    blank = int(rng.integers(-V, V))
    clamp = float(rng.choice([-1.0, -1.0, 0.05, 0.3]))
    lam = float(rng.choice([0.0, 0.0, 0.01, 0.5]))
    reduction = str(rng.choice(["none", "mean", "sum"]))
    return dict(Ts=Ts, Us=Us, V=V, dtype=dtype, fused=fused, blank=blank, clamp=clamp, lam=lam,
                reduction=reduction, unaligned=bool(rng.random() < 0.2), padded=bool(rng.random() < 0.2))


@pytest.mark.parametrize("seed", range(1000, 1024))
def test_random_option_sweep(rl, seed):
    c = _random_case(seed)
    w = _custom(c["Ts"], c["Us"], c["V"], dtype=c["dtype"], std=2.0 if c["fused"] else 1.5, blank=c["blank"],
                clamp=c["clamp"], fused=c["fused"], prenormalise=not c["fused"], reduction=c["reduction"], seed=seed)
    if c["unaligned"]:
        buf = torch.empty(w.logits.numel() + 1, dtype=w.logits.dtype, device="cuda")
        buf[1:].copy_(w.logits.reshape(-1))
        w.logits = buf[1:].view(w.N, w.V)
    loss, red, grad, flags = run(rl, w, fastemit=c["lam"])
    assert flags == 0, c
    check_against_oracle(w, loss, grad, c["reduction"], fastemit=c["lam"])
    _reduced_ok(w, loss, red, c["reduction"])
    if c["padded"]:
        max_T, max_U1 = max(c["Ts"]) + 2, max(c["Us"]) + 3
        xp = _to_padded(w, max_T, max_U1)
        tg = torch.from_numpy(w.targets).to("cuda")
        lp_, _, gp_, _ = rl.rnnt_loss_fused(xp, tg, w.logit_lengths, w.target_lengths, blank=w.blank,
                                            clamp=c["clamp"], reduction=c["reduction"], fused_log_softmax=w.fused,
                                            fastemit_lambda=c["lam"])
        torch.cuda.synchronize()
        rows, pad = _padded_rows(w, gp_, max_T, max_U1)
        assert bool((pad == 0).all())
        row_bytes = c["V"] * w.logits.element_size()
        if row_bytes > 1024 and row_bytes % 16 != 0:
            # rows off 16-byte boundaries: the row pass's lanes take a row's elements by their place in 16-byte
            # blocks, so the padded copy (its rows at other addresses) agrees to rounding: against the oracle
            check_against_oracle(w, lp_, rows, c["reduction"], fastemit=c["lam"])
        else:
            if c["unaligned"]:
                # the unaligned call's rows sit elsewhere in their 16-byte blocks (or take the scalar kernels):
                # the bitwise reference is the same packed logits, aligned
                w.logits = w.logits.contiguous().clone()
                loss, red, grad, flags = run(rl, w, fastemit=c["lam"])
            assert torch.equal(lp_, loss) and torch.equal(rows, grad)
