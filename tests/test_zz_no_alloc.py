"""rnnt_loss_fused_noalloc against rnnt_loss_fused, through the C ABI (run on an MI355X).

The allocation-free call is for callers that cannot allocate device memory during the call (HIP graph
capture, serving loops, harnesses that forbid hipMalloc): its workspace is the library's fixed device scratch.
It must give what the call with a caller workspace gives, bit for bit (same kernels, same schedule), and so
meet the oracle's gates.  Several calls in a row share the scratch: a larger batch, then a smaller one (whose
schedule and status word must not inherit anything), then one with a bad label (status bit set) and a clean
one after it (status clear again).
"""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rl():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rnn_transducer_loss_amd as rl
    rl._lib.load()
    return rl


def _code(w):
    from rnn_transducer_loss_amd import _lib
    return _lib.RNNT_F16 if w.logits.dtype == torch.float16 else _lib.RNNT_F32


def _noalloc(rl, w):
    """One allocation-free call; returns (loss, loss_reduced, grad, status word)."""
    from rnn_transducer_loss_amd import _lib
    tg = torch.from_numpy(w.targets).to("cuda")
    loss = torch.full((w.B,), float("nan"), dtype=torch.float32, device="cuda")
    red = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    grad = torch.full_like(w.logits, float("nan"))
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    _lib.loss_fused_noalloc(w.logits.data_ptr(), _code(w), w.N, w.V, tg.data_ptr(), tg.shape[1], w.logit_lengths,
                            w.target_lengths, w.blank, w.clamp, w.fused, w.reduction, loss.data_ptr(),
                            red.data_ptr() if w.reduction != "none" else 0, grad.data_ptr(), status.data_ptr(),
                            stream)
    torch.cuda.synchronize()
    return loss, (red if w.reduction != "none" else None), grad, int(status.item()) & 0xffffffff


def _with_workspace(rl, w):
    tg = torch.from_numpy(w.targets).to("cuda")
    loss, red, grad, ws = rl.rnnt_loss_fused(w.logits, tg, w.logit_lengths, w.target_lengths, blank=w.blank,
                                             clamp=w.clamp, reduction=w.reduction, fused_log_softmax=w.fused)
    flags = rl.device_flags(ws)
    torch.cuda.synchronize()
    return loss, red, grad, flags


def _same(a, b):
    la, ra, ga, fa = a
    lb, rb, gb, fb = b
    assert fa == fb, (fa, fb)
    assert torch.equal(la, lb)
    assert (ra is None and rb is None) or torch.equal(ra, rb)
    assert torch.equal(ga, gb)


def test_noalloc_matches_the_workspace_call_on_consecutive_calls(rl):
    from test_parity_gpu import check_against_oracle
    big = workloads.make_custom([300, 250, 220, 180], [60, 80, 40, 75], 1024, std=2.0, blank=-1,
                                reduction="mean", seed=301, device="cuda")
    odd = workloads.make_custom([70, 45], [25, 31], 1025, std=2.0, blank=-1, reduction="sum", seed=303,
                                device="cuda")  # 4100-byte rows: the odd row and gradient forms
    small = workloads.make("char", device="cuda")
    for w, rows in ((big, 300), (odd, "all"), (small, "all")):
        out = _noalloc(rl, w)
        ref = _with_workspace(rl, w)
        _same(out, ref)
        assert out[3] == 0
        check_against_oracle(w, out[0], out[2], w.reduction, grad_rows=rows)


def test_noalloc_status_word_starts_clear_on_each_call(rl):
    from test_parity_gpu import check_against_oracle
    w = workloads.make("tiny", device="cuda")
    bad = workloads.make("tiny", device="cuda")
    tg = bad.targets.copy()
    tg[0, 1] = 15          # equals blank (V-1): no alignment for sample 0
    bad.targets = tg
    out = _noalloc(rl, bad)
    assert out[3] & 2
    _same(out, _with_workspace(rl, bad))
    assert np.isinf(out[0][0].item()) and bool((out[2][bad.rows(0)] == 0).all())
    clean = _noalloc(rl, w)
    assert clean[3] == 0
    _same(clean, _with_workspace(rl, w))
    check_against_oracle(w, clean[0], clean[2], w.reduction)


def test_noalloc_fp16_and_score_only(rl):
    from rnn_transducer_loss_amd import _lib
    from test_parity_gpu import check_against_oracle
    w = workloads.make_custom([90, 61, 40], [20, 33, 0], 4096, dtype=torch.float16, std=2.0, blank=-1, clamp=1.0,
                              reduction="mean", seed=302, device="cuda")
    out = _noalloc(rl, w)
    _same(out, _with_workspace(rl, w))
    check_against_oracle(w, out[0], out[2], "mean", grad_rows=200)
    # grad = NULL: the losses alone
    tg = torch.from_numpy(w.targets).to("cuda")
    loss = torch.empty(w.B, dtype=torch.float32, device="cuda")
    _lib.loss_fused_noalloc(w.logits.data_ptr(), _code(w), w.N, w.V, tg.data_ptr(), tg.shape[1], w.logit_lengths,
                            w.target_lengths, w.blank, w.clamp, w.fused, "none", loss.data_ptr(), 0, 0, 0,
                            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(loss, out[0])
