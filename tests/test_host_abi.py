"""CPU-only checks of librnnt's C ABI: symbols, host validation and the schedule.

No compute call is made (there is no GPU here): rnnt_loss_fused_workspace_size
and rnnt_plan_describe touch no device, and argument errors are rejected by
rnnt_loss_fused before anything is enqueued.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from rnn_transducer_loss_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"\b(rnnt_\w+)\s*\(", text)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    declared = _declared_functions()
    assert set(_lib.EXPORTS) <= set(declared)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    assert _lib.status_string(0) == "success"
    assert "invalid" in _lib.status_string(1)
    assert _lib.status_string(99) == "unknown status"


def _ws(T, U, V=16, dtype=_lib.RNNT_F32, N=None):
    T = np.asarray(T, np.int32)
    U = np.asarray(U, np.int32)
    if N is None:
        N = int((T.astype(np.int64) * (U + 1)).sum())
    return _lib.workspace_size(len(T), V, N, dtype, T, U)


def test_workspace_size_grows_with_the_batch():
    a = _ws([12, 9], [4, 3])
    b = _ws([12, 9, 30], [4, 3, 7])
    assert 0 < a < b
    # per-node aux: 4 B den per row + 24 B per skewed slot, plus tables.
    T, U = 300, 70
    rows, slots = T * (U + 1), (T + U) * (U + 1)
    assert _ws([T], [U], V=1024) >= 4 * rows + 24 * slots


@pytest.mark.parametrize("T,U,N", [([0, 3], [1, 1], None), ([3, 3], [-1, 1], None), ([4], [2], 11),
                                   ([4], [2047], None), ([2], [2048], None)])
def test_workspace_size_rejects_bad_lengths(T, U, N):
    if U == [2047]:
        assert _ws(T, U) > 0      # widest lattice the kernels support
        return
    with pytest.raises(ValueError):
        _ws(T, U, N=N)


def test_workspace_size_rejects_bad_dtype_and_sizes():
    T = np.array([3], np.int32)
    U = np.array([1], np.int32)
    with pytest.raises(ValueError):
        _lib.workspace_size(1, 8, 6, 7, T, U)
    with pytest.raises(ValueError):
        _lib.workspace_size(1, 0, 6, 0, T, U)
    with pytest.raises(ValueError):
        _lib.workspace_size(0, 8, 0, 0, T[:0], U[:0])


def _call_fused(**over):
    """rnnt_loss_fused with fake (never dereferenced) device pointers; only host checks can run."""
    T = np.array([4, 6], np.int32)
    U = np.array([2, 1], np.int32)
    args = dict(logits_ptr=0x100000, dtype_code=0, N=24, V=8, targets_ptr=0x200000, S=2, logit_lengths=T,
                target_lengths=U, blank=-1, clamp=-1.0, fused=True, reduction="mean", loss_ptr=0x300000,
                loss_reduced_ptr=0x400000, grad_ptr=0x500000, ws_ptr=0x600000, ws_bytes=1 << 20, stream=0)
    args.update(over)
    _lib.loss_fused(**args)


@pytest.mark.parametrize("over", [
    dict(blank=8), dict(blank=-9), dict(N=25), dict(S=1), dict(targets_ptr=0), dict(loss_ptr=0),
    dict(ws_ptr=0), dict(logits_ptr=0), dict(dtype_code=3), dict(V=0),
    dict(grad_ptr=0x100000 + 64),                # partial overlap with logits
    dict(ws_bytes=64),                           # workspace too small
    dict(ws_ptr=0x600010),                       # workspace not 256-byte aligned
    dict(logit_lengths=np.array([4, 0], np.int32)),
    dict(target_lengths=np.array([2, -1], np.int32)),
    dict(fastemit_lambda=-0.5), dict(fastemit_lambda=float("inf")), dict(fastemit_lambda=float("nan")),
])
def test_fused_call_rejects_invalid_arguments_before_any_launch(over):
    with pytest.raises(ValueError):
        _call_fused(**over)


def test_reduction_names_are_checked():
    with pytest.raises(ValueError):
        _call_fused(reduction="avg")


@pytest.mark.parametrize("V,dtype", [(16, _lib.RNNT_F32), (29, _lib.RNNT_F32), (1024, _lib.RNNT_F32),
                                     (4096, _lib.RNNT_F16), (2048, _lib.RNNT_F16)])
def test_schedule_is_longest_first_and_covers_every_row_once(V, dtype):
    rng = np.random.default_rng(V)
    B = 37
    T = rng.integers(1, 200, size=B).astype(np.int32)
    U = rng.integers(0, 60, size=B).astype(np.int32)
    T[5], U[5] = T[6], U[6]                       # a tie in area
    order, chunks = _lib.plan_describe(V, dtype, T, U)
    area = T.astype(np.int64) * (U + 1)
    assert sorted(order.tolist()) == list(range(B))
    for a, b in zip(order[:-1], order[1:]):
        key_a = (area[a], T[a] + U[a], -a)
        key_b = (area[b], T[b] + U[b], -b)
        assert key_a > key_b
    # chunks: samples appear in schedule order, each row of each sample exactly once
    seen = {i: np.zeros(area[i], np.int32) for i in range(B)}
    pos = {int(s): k for k, s in enumerate(order)}
    last = -1
    for s, b0, n in chunks:
        assert pos[int(s)] >= last
        last = pos[int(s)]
        assert n > 0 and 0 <= b0 and b0 + n <= area[s]
        seen[int(s)][b0:b0 + n] += 1
    for i in range(B):
        assert (seen[i] == 1).all()


@pytest.mark.parametrize("V,dtype", [(29, _lib.RNNT_F32), (1024, _lib.RNNT_F32), (4096, _lib.RNNT_F16)])
def test_diagonal_order_runs_match_the_row_order_runs(V, dtype):
    # The wide kernels walk each run in anti-diagonal order from its first
    # node: the runs must have the same sizes as the row-order runs and,
    # walked node by node, cover every lattice node of every sample once.
    rng = np.random.default_rng(V + 1)
    B = 23
    T = rng.integers(1, 160, size=B).astype(np.int32)
    U = rng.integers(0, 80, size=B).astype(np.int32)
    T[0], U[0] = 1, 0
    T[1], U[1] = 1, 70
    T[2], U[2] = 150, 0
    order, rows = _lib.plan_describe(V, dtype, T, U)
    _, diag = _lib.plan_describe(V, dtype, T, U, diagonal=True)
    assert len(rows) == len(diag)
    assert (rows[:, 0] == diag[:, 0]).all() and (rows[:, 2] == diag[:, 3]).all()
    seen = {i: np.zeros((T[i], U[i] + 1), np.int32) for i in range(B)}
    for s, n, u, cnt in diag:
        Ti, Ui = int(T[s]), int(U[s])
        for _ in range(cnt):
            t = n - u
            assert 0 <= u <= Ui and 0 <= t < Ti
            seen[int(s)][t, u] += 1
            # next node in anti-diagonal order
            if u < min(n, Ui):
                u += 1
            else:
                n += 1
                u = max(0, n - Ti + 1)
    for i in range(B):
        assert (seen[i] == 1).all()


def test_padded_workspace_matches_packed_and_checks_extents():
    T = np.array([12, 9, 30], np.int32)
    U = np.array([4, 3, 11], np.int32)
    N = int((T * (U + 1)).sum())
    packed = _lib.workspace_size(3, 64, N, _lib.RNNT_F32, T, U)
    padded = _lib.workspace_size_padded(3, 64, 30, 12, _lib.RNNT_F32, T, U)
    assert packed == padded
    assert _lib.workspace_size_padded(3, 64, 40, 20, _lib.RNNT_F32, T, U) == packed
    for max_T, max_U1 in [(29, 12), (30, 11), (0, 12), (30, 0)]:
        with pytest.raises(ValueError):
            _lib.workspace_size_padded(3, 64, max_T, max_U1, _lib.RNNT_F32, T, U)


def test_schedule_chunk_sizes_follow_row_bytes():
    T = np.array([400] * 8, np.int32)
    U = np.array([100] * 8, np.int32)
    _, c32 = _lib.plan_describe(1024, _lib.RNNT_F32, T, U)
    _, c16 = _lib.plan_describe(4096, _lib.RNNT_F16, T, U)
    # about 256 KiB of logits per chunk, in multiples of 64 rows
    assert c32[0, 2] == 64 and c16[0, 2] == 64
    assert (c32[:, 2] % 64 == 0).sum() >= len(c32) - 8


def test_small_batches_get_fine_chunks():
    # a character-vocabulary batch (~13 K rows of 29 classes): chunks of 8 rows, so ~1600 workgroups each take
    # one iteration instead of 200 walking 64 rows
    rng = np.random.default_rng(2)
    T = rng.integers(50, 101, size=8).astype(np.int32)
    U = rng.integers(10, 31, size=8).astype(np.int32)
    _, c = _lib.plan_describe(29, _lib.RNNT_F32, T, U)
    N = int((T.astype(np.int64) * (U + 1)).sum())
    assert c[:, 2].max() == 8 and len(c) >= N // 8
    _, tiny = _lib.plan_describe(16, _lib.RNNT_F32, np.array([12, 9], np.int32), np.array([4, 3], np.int32))
    assert tiny[:, 2].max() == 8 and tiny[:, 2].sum() == 12 * 5 + 9 * 4


def _call_multiblank(**over):
    """rnnt_multiblank_loss with fake (never dereferenced) device pointers; only host checks can run."""
    T = np.array([4, 6], np.int32)
    U = np.array([2, 1], np.int32)
    args = dict(logits_ptr=0x100000, dtype_code=0, N=24, V=8, targets_ptr=0x200000, S=2, logit_lengths=T,
                target_lengths=U, blank=-1, big_blank_ids=[6, 5], big_blank_durations=[2, 3], sigma=0.0, clamp=-1.0,
                fastemit_lambda=0.0, fused=True, reduction="mean", loss_ptr=0x300000, loss_reduced_ptr=0x400000,
                grad_ptr=0x500000, ws_ptr=0x600000, ws_bytes=1 << 20, stream=0)
    args.update(over)
    _lib.loss_multiblank(**args)


@pytest.mark.parametrize("over", [
    dict(big_blank_ids=[7, 5]),                       # equal to the standard blank (V-1)
    dict(big_blank_ids=[6, 6]),                       # duplicate
    dict(big_blank_ids=[8, 5]),                       # outside [0, V)
    dict(big_blank_durations=[0, 3]), dict(big_blank_durations=[2, 17]),
    dict(big_blank_ids=[1, 2, 3, 4, 5], big_blank_durations=[2, 2, 2, 2, 2]),   # more than four
    dict(sigma=float("nan")), dict(fastemit_lambda=-1.0), dict(blank=8), dict(N=25), dict(S=1),
    dict(ws_bytes=64), dict(ws_ptr=0x600010), dict(loss_ptr=0),
])
def test_multiblank_call_rejects_invalid_arguments_before_any_launch(over):
    with pytest.raises(ValueError):
        _call_multiblank(**over)


def test_multiblank_ring_limit():
    # R diagonals of the widest lattice (8 bytes a column), R the power of two above the longest duration, must fit
    # 64 KiB of LDS: U+1 = 1000 pads to 1024 columns, so durations up to 7 fit and 8 does not; U+1 = 401 pads to
    # 512, durations up to 15 fit
    T, U = np.array([3], np.int32), np.array([999], np.int32)
    N = 3 * 1000
    assert _lib.workspace_size_multiblank(1, 8, N, 0, T, U, [7]) > 0
    with pytest.raises(ValueError):
        _lib.workspace_size_multiblank(1, 8, N, 0, T, U, [8])
    U4 = np.array([400], np.int32)
    assert _lib.workspace_size_multiblank(1, 8, 3 * 401, 0, T, U4, [2, 15]) > 0
    with pytest.raises(ValueError):
        _lib.workspace_size_multiblank(1, 8, 3 * 401, 0, T, U4, [16])
    assert _lib.workspace_size_multiblank(1, 8, 3 * 200, 0, T, np.array([199], np.int32), [16]) > 0


def test_multiblank_width_limit():
    # the multi-blank sweep keeps an anti-diagonal of up to 1024 columns in one wave (the plain path 2048)
    T = np.array([3], np.int32)
    assert _lib.workspace_size_multiblank(1, 8, 3 * 1024, 0, T, np.array([1023], np.int32), [2]) > 0
    with pytest.raises(ValueError):
        _lib.workspace_size_multiblank(1, 8, 3 * 1025, 0, T, np.array([1024], np.int32), [2])
    assert _ws([3], [1024]) > 0


def test_multiblank_table_span_limit():
    # the sweep addresses a sample's T+U diagonals of 128 (padded) columns of fp64 with 32-bit byte offsets:
    # (T+U) * 128 * 8 must stay below 2^31
    U = np.array([0], np.int32)
    ok, bad = 2 ** 31 // 1024 - 1, 2 ** 31 // 1024
    assert _lib.workspace_size_multiblank(1, 8, ok, 0, np.array([ok], np.int32), U, [2]) > 0
    with pytest.raises(ValueError):
        _lib.workspace_size_multiblank(1, 8, bad, 0, np.array([bad], np.int32), U, [2])


def test_multiblank_padded_sizes_and_limits():
    T = np.array([4, 6, 3], np.int32)
    U = np.array([2, 1, 5], np.int32)
    N = int((T * (U + 1)).sum())
    packed = _lib.workspace_size_multiblank(3, 32, N, _lib.RNNT_F32, T, U, [2, 3])
    padded = _lib.workspace_size_multiblank_padded(3, 32, 6, 6, _lib.RNNT_F32, T, U, [2, 3])
    # the padded layout only adds the per-row normalisers (two fp32 values: the row maximum and log2 of the
    # sum of exp(x - maximum)) of its padding rows
    assert padded - packed == (lambda b: (b + 255) // 256 * 256)(8 * 3 * 6 * 6) - \
        (lambda b: (b + 255) // 256 * 256)(8 * N)
    for max_T, max_U1 in ((5, 6), (6, 5), (0, 6)):   # a sample does not fit, or an empty extent
        with pytest.raises(ValueError):
            _lib.workspace_size_multiblank_padded(3, 32, max_T, max_U1, _lib.RNNT_F32, T, U, [2, 3])
    with pytest.raises(ValueError):
        _lib.loss_multiblank_padded(0x100000, 0, 6, 5, 32, 0x200000, 5, T, U, -1, [30], [2], 0.0, -1.0, 0.0, True,
                                    "sum", 0x300000, 0x400000, 0x500000, 0x600000, 1 << 20, 0)


def test_noalloc_refusals_before_any_device_work():
    """rnnt_loss_fused_noalloc refuses on the host, before enqueuing anything: more than 64 samples (its schedule
    travels as kernel arguments), and a batch whose workspace exceeds the fixed scratch of 128 MiB.  The device
    pointers are never dereferenced on these paths."""
    T = np.full(65, 3, np.int32)
    U = np.full(65, 1, np.int32)
    with pytest.raises(ValueError):
        _lib.loss_fused_noalloc(0x100000, _lib.RNNT_F32, int((T * (U + 1)).sum()), 8, 0x200000, 1, T, U, -1, -1.0,
                                True, "sum", 0x300000, 0x400000, 0x500000, 0, 0)
    # one lattice of 20000 x 1001 nodes: ~40 bytes of workspace per node, far beyond 128 MiB
    T1 = np.array([20000], np.int32)
    U1 = np.array([1000], np.int32)
    need = _lib.workspace_size(1, 8, 20000 * 1001, _lib.RNNT_F32, T1, U1)
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    with pytest.raises(ValueError, match="workspace too small"):
        _lib.loss_fused_noalloc(1 << 40, _lib.RNNT_F32, 20000 * 1001, 8, 0x200000, 1000, T1, U1, -1, -1.0, True,
                                "sum", 0x300000, 0x400000, 2 << 40, 0, 0)
    # the skewed workload's batch (the largest of the named ones, 64 samples) fits
    import workloads
    Ts, Us = workloads.lengths("skewed")[:2]
    assert _lib.workspace_size(len(Ts), 2048, int((Ts.astype(np.int64) * (Us + 1)).sum()), _lib.RNNT_F16, Ts,
                               Us) <= _lib.NOALLOC_SCRATCH_BYTES


def test_table_span_limit():
    """The recursions address one sample's tables with 32-bit offsets: (T+U) * max(8 * U1p, 16 * (U+1)) must stay
    below 2^31.  At U = 1023 (U1p = 1024) that allows T+U up to 131071, at U = 2047 up to 65535; at U = 10
    (U1p = 64) up to 2^31 / 512."""
    for U, limit in ((1023, 2 ** 31 // (16 * 1024)), (2047, 2 ** 31 // (16 * 2048)), (10, 2 ** 31 // 512)):
        ok_T, bad_T = limit - 1 - U, limit - U
        for T, fine in ((ok_T, True), (bad_T, False)):
            Ta, Ua = np.array([T], np.int32), np.array([U], np.int32)
            N = T * (U + 1)
            if fine:
                assert _lib.workspace_size(1, 2, N, _lib.RNNT_F32, Ta, Ua) > 0
            else:
                with pytest.raises(ValueError):
                    _lib.workspace_size(1, 2, N, _lib.RNNT_F32, Ta, Ua)


def test_workload_vocabulary_override():
    """A named workload at another vocabulary size keeps its lengths and draws its targets over the new
    non-blank classes; the multi-blank workload (whose big blanks are fixed classes) refuses one."""
    import workloads
    T, U, tg, V, blank = workloads.lengths("half")
    T2, U2, tg2, V2, blank2 = workloads.lengths("half", vocab=4097)
    assert V == 4096 and V2 == 4097 and blank2 == blank == -1
    assert (T2 == T).all() and (U2 == U).all()
    for i, u in enumerate(U2):
        assert ((tg2[i, :u] >= 0) & (tg2[i, :u] < V2 - 1)).all()
    _, _, tgc, Vc, bc = workloads.lengths("char", vocab=31)
    assert Vc == 31 and bc == 0 and all(((tgc[i, :u] >= 1) & (tgc[i, :u] < 31)).all()
                                         for i, u in enumerate(workloads.lengths("char")[1]))
    with pytest.raises(ValueError):
        workloads.lengths("multiblank", vocab=2000)
