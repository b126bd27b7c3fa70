#!/usr/bin/env python3
"""Throughput of the fused RNN-T loss (forward + backward) on one MI355X.

One step is one ``rnnt_loss_fused`` call over one seeded synthetic batch: the
host schedule upload, the row-statistics pass, the alpha/beta recursions, the
gradient pass and the loss reduction -- every step of the hot path.  Inputs,
outputs and workspace are resident in HBM before the timed region starts.
``--workload multiblank`` times ``rnnt_multiblank_loss`` (big blanks of 2, 4
and 8 frames on the bpe shapes) the same way.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload half]

The default workload is ``half``, the largest named batch (16 samples, V =
4096, fp16 logits with fp32 arithmetic: 3.56e9 packed elements, 14.2 GB of
one-read-one-write traffic per step).  Prints one JSON line.  ``value`` is
packed logits elements per second (N*V per step / time per step); the line
also carries the effective HBM bandwidth of the whole step, the roofline of
the dominant kernel (its algorithmic bytes per step over its device time per
step, measured with HIP events around each of its launches on the stream the
launch runs on), the host time to schedule a batch whose plan is not cached,
and the fp64 CPU oracle timed on a bounded sample of the same batch on every
core available to this process, plus one-thread oracle rates on the tiny,
char and bpe workloads.

``--copy-calibration`` instead runs a plain device-to-device copy of known
size, so that rocprofv3's FETCH_SIZE / WRITE_SIZE can be scaled to bytes.
"""
import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "packed logits elements/s (fwd+bwd) & effective HBM GB/s vs peak, 1 MI355X"
PEAK_HBM_GBPS = 8000.0   # MI355X HBM3E, AMD published peak
KERNEL_SOURCE = os.path.join(ROOT, "rnn_transducer_loss_amd", "csrc", "rnnt_kernels.hip")
KERNEL_SYMBOLS = {"rowstats": "k_rowstats", "alpha_beta": "k_alpha_beta", "grad": "k_grad", "reduce": "k_reduce"}
# the multi-blank path's own passes (rnnt_multiblank_loss)
MB_KERNEL_SYMBOLS = {"rowstats": "k_mb_rows", "alpha_beta": "k_mb_sweep", "grad": "k_mb_grad", "reduce": "k_reduce"}


def esize(dtype) -> int:
    import torch
    return 2 if dtype == torch.float16 else 4


def algorithmic_bytes(w) -> dict:
    """Bytes each pass must move at minimum, and the whole path's ideal.

    Fused: the path reads the logits once and writes the gradient once
    (N*V*(s_in + s_out)); non-fused: the gradient is written once and two
    values per row are gathered.  Targets, lengths and losses are added.
    """
    s = esize(w.dtype)
    NV = w.N * w.V
    aux = w.targets.size * 4 + w.B * 4 * 3
    if w.fused:
        path = NV * (s + s) + aux
        rowstats = NV * s
        grad = NV * (s + s)
    else:
        path = NV * s + 2 * w.N * s + aux
        rowstats = 2 * w.N * s
        grad = NV * s
    return {"path": path, "rowstats": rowstats, "grad": grad}


def kernel_source_hash() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def committed_traffic(kernel: str, workload: str):
    """HBM bytes per step from a committed rocprofv3 counter summary, if it matches this kernel source."""
    want = kernel_source_hash()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        text = open(path).read()
        for block in re.findall(r"```json\n(.*?)\n```", text, flags=re.S):
            try:
                d = json.loads(block)
            except ValueError:
                continue
            if (d.get("kind") == "pmc_traffic" and d.get("kernel") == kernel and d.get("workload") == workload
                    and d.get("source_sha256_16") == want):
                return d.get("traffic_bytes_per_step")
    return None


def host_cores() -> dict:
    """The cores this process may run on (its affinity mask), the machine's count, and the cgroup CPU quota."""
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count() or 1
    quota = None
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            q, period = f.read().split()[:2]
            if q != "max":
                quota = float(q) / float(period)
    except (OSError, ValueError):
        pass
    return {"affinity": affinity, "machine": os.cpu_count(), "cgroup_quota": quota}


def cpu_baseline(w, threads: int, budget_s: float = 12.0, min_wall_s: float = 1.5, fastemit_lambda: float = 0.0):
    """The fp64 oracle with ``threads`` threads over a bounded set of the batch's samples.

    Samples go out one per thread in batch order until ``budget_s`` of wall time is spent; when the whole batch
    takes less than ``min_wall_s`` it is run again (whole passes) until that much time has passed, so the rate
    rests on ~10-30 s of CPU work.
    """
    import concurrent.futures as cf
    import numpy as np
    import oracle

    threads = max(1, int(threads))
    b = w.blank + w.V if w.blank < 0 else w.blank
    rows = (w.logit_lengths.astype(np.int64) * (w.target_lengths + 1))
    # batch order, skipping samples whose fp64 gradient would exceed 4 GiB per thread (none of the named
    # workloads has one: half's largest is ~2.9 GB)
    cand = [i for i in range(w.B) if rows[i] * w.V * 8 <= (4 << 30)]
    host = {}

    def one(i):
        T, U = int(w.logit_lengths[i]), int(w.target_lengths[i])
        if w.big_blank_durations:
            r = oracle.multiblank_sample(host[i], T, U, w.targets[i], b, w.big_blank_ids, w.big_blank_durations,
                                         w.sigma, w.fused, w.clamp, fastemit_lambda, want_grad=True)
        else:
            r = oracle.sample(host[i], T, U, w.targets[i], b, w.fused, w.clamp, want_grad=True,
                              fastemit_lambda=fastemit_lambda)
        return int(rows[i]) * w.V, r.loss

    done_elems, done_samples, passes = 0, 0, 0
    elapsed = 0.0
    with cf.ThreadPoolExecutor(threads) as ex:
        while True:
            k = 0
            while k < len(cand) and elapsed < budget_s:
                wave = cand[k:k + threads]
                k += len(wave)
                for i in wave:
                    host[i] = w.logits[w.rows(i)].cpu().numpy()
                t0 = time.perf_counter()
                for n, _ in ex.map(one, wave):
                    done_elems += n
                elapsed += time.perf_counter() - t0
                done_samples += len(wave)
                for i in wave:
                    host.pop(i, None)
            passes += 1
            if k < len(cand) or elapsed >= min_wall_s or not cand:
                break
    if done_samples == 0:
        return None
    what = (f"{passes} pass(es) over the {len(cand)} samples" if k >= len(cand)
            else f"{done_samples} of {w.B} samples")
    return {"value": done_elems / elapsed, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "sample": f"{what} of the {w.name} batch ({done_elems} packed elements), loss and full gradient, "
                      f"fp64, one sample per thread, {elapsed:.2f} s wall"}


def single_thread_oracle(names=("tiny", "char", "bpe"), budget_s: float = 4.0) -> dict:
    """The fp64 oracle on one thread (loss and full gradient) on the small named workloads: the whole batch for
    tiny and char, the samples in batch order until ``budget_s`` for bpe.  Elements/s and the sample timed."""
    import oracle
    import workloads
    out = {}
    for name in names:
        w = workloads.make(name, device="cuda")
        b = w.blank + w.V if w.blank < 0 else w.blank
        done, n_samples, t = 0, 0, 0.0
        passes = 0
        while True:
            for i in range(w.B):
                x = w.logits[w.rows(i)].cpu().numpy()
                T, U = int(w.logit_lengths[i]), int(w.target_lengths[i])
                t0 = time.perf_counter()
                oracle.sample(x, T, U, w.targets[i], b, w.fused, w.clamp, want_grad=True)
                t += time.perf_counter() - t0
                done += T * (U + 1) * w.V
                n_samples += 1
                if t >= budget_s:
                    break
            passes += 1
            if t >= 0.5 or n_samples < w.B * passes:
                break
        out[name] = {"value": done / t, "unit": "elements/s", "threads": 1,
                     "sample": f"{n_samples} sample(s) of the {name} batch in {passes} pass(es), "
                               f"{done} packed elements, {t:.2f} s"}
        del w
    return out


def host_schedule_us(rl, w, reps: int = 20) -> dict:
    """Host time to validate and schedule a batch whose plan is not cached (the longest-first order, the
    descriptors, the workspace layout), in microseconds: the median over ``reps`` workspace queries of this
    batch's lengths, each after a query with other lengths that replaces the cached plan.  Also the host time
    of one call whose plan is cached (validation and kernel launches)."""
    import numpy as np
    T, U = w.logit_lengths, w.target_lengths
    T2 = T.copy()
    T2[0] += 1
    N2 = int((T2.astype(np.int64) * (U + 1)).sum())
    code = rl._lib.RNNT_F16 if w.logits.dtype.itemsize == 2 else rl._lib.RNNT_F32
    fresh = []
    for _ in range(reps):
        rl._lib.workspace_size(w.B, w.V, N2, code, T2, U)
        t0 = time.perf_counter()
        rl._lib.workspace_size(w.B, w.V, w.N, code, T, U)
        fresh.append((time.perf_counter() - t0) * 1e6)
    return {"fresh_plan_us": round(float(np.median(fresh)), 2)}


def copy_calibration(steps: int):
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        b.copy_(a)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms_per_copy": ms,
                      "GBps_read_plus_write": 2 * n / ms / 1e6}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="half", choices=["tiny", "char", "bpe", "half", "skewed", "multiblank", "vocab5k"])
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--vocab", type=int, default=None,
                    help="the workload's lattices and lengths with another vocabulary size V (any width: rows off "
                         "16-byte boundaries, rows a little over 4 KiB, ...); not for multiblank")
    ap.add_argument("--fastemit-lambda", type=float, default=0.0,
                    help="FastEmit weight on the label-emission gradient (0: the plain loss)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one captured call (a HIP graph) instead of eager calls: the same kernels "
                         "without the per-call host work; batches of up to 64 samples, not the multi-blank path")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the loss is computed per sample and its batch is one GPU's share; "
              "run it with --gpus 1 (a multi-GPU run would shard samples with no exchange).", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(args.steps)
        return

    import rnn_transducer_loss_amd as rl
    import workloads

    print(f"bench: drawing workload {args.workload}", file=sys.stderr, flush=True)
    w = workloads.make(args.workload, seed=args.seed, device="cuda", vocab=args.vocab)
    tg = torch.from_numpy(w.targets).cuda()
    T, U = w.logit_lengths, w.target_lengths
    dev = w.logits.device
    loss = torch.empty(w.B, dtype=torch.float32, device=dev)
    red = torch.empty(1, dtype=torch.float32, device=dev)
    grad = torch.empty_like(w.logits)
    multiblank = bool(w.big_blank_durations)
    if multiblank:
        nbytes = rl._lib.workspace_size_multiblank(w.B, w.V, w.N, rl._lib.RNNT_F32 if esize(w.dtype) == 4
                                                   else rl._lib.RNNT_F16, T, U, w.big_blank_durations)
    else:
        nbytes = rl.workspace_bytes(w.logits, T, U)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    symbols = MB_KERNEL_SYMBOLS if multiblank else KERNEL_SYMBOLS

    def step():
        if multiblank:
            rl.rnnt_multiblank_fused(w.logits, tg, T, U, big_blank_ids=w.big_blank_ids,
                                     big_blank_durations=w.big_blank_durations, blank=w.blank,
                                     sigma=w.sigma, clamp=w.clamp, reduction=w.reduction,
                                     fused_log_softmax=w.fused, fastemit_lambda=args.fastemit_lambda, grad=grad,
                                     workspace=ws, loss=loss, loss_reduced=red)
        else:
            rl.rnnt_loss_fused(w.logits, tg, T, U, blank=w.blank, clamp=w.clamp, reduction=w.reduction,
                               fused_log_softmax=w.fused, grad=grad, workspace=ws, loss=loss, loss_reduced=red,
                               fastemit_lambda=args.fastemit_lambda)

    print(f"bench: N={w.N} V={w.V} B={w.B}; warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    flags = rl.device_flags(ws)
    torch.cuda.synchronize()

    run = step
    if args.graph:
        if multiblank or w.B > 64:
            print("bench: --graph needs a plain batch of at most 64 samples", file=sys.stderr)
            sys.exit(2)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        run = graph.replay

    # whole-step timing: K steps bracketed by synchronisation on both sides
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - w0) * 1e3 / args.steps
    ms = e0.elapsed_time(e1) / args.steps
    print(f"bench: {ms:.4f} ms/step (host wall {wall_ms:.4f})", file=sys.stderr, flush=True)

    # host side: the call's own host time with its plan cached (validation and launches, no synchronisation),
    # then the scheduling of a batch whose plan is not cached
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    call_us = (time.perf_counter() - t0) * 1e6 / args.steps
    torch.cuda.synchronize()
    sched = None if multiblank else host_schedule_us(rl, w)
    if sched is not None:
        sched["cached_call_us"] = round(call_us, 2)

    # per-kernel timing: HIP events around each launch, on the stream the
    # launch runs on (a step makes one or two launches of each pass, see
    # launches_per_step); times are summed per step
    rl._lib.timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt = rl._lib.timing_read()
    rl._lib.timing_enable(False)
    per_kernel = {k: (v[0] / args.steps if v[1] else None) for k, v in kt.items()}
    launches = {k: v[1] / args.steps for k, v in kt.items()}

    # secondary: the autograd round trip, rnnt_loss forward then loss.backward(), as a training step calls it
    # (its gradient buffer allocated per call by torch's caching allocator; the upstream gradient is applied by
    # the library's scaling kernel, which returns at once for a unit factor)
    autograd_ms = None
    if not multiblank and not args.graph:
        x = w.logits.detach().requires_grad_(True)

        def train_step():
            out = rl.rnnt_loss(x, tg, T, U, blank=w.blank, clamp=w.clamp, reduction=w.reduction,
                               fused_log_softmax=w.fused, fastemit_lambda=args.fastemit_lambda)
            (out.sum() if w.reduction == "none" else out).backward()
            x.grad = None
        for _ in range(args.warmup):
            train_step()
        torch.cuda.synchronize()
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(args.steps):
            train_step()
        a1.record()
        torch.cuda.synchronize()
        autograd_ms = round(a0.elapsed_time(a1) / args.steps, 5)
        del x

    ab = algorithmic_bytes(w)
    dominant = max((k for k in per_kernel if per_kernel[k] is not None), key=lambda k: per_kernel[k])
    dom_bytes = ab.get(dominant)
    roofline = None
    if dom_bytes is not None:
        ach = dom_bytes / (per_kernel[dominant] * 1e-3) / 1e9
        # the committed counters are the named workloads' own
        traffic = committed_traffic(symbols[dominant], w.name) if args.vocab is None else None
        roofline = {"bound": "hbm", "kernel": symbols[dominant], "achieved": round(ach, 1),
                    "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBPS, 4),
                    "traffic": traffic, "algorithmic_bytes_per_step": dom_bytes,
                    "kernel_ms_per_step": round(per_kernel[dominant], 5),
                    "launches_per_step": launches[dominant]}

    eff = ab["path"] / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        cores = host_cores()
        # every core of the affinity mask, unless a cgroup quota allows fewer (then more threads only share them)
        threads = cores["affinity"]
        if cores["cgroup_quota"]:
            threads = max(1, min(threads, int(cores["cgroup_quota"])))
        print(f"bench: timing the CPU oracle on {threads} threads ({cores})", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, threads, fastemit_lambda=args.fastemit_lambda)
        if cpu is not None:
            cpu["host_cores"] = cores
            print("bench: timing the CPU oracle on one thread (tiny, char, bpe)", file=sys.stderr, flush=True)
            cpu["single_thread"] = single_thread_oracle()

    out = {
        "metric": METRIC,
        "value": w.N * w.V / (ms * 1e-3),
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",   # the arithmetic of the row passes; the recursion accumulates in f64

        "data": "synthetic",
        "config": {"workload": w.name + (f"@V={w.V}" if args.vocab is not None else ""), "B": w.B, "V": w.V,
                   "rows": w.N, "elements": w.N * w.V,
                   "io_dtype": "fp16" if esize(w.dtype) == 2 else "fp32", "fused_log_softmax": w.fused,
                   "reduction": w.reduction, "clamp": w.clamp, "fastemit_lambda": args.fastemit_lambda,
                   **({"big_blank_durations": list(w.big_blank_durations), "sigma": w.sigma} if multiblank else {}),
                   "T_max": int(T.max()), "U_max": int(U.max()), "recursion_dtype": "f64",
                   "launch": "hip_graph_replay" if args.graph else "eager"},
        "effective_GBps": round(eff, 1),
        "effective_frac_of_peak": round(eff / PEAK_HBM_GBPS, 4),
        "algorithmic_bytes_per_step": ab["path"],
        "kernel_ms": {k: (round(v, 5) if v is not None else None) for k, v in per_kernel.items()},
        "launches_per_step": launches,
        "host_wall_ms_per_step": round(wall_ms, 4),
        "autograd_ms_per_step": autograd_ms,
        "host_schedule": sched,
        "device_flags": flags,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
