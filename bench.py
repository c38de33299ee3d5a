#!/usr/bin/env python3
"""Benchmark of the fused vocabulary projection + cross-entropy, forward + backward.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload stress]

One step = lce_forward + lce_backward over one batch of the workload (all
shards in ring order), inputs resident in HBM before the timed region. Prints
one JSON line: tokens/s over the K timed steps, the fraction of MI355X dense
bf16 MFMA peak the step reaches, peak device bytes, a roofline figure for the
kernel with the largest share of the step (durations from HIP events recorded
around every launch on the launching stream, in a second pass of K steps),
the forward / backward split per step (median and min), the same step and
torch's bf16 GEMM on random and on all-zero data (the chip's power limit makes
the MFMA rate depend on the data), and the CPU oracle timed on a bounded
sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused linear-CE fwd+bwd tokens/s on 1 MI355X; % bf16 MFMA peak; peak HBM bytes"
PEAK_BF16_TFLOPS = 2516.6      # dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk/CU
PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "memory_bounded_vocabulary_amd", "csrc")


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".hpp", ".cpp")):
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed PMC summary, if it was taken on this source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rows = json.load(f)
    sha = kernel_source_sha()
    for r in rows:
        if r.get("kernel") == kernel and r.get("workload") == workload and r.get("source_sha") == sha:
            return r.get("hbm_bytes_per_launch")
    return None


def cpu_baseline(batch, target_s: float):
    """The oracle as it stands, on the first n' tokens of the same batch (full H, V, P)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        cores = int(info[0]["num_threads"]) if info else None
        blas = info[0].get("internal_api") if info else None
    except Exception:  # pragma: no cover
        cores, blas = None, None
    w = batch.workload
    x_all = batch.hidden
    wt = oracle.bf16_to_f64(batch.weight)

    def run(n, reps=1):
        x = oracle.bf16_to_f64(x_all[:n])
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.cross_entropy(x, wt, batch.targets[:n])
        return time.perf_counter() - t0

    # The oracle works in blocks of rows, and each block pays a pass over the
    # V x H gradient whatever its row count, so the sample starts at one full
    # block of rows; it grows geometrically, at most 4x per run, until one run
    # takes about half the target; if the whole batch takes less than that,
    # it is repeated.
    n = max(8, min(w.n_tokens, (1 << 26) // w.vocab))
    t = run(n)
    print(f"[bench] oracle sample: {n} tokens in {t:.1f} s", file=sys.stderr, flush=True)
    while n < w.n_tokens and t < 0.5 * target_s:
        n = min(w.n_tokens, int(n * min(4.0, max(1.5, 0.8 * target_s / max(t, 1e-3)))))
        t = run(n)
        print(f"[bench] oracle sample: {n} tokens in {t:.1f} s", file=sys.stderr, flush=True)
    reps = 1
    if n == w.n_tokens and t < 0.5 * target_s:
        reps = max(1, int(target_s / max(t, 1e-3)))
        t = run(n, reps)
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    # the forward alone on the same sample, once, for the split (the oracle's
    # forward forms the same full logit rows without the gradient products)
    x = oracle.bf16_to_f64(x_all[:n])
    t0 = time.perf_counter()
    oracle.cross_entropy(x, wt, batch.targets[:n], grad=False)
    t_fwd = time.perf_counter() - t0
    del np, x
    what = f"first {n} of {w.n_tokens} tokens" if n < w.n_tokens else f"all {n} tokens ({reps} passes)"
    return {"value": n * reps / t, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{what} of the {w.name} batch at full H={w.hidden}, V={w.vocab}, P={w.n_shards}; "
                      f"float64 numpy/BLAS, forward+backward, {t:.1f} s",
            "forward_tokens_per_s": round(n / t_fwd, 1),
            "backward_tokens_per_s": round(n / max(t / reps - t_fwd, 1e-9), 1),
            "blas": blas, "cpu": cpu, "affinity_cores": len(os.sched_getaffinity(0))}


def sclk_reader(dev_index: int):
    """A callable returning the GPU's current shader clock in MHz (the starred
    level of the amdgpu driver's pp_dpm_sclk for the device's PCI function), or
    None where that file cannot be read."""
    import glob
    import torch
    try:
        pr = torch.cuda.get_device_properties(dev_index)
        bdf = "%04x:%02x:%02x.0" % (pr.pci_domain_id, pr.pci_bus_id, pr.pci_device_id)
    except Exception:
        return None
    path = None
    for dev in glob.glob("/sys/class/drm/card*/device"):
        try:
            with open(os.path.join(dev, "uevent")) as f:
                if f"PCI_SLOT_NAME={bdf}" in f.read():
                    path = os.path.join(dev, "pp_dpm_sclk")
                    break
        except OSError:
            continue
    if path is None:
        return None

    def read():
        try:
            with open(path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        return float(line.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz"))
        except (OSError, ValueError, IndexError):
            return None
        return None
    return read if read() is not None else None


class ClockSampler:
    """Samples the shader clock every few milliseconds on a host thread."""

    def __init__(self, reader, period_s: float = 0.002):
        import threading
        self.reader, self.period, self.samples = reader, period_s, []
        self._stop = threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True) if reader else None

    def _run(self):
        while not self._stop.is_set():
            v = self.reader()
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        self._t0 = time.perf_counter()
        if self._t:
            self._t.start()
        return self

    def __exit__(self, *exc):
        self._window = time.perf_counter() - self._t0
        if self._t:
            self._stop.set()
            self._t.join()

    def summary(self):
        if not self.samples:
            return None
        v = sorted(self.samples)
        # the driver's level is an average over a few milliseconds: meaningful
        # for a window of about 100 ms or more
        return {"source": "pp_dpm_sclk", "samples": len(v), "window_s": round(self._window, 2),
                "median_mhz": round(v[len(v) // 2], 1), "min_mhz": round(v[0], 1), "max_mhz": round(v[-1], 1)}


def _time_steps(fn, args, dev):
    import torch
    for _ in range(args.warmup):
        fn()
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        fn()
    e1.record()
    torch.cuda.synchronize(dev)
    return e0.elapsed_time(e1) / args.steps


def variants(lce, hidden, shards, targets, d_hidden, d_shards, dloss, args, out, dev):
    """The same step through other entry points of the library:
    * rounds: lce_fwd_round x P, lce_fwd_finish, lce_bwd_round x P, as one rank of
      a ring calls them (round k holds shard (P - k) mod P);
    * bf16_grads: lce_forward + lce_backward with bf16 gradient outputs."""
    import torch
    n, h = hidden.shape
    p = len(shards)
    v = p * shards[0].shape[0]
    dims = lce.make_dims(n, h, v, p)
    ws = lce.alloc_workspace(n, h, v, p, dev)
    order = [(p - k) % p for k in range(p)]

    def rounds():
        for k, s in enumerate(order):
            lce.fwd_round(dims, k, s, hidden, shards[s], targets, ws)
        _, lse = lce.fwd_finish(dims, targets, ws)
        for k, s in enumerate(order):
            lce.bwd_round(dims, k, s, hidden, shards[s], targets, lse, dloss, d_hidden, d_shards[s], False, ws)

    ws16 = lce.alloc_workspace(n, h, v, p, dev, flags=lce.FLAG_BF16_GRADS)
    dx16 = torch.empty((n, h), dtype=torch.bfloat16, device=dev)
    dw16 = [torch.empty_like(s) for s in shards]

    def bf16_grads():
        _, lse = lce.forward(hidden, shards, targets, workspace=ws16)
        lce.backward(hidden, shards, targets, lse, dloss, workspace=ws16, d_hidden=dx16, d_shards=dw16,
                     grad_dtype=torch.bfloat16)

    res = {}
    for name, fn in (("rounds", rounds), ("bf16_grads", bf16_grads)):
        ms = _time_steps(fn, args, dev)
        res[name] = {"ms_per_step": round(ms, 4), "tokens_per_s": round(n / (ms / 1e3), 1),
                     "mfma_frac": round(8.0 * n * h * v / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "vs_whole_pass": round(ms / out["ms_per_step"], 4)}
    del ws, ws16, dx16, dw16
    return res


def power_context(lce, hidden, shards, targets, ws, dloss, d_hidden, d_shards, dev, window_ms: float = 300.0):
    """How far the chip's power limit, rather than the schedule, sets the MFMA
    rate. The same step of this library, on the workload's random inputs and
    on all-zero inputs of the same shapes (same targets, same launches, same
    memory traffic; only the bits the MFMA pipes and the data paths toggle
    differ), alternated random / zero / random / zero; and torch's bf16 GEMM
    (hipBLASLt) at 8192^3 on random N(0, 1) operands and on zeros. Each entry
    gives the rate as a fraction of the published dense bf16 peak and the
    shader clock sampled meanwhile (each measurement repeats its step for
    about window_ms, at least 3 times, so the driver's clock average covers it)."""
    import torch
    n, h = hidden.shape
    v = len(shards) * shards[0].shape[0]
    zx = torch.zeros_like(hidden)
    zw = [torch.zeros_like(s) for s in shards]

    def one(x, w, e):
        e[0].record()
        _, lse = lce.forward(x, w, targets, workspace=ws)
        e[1].record()
        lce.backward(x, w, targets, lse, dloss, workspace=ws, d_hidden=d_hidden, d_shards=d_shards)
        e[2].record()

    def lib(x, w):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        one(x, w, e)  # warm-up, and the step's length
        torch.cuda.synchronize(dev)
        reps = max(3, min(400, int(window_ms / max(e[0].elapsed_time(e[2]), 1e-3)) + 1))
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
        with ClockSampler(sclk_reader(0)) as clk:
            for e in ev:
                one(x, w, e)
            torch.cuda.synchronize(dev)
        fwd = sum(e[0].elapsed_time(e[1]) for e in ev) / reps
        bwd = sum(e[1].elapsed_time(e[2]) for e in ev) / reps
        c = clk.summary()
        return {"reps": reps, "fwd_ms": round(fwd, 4), "bwd_ms": round(bwd, 4),
                "fwd_frac": round(2.0 * n * h * v / (fwd / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "step_frac_8nhv": round(8.0 * n * h * v / ((fwd + bwd) / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "sclk_median_mhz": c["median_mhz"] if c else None}

    runs = {"random": [], "zeros": []}
    for _ in range(2):
        runs["random"].append(lib(hidden, shards))
        runs["zeros"].append(lib(zx, zw))
    del zx, zw

    def best(rs):
        return min(rs, key=lambda r: r["fwd_ms"] + r["bwd_ms"])

    m = 8192
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    a = torch.randn((m, m), device=dev, dtype=torch.float32, generator=g).to(torch.bfloat16)
    b = torch.randn((m, m), device=dev, dtype=torch.float32, generator=g).to(torch.bfloat16)
    za, zb = torch.zeros_like(a), torch.zeros_like(b)
    c = torch.empty_like(a)

    def gemm(x, y, iters=400):
        for _ in range(10):
            torch.mm(x, y, out=c)
        torch.cuda.synchronize(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with ClockSampler(sclk_reader(0)) as clk:
            e0.record()
            for _ in range(iters):
                torch.mm(x, y, out=c)
            e1.record()
            torch.cuda.synchronize(dev)
        ms = e0.elapsed_time(e1) / iters
        cs = clk.summary()
        tf = 2.0 * m * m * m / (ms / 1e3) / 1e12
        return {"ms": round(ms, 4), "tflops": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                "sclk_median_mhz": cs["median_mhz"] if cs else None}

    res = {"library_step_random": best(runs["random"]), "library_step_zeros": best(runs["zeros"]),
           "hipblaslt_gemm_8192_random": gemm(a, b), "hipblaslt_gemm_8192_zeros": gemm(za, zb)}
    del a, b, za, zb, c
    return res


def materialized(hidden, shards, targets, args, out, dev):
    """The plain path the method replaces, on the same inputs: the full logits
    from a bf16 linear layer, cast to fp32, torch's cross-entropy (mean over
    non-ignored tokens), gradients by autograd. A measurement beside the
    library, not a code path of it; its peak bytes and step time against the
    library's give the shape of the pages' memory/time claim."""
    import torch
    import torch.nn.functional as F
    w = torch.cat(list(shards)).detach()
    del shards
    torch.cuda.synchronize(dev)
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated(dev)
    x = hidden.detach().clone().requires_grad_(True)
    wp = w.clone().requires_grad_(True)
    x_shape, w_rows = tuple(x.shape), w.shape[0]
    tl = targets.long()
    io = torch.cuda.memory_allocated(dev) - base

    def step():
        x.grad = None
        wp.grad = None
        logits = F.linear(x, wp)
        loss = F.cross_entropy(logits.float(), tl, ignore_index=-100)
        loss.backward()
        return loss

    try:
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize(dev)
        torch.cuda.reset_peak_memory_stats(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            loss = step()
        e1.record()
        torch.cuda.synchronize(dev)
    except torch.cuda.OutOfMemoryError as e:
        # the plain path does not fit: record what it asked for
        msg = str(e).splitlines()[0]
        peak = torch.cuda.max_memory_allocated(dev) - base
        x.grad = None
        wp.grad = None
        del x, wp, w
        torch.cuda.empty_cache()
        return {"what": "bf16 linear -> fp32 cross_entropy (mean, ignore_index=-100) -> autograd; bf16 gradients",
                "out_of_memory": msg, "peak_bytes_before_failure": int(peak),
                "device_bytes": int(torch.cuda.get_device_properties(dev).total_memory),
                "full_logits_bf16_bytes": int(x_shape[0]) * int(w_rows) * 2,
                "full_logits_fp32_bytes": int(x_shape[0]) * int(w_rows) * 4,
                "lce_ms_per_step": out["ms_per_step"], "lce_transient_bytes": out["transient_bytes"]}
    ms = e0.elapsed_time(e1) / args.steps
    peak = torch.cuda.max_memory_allocated(dev) - base
    grads = x.grad.numel() * x.grad.element_size() + wp.grad.numel() * wp.grad.element_size()
    res = {
        "what": "bf16 linear -> fp32 cross_entropy (mean, ignore_index=-100) -> autograd; bf16 gradients",
        "ms_per_step": round(ms, 4),
        "tokens_per_s": round(x.shape[0] / (ms / 1e3), 1),
        "loss": float(loss.item()),
        "peak_bytes": int(peak),
        "transient_bytes": int(peak - io - grads),
        "lce_ms_per_step": out["ms_per_step"],
        "lce_transient_bytes": out["transient_bytes"],
        "time_ratio_lce_over_materialized": round(out["ms_per_step"] / ms, 4),
        "transient_reduction": round(1.0 - out["transient_bytes"] / max(1, peak - io - grads), 4),
    }
    del x, wp, w
    torch.cuda.empty_cache()
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="stress",
                    help="workload name (default: stress, the largest one that fits one GPU)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target length of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--variants", action="store_true",
                    help="also time the same step through the one-round-at-a-time calls (the ring's per-rank "
                         "sequence, default ring order) and with bf16 gradient outputs")
    ap.add_argument("--compare-materialized", action="store_true",
                    help="also time the plain materialising path (bf16 linear, fp32 cross-entropy, autograd) on "
                         "the same inputs and report its step time and peak bytes beside this library's")
    ap.add_argument("--no-power-context", action="store_true",
                    help="skip the random-vs-zero-data comparison (library step and hipBLASLt GEMM)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="copy this many MiB device-to-device once before timing (a plain copy of known size, "
                         "for scaling hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the ring across P GPUs is a "
              "design note only). Run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import memory_bounded_vocabulary_amd as lce
    import workloads

    w = workloads.WORKLOADS[args.workload]
    t0 = time.time()
    batch = workloads.make(w, seed=args.seed)
    print(f"[bench] {w.name}: N={w.n_tokens} H={w.hidden} V={w.vocab} P={w.n_shards}; "
          f"inputs drawn in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    base_alloc = torch.cuda.memory_allocated(dev)
    hidden = torch.from_numpy(batch.hidden.view(np.int16)).view(torch.bfloat16).to(dev)
    vs = w.shard_rows
    shards = [torch.from_numpy(batch.weight[s * vs:(s + 1) * vs].view(np.int16)).view(torch.bfloat16).to(dev)
              for s in range(w.n_shards)]
    targets = torch.from_numpy(batch.targets).to(dev)
    input_bytes = torch.cuda.memory_allocated(dev) - base_alloc
    d_hidden = torch.empty((w.n_tokens, w.hidden), dtype=torch.float32, device=dev)
    d_shards = [torch.empty((vs, w.hidden), dtype=torch.float32, device=dev) for _ in range(w.n_shards)]
    dloss = torch.ones((), dtype=torch.float32, device=dev)
    ws = lce.alloc_workspace(w.n_tokens, w.hidden, w.vocab, w.n_shards, dev)
    torch.cuda.synchronize(dev)

    def step():
        loss, lse = lce.forward(hidden, shards, targets, workspace=ws)
        lce.backward(hidden, shards, targets, lse, dloss, workspace=ws, d_hidden=d_hidden, d_shards=d_shards)
        return loss

    if args.copy_calibration_mib:
        # a plain device-to-device copy of known size from a cold source: the
        # source is written, then evicted from the caches by filling a larger
        # buffer, then copied once
        src = torch.empty(args.copy_calibration_mib << 20, dtype=torch.uint8, device=dev)
        src.fill_(1)
        evict = torch.empty(2 * src.numel(), dtype=torch.uint8, device=dev)
        evict.fill_(2)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize(dev)
        del src, dst, evict
    for _ in range(args.warmup):
        loss = step()
    torch.cuda.synchronize(dev)
    loss_val = float(loss.item())
    peak = torch.cuda.max_memory_allocated(dev) - base_alloc
    output_bytes = (w.n_tokens * w.hidden + w.vocab * w.hidden) * 4 + w.n_tokens * 4 + 4

    # launches per step, to size the event trace
    lce.trace_enable(1024)
    step()
    per_step = sum(e["launches"] for e in lce.trace_collect())
    lce.trace_enable(0)

    # the headline: K steps back to back, nothing else on the stream
    torch.cuda.synchronize(dev)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        loss = step()
    end.record()
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - wall0
    elapsed_ms = start.elapsed_time(end)

    # per-kernel durations: the same K steps again with a HIP event pair
    # recorded around every launch on the launching stream (the pairs add a
    # little time between launches, so this pass is not the headline)
    lce.trace_enable(per_step * args.steps + 16)
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start.record()
    for _ in range(args.steps):
        step()
    t_end.record()
    torch.cuda.synchronize(dev)
    traced_ms = t_start.elapsed_time(t_end)
    kernels = lce.trace_collect()
    lce.trace_enable(0)

    # per-step forward / backward split (median and min), with the shader
    # clock sampled meanwhile; a separate pass so the headline loop above has
    # no extra events in it
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    with ClockSampler(sclk_reader(0)) as clk:
        for e0, e1, e2 in ev:
            e0.record()
            loss_s, lse_s = lce.forward(hidden, shards, targets, workspace=ws)
            e1.record()
            lce.backward(hidden, shards, targets, lse_s, dloss, workspace=ws, d_hidden=d_hidden, d_shards=d_shards)
            e2.record()
        torch.cuda.synchronize(dev)
    fwd_ms = sorted(e0.elapsed_time(e1) for e0, e1, _ in ev)
    bwd_ms = sorted(e1.elapsed_time(e2) for _, e1, e2 in ev)
    step_ms = sorted(e0.elapsed_time(e2) for e0, _, e2 in ev)
    split = {"fwd_ms_median": round(fwd_ms[len(fwd_ms) // 2], 4), "fwd_ms_min": round(fwd_ms[0], 4),
             "bwd_ms_median": round(bwd_ms[len(bwd_ms) // 2], 4), "bwd_ms_min": round(bwd_ms[0], 4),
             "step_ms_median": round(step_ms[len(step_ms) // 2], 4), "step_ms_min": round(step_ms[0], 4)}
    if not np.isfinite(loss_val):
        print(f"[bench] loss is not finite: {loss_val}", file=sys.stderr)
        return 1

    n, h, v = w.n_tokens, w.hidden, w.vocab
    ms_per_step = elapsed_ms / args.steps
    executed = sum(e["flops"] for e in kernels) / args.steps  # algorithmic MFMA flops of the traced launches
    tokens_s = n / (ms_per_step / 1e3)
    flops_8 = 8.0 * n * h * v
    flops_6 = 6.0 * n * h * v
    tflops_8 = flops_8 / (ms_per_step / 1e3) / 1e12
    kern = []
    for e in kernels:
        avg_ms = e["total_ms"] / max(e["launches"], 1)
        kern.append({"kernel": e["name"], "launches_per_step": e["launches"] / args.steps,
                     "avg_ms": round(avg_ms, 5), "share": round(e["total_ms"] / traced_ms, 4),
                     "tflops": round(e["flops"] / (e["total_ms"] / 1e3) / 1e12, 2) if e["flops"] else None,
                     "gbs": round(e["bytes"] / (e["total_ms"] / 1e3) / 1e9, 1)})
    dom = max(kernels, key=lambda e: e["total_ms"])
    dom_avg_s = dom["total_ms"] / dom["launches"] / 1e3
    if dom["flops"] > 0:
        achieved = dom["flops"] / dom["launches"] / dom_avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    else:
        achieved = dom["bytes"] / dom["launches"] / dom_avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof["traffic"] = measured_traffic(dom["name"], w.name)
    roof["kernel"] = dom["name"]
    roof["avg_launch_ms"] = round(dom_avg_s * 1e3, 5)
    roof["algorithmic_per_launch"] = (dom["flops"] if dom["flops"] > 0 else dom["bytes"]) / dom["launches"]

    out = {
        "metric": METRIC,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "n_tokens": n, "hidden": h, "vocab": v, "n_shards": w.n_shards,
                   "shard_rows": vs, "ignore_frac": w.ignore_frac, "targets": w.targets, "seed": args.seed},
        # 8NHV counts every token, ignored ones included (the pages' work per
        # token); the backward leaves ignored tokens out when that saves a
        # tile, so the MFMA work executed is also reported
        "mfma_frac": round(tflops_8 / PEAK_BF16_TFLOPS, 4),
        "executed_flops_per_step": executed,
        "mfma_frac_executed": round(executed / (ms_per_step / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "valid_tokens": int(np.sum(batch.targets != -100)),
        "tflops_8nhv": round(tflops_8, 2),
        "tflops_6nhv": round(flops_6 / (ms_per_step / 1e3) / 1e12, 2),
        "peak_hbm_bytes": int(peak),
        "input_bytes": int(input_bytes),
        "output_bytes": int(output_bytes),
        "workspace_bytes": int(ws.numel()),
        "transient_bytes": int(peak - input_bytes - output_bytes),
        "full_logits_fp32_bytes": int(n) * int(v) * 4,
        "strip_fp32_bytes": int(n) * int(vs) * 4,
        "loss": loss_val,
        "wall_s": round(wall, 3),
        "timing": dict(split, traced_ms_per_step=round(traced_ms / args.steps, 4)),
        "sclk": clk.summary(),
        "roofline": roof,
        "kernels": kern,
        "source_sha": kernel_source_sha(),
        "host": platform.node(),
    }
    if args.variants:
        print("[bench] timing the per-round and bf16-gradient variants", file=sys.stderr, flush=True)
        out["variants"] = variants(lce, hidden, shards, targets, d_hidden, d_shards, dloss, args, out, dev)
    if args.compare_materialized:
        # before anything else calls torch's GEMM, so that the GEMM library's
        # workspace counts in the materialising path's transient
        print("[bench] timing the materialising path", file=sys.stderr, flush=True)
        out["materialized"] = materialized(hidden, shards, targets, args, out, dev)
    if not args.no_power_context:
        print("[bench] timing the step and a library GEMM on random and on zero data", file=sys.stderr, flush=True)
        out["power_context"] = power_context(lce, hidden, shards, targets, ws, dloss, d_hidden, d_shards, dev)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(batch, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
