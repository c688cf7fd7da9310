"""Benchmark of the KDA chunked forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c3|c2|c4]

One step is one kda_fwd call (every kernel of the forward pass).  The default
workload is the throughput headline (--config c3): B=1, T=32768, H=96,
K=V=128, bf16 q/k/v/raw_gate and raw_beta ~N(0,1), A_log ~U(0, ln 16),
dt_bias ~N(0, 0.1), lower_bound -5, scale K^-0.5, a zero fp32 initial state,
final state written.  --config c2 is one tensor-parallel rank's share (B=2,
T=4096, H=12, initial states ~N(0, 0.1)); --config c4 the packed varlen batch
(16 sequences of U[1, 8192] tokens, H=32, per-sequence initial states).
Inputs are synthetic (seeded, tests/workloads.py) and resident in HBM before
timing starts.  Prints one JSON line.

Timing: W untimed warm-up steps (default 20: after only 3, the timed C3
steps took about 1 % longer on the wall clock, 2.63 against 2.61 ms, while
the per-launch event times matched), then K timed steps between two device
synchronisations (`value` and `ms_per_step` come from that wall clock), each
launch also bracketed by HIP events on its stream; the roofline uses the
median of those per-launch event times.  A workload whose inputs and outputs
fit in the 256 MB Infinity Cache (C2) is run cold: 512 MB are written
between launches (outside the events), and `value` then comes from the median
event time.  The loaded shader clock is sampled while the forward runs back to
back and reported with its fraction of the maximum; a fraction below 0.70
marks the line (`clock.gate`), since such a row measures the power cap rather
than the kernel.

Roofline: the forward kernel is HBM-bound.  Its algorithmic traffic is
1282 bytes per head-token (q, k, v, raw_gate: 4 x 128 x 2 B; raw_beta 2 B;
out 128 x 2 B) plus 2 x 64 KiB of fp32 state I/O per (sequence, head); the
achieved rate is that byte count divided by the median device time of one
forward.  ``traffic`` is the measured HBM bytes per launch from rocprofv3
FETCH_SIZE / WRITE_SIZE counters (profiles/), reported only while the kernel
source is unchanged since the counters were taken.

cpu_baseline: the fp64 CPU oracle (test infrastructure) timed on the host's
cores over a bounded sample of the same workload.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path[:0] = [ROOT, os.path.join(ROOT, "tests")]

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
BF16_DENSE_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA, published
BYTES_PER_HEAD_TOKEN = 4 * 128 * 2 + 2 + 128 * 2
STATE_BYTES = 128 * 128 * 4
_CSRC = os.path.join(ROOT, "chunked_gated_delta_amd", "csrc")
_FWD_SRCS = ("kda_common.h", "kda_host.h", "kda_intra.hip", "kda_inter.hip", "kda_chain.h", "kda_chain.hip",
             "kda_api.hip")
# the sources whose kernels each mode's counters measure (the build script too:
# compile flags shape the kernels)
KERNEL_SRCS = {
    "fwd": _FWD_SRCS,
    "single": _FWD_SRCS,
    "bwd": _FWD_SRCS + ("kda_bwd.h", "kda_bwd_dev.h", "kda_bwd.hip", "kda_bwd_grad.hip"),
    "decode": ("kda_common.h", "kda_decode.hip"),
}
# rocprofv3 FETCH_SIZE / WRITE_SIZE summaries per mode (--write-traffic writes them)
TRAFFIC_FILES = {
    "fwd": os.path.join(ROOT, "profiles", "kda_fwd_c3_traffic.json"),
    "single": os.path.join(ROOT, "profiles", "kda_fwd_c3_single_launch_traffic.json"),
    "bwd": os.path.join(ROOT, "profiles", "kda_bwd_c3_traffic.json"),
    "decode": os.path.join(ROOT, "profiles", "kda_decode_B64_H96_traffic.json"),
}
WORKLOADS = {
    "fwd": "kda_fwd B=1 T=32768 H=96 K=V=128 (bench.py defaults)",
    "single": "kda_fwd B=1 T=32768 H=96 K=V=128 (bench.py defaults, --single-launch)",
    "bwd": "kda_bwd B=1 T=32768 H=96 K=V=128 (bench.py --bwd)",
    "decode": "kda_decode B=64 T=1 H=96 K=V=128 (bench.py --decode 64)",
}


def kernel_source_hash(mode="fwd") -> str:
    h = hashlib.sha256()
    for path in [os.path.join(_CSRC, f) for f in KERNEL_SRCS[mode]] + [
            os.path.join(ROOT, "chunked_gated_delta_amd", "build.py")]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(mode="fwd"):
    """HBM bytes per launch (call) from the committed counter summary of `mode`, if
    its kernel sources still hash to the value stored with it."""
    try:
        with open(TRAFFIC_FILES[mode]) as f:
            doc = json.load(f)
    except (OSError, ValueError):
        return None
    if doc.get("kernel_source_sha256") != kernel_source_hash(mode):
        return None
    return doc.get("hbm_bytes_per_launch")


def algorithmic_flops_per_head_token(C=64, K=128, V=128):
    # triangular-aware count of the chunk algebra (A_kk, A_qk, T, W, U, D, O, S update)
    return (C - 1) * K + (C + 1) * K + C * C / 3 + (C + 1) * K + (C + 1) * V + 3 * 2 * K * V \
        + (C + 1) * V


def cpu_baseline(x, heads):
    """Time the oracle on `heads` of the workload (all tokens)."""
    from oracle import oracle_fwd, oracle_threads

    t0 = time.perf_counter()
    oracle_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias,
               x.lower_bound, x.initial_state, x.cu_seqlens, heads=heads, want_final=True)
    dt = time.perf_counter() - t0
    ht = x.B * x.T * len(heads)
    cores = oracle_threads()  # before the one-thread run below changes the OpenMP default
    # the same recurrence on one host thread, over the first head only
    t1 = time.perf_counter()
    oracle_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias,
               x.lower_bound, x.initial_state, x.cu_seqlens, heads=heads[:1], want_final=True, threads=1)
    dt1 = time.perf_counter() - t1
    return {"value": ht / dt, "unit": "head-tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 token recurrence over heads 0..{len(heads) - 1} of {x.H}, all "
                      f"{x.T} tokens ({ht} head-tokens, {dt:.1f} s)",
            "single_core_value": x.B * x.T / dt1,
            "single_core_sample": f"head 0, all {x.T} tokens, one thread ({dt1:.2f} s)"}


def cpu_baseline_bwd(x, T_sample, heads):
    """Time the gradient oracle (fp64 autograd through the token recurrence) on the
    first T_sample tokens of `heads`: it is orders of magnitude slower than the C
    recurrence, so the sample is small; the rate is head-tokens of gradients per second."""
    import torch

    from oracle.grad import oracle_bwd

    sl = lambda t: t[:1, :T_sample][:, :, heads].contiguous()  # noqa: E731  (the first batch row)
    gen = torch.Generator().manual_seed(9)
    d_out = torch.randn(1, T_sample, len(heads), x.V, generator=gen).to(torch.bfloat16)
    t0 = time.perf_counter()
    oracle_bwd(sl(x.q), sl(x.k), sl(x.v), sl(x.raw_gate), x.raw_beta[:1, :T_sample][:, :, heads].contiguous(),
               x.scale, x.A_log[heads], x.dt_bias[heads], x.lower_bound, d_out)
    dt = time.perf_counter() - t0
    ht = T_sample * len(heads)
    return {"value": ht / dt, "unit": "head-tokens/s", "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": f"fp64 autograd of the token recurrence, heads {heads}, first {T_sample} tokens "
                      f"({ht} head-tokens, {dt:.1f} s)"}


def copy_calibration(gib: float = 2.0):
    """A plain device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch

    n = int(gib * (1 << 30)) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": n * 4, "launches": 3}))


def write_traffic(fetch_csv, write_csv, copy_fetch, copy_write, calls, mode="fwd", copy_bytes=2 << 30):
    """Turn four rocprofv3 --pmc counter CSVs (FETCH_SIZE / WRITE_SIZE, KiB per
    dispatch) of `calls` identical calls of a bench mode and of --copy-calibration
    into that mode's traffic file.

    Each counter is scaled by what it reads for the plain copy of known size.  A
    kernel's bytes per call are the sum over its dispatches divided by `calls`
    (so a kernel launched twice per call counts twice); the call's total sums the
    library's kernels."""
    import collections
    import csv

    def per_kernel(path, counter):
        acc = collections.defaultdict(float)
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                acc[(int(r["Dispatch_Id"]), r["Kernel_Name"])] += float(r["Counter_Value"])
        by = collections.defaultdict(list)
        for (_, name), kib in acc.items():
            by[name].append(kib)
        return by

    def factor(path, counter):
        runs = [k for name, ks in per_kernel(path, counter).items() if "copyBuffer" in name for k in ks]
        kib = max(runs)  # the 2 GiB copies (small runtime copies read far less)
        return copy_bytes / (kib * 1024.0)

    ff, wf = factor(copy_fetch, "FETCH_SIZE"), factor(copy_write, "WRITE_SIZE")
    kernels = {}
    for path, counter, fac, key in ((fetch_csv, "FETCH_SIZE", ff, "read_bytes"),
                                    (write_csv, "WRITE_SIZE", wf, "write_bytes")):
        for name, ks in per_kernel(path, counter).items():
            m = re.search(r"(kda_\w+_kernel(?:<[^>]*>)?)", name)
            if not m:
                continue
            kernels.setdefault(m.group(1), {})[key] = sum(ks) / calls * 1024.0 * fac
    total = sum(v.get("read_bytes", 0.0) + v.get("write_bytes", 0.0) for v in kernels.values())
    doc = {"workload": WORKLOADS[mode],
           "kernel_source_sha256": kernel_source_hash(mode),
           "calls_profiled": calls,
           "hbm_bytes_per_launch": total,
           "kernels": kernels,
           "calibration": {"copy_bytes": copy_bytes, "fetch_size_factor": ff,
                           "write_size_factor": wf}}
    with open(TRAFFIC_FILES[mode], "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print(json.dumps(doc))


def timed(fn, steps, warmup, stream, setup=None):
    """Median device time (ms) of fn() over `steps` launches, HIP events on `stream`
    (setup(), if given, runs before each launch, outside its events)."""
    import torch

    for _ in range(warmup):
        if setup:
            setup()
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        if setup:
            setup()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return median([a.elapsed_time(b) for a, b in evs])


def bench_kcp(args):
    """Split-sequence path on the headline workload: the sequence is cut into
    `args.kcp_shards` equal shards (one varlen batch); time the per-shard
    affine maps, the shard scan and the forward over the shards from the
    scanned entering states."""
    import torch

    import chunked_gated_delta_amd as kda
    import workloads

    x = workloads.c3_headline(T=args.T, H=args.H)
    n = args.kcp_shards
    dev = torch.device("cuda:0")
    d = lambda t: t.to(dev)  # noqa: E731
    q, k, v, g, b, al, dt = (d(t) for t in (x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.A_log, x.dt_bias))
    cut = torch.tensor([i * x.T // n for i in range(n + 1)], dtype=torch.int32, device=dev)
    ws = torch.empty(kda.kda_workspace_size(x.T, x.H, n), dtype=torch.uint8, device=dev)
    P = torch.empty(n, x.H, 128, 128, device=dev)
    R = torch.empty_like(P)
    starts = torch.empty_like(P)
    fin = torch.empty_like(P)
    out = torch.empty_like(v)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    t_aff = timed(lambda: kda.kda_shard_affine(q, k, v, g, b, ws, al, dt, x.lower_bound, P, R, cut, stream=sh),
                  args.steps, args.warmup, stream)
    t_scan = timed(lambda: kda.kda_shard_scan(P, R, starts, stream=sh), args.steps, args.warmup, stream)
    t_fwd = timed(lambda: kda.kda_fwd(q, k, v, g, b, x.scale, out, ws, al, dt, x.lower_bound, starts, fin, cut,
                                      stream=sh), args.steps, args.warmup, stream)
    # the same forward on the records kda_shard_affine left in the workspace
    kda.kda_shard_affine(q, k, v, g, b, ws, al, dt, x.lower_bound, P, R, cut, stream=sh)
    t_reuse = timed(lambda: kda.kda_fwd_ex(q, k, v, g, b, x.scale, out, ws, al, dt, x.lower_bound, starts, fin,
                                           cut, flags=kda.FLAG_REUSE_RECORDS, stream=sh),
                    args.steps, args.warmup, stream)
    ht = x.T * x.H
    total = t_aff + t_scan + t_reuse
    print(json.dumps({
        "metric": "KDA split-sequence (per-shard affine map + scan + forward) head-tokens/s",
        "value": ht / (total / 1e3), "unit": "head-tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"kda_shard_affine + kda_shard_scan + kda_fwd_ex (reusing the records), B=1 "
                               f"T={x.T} H={x.H} K=V=128 cut into {n} equal shards", "shards": n},
        "ms": {"shard_affine": t_aff, "shard_scan": t_scan, "forward_reusing_records": t_reuse,
               "forward_recomputing_records": t_fwd, "total": total},
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_kcp(x, n, list(range(min(4, x.H)))),
    }), flush=True)


def cpu_baseline_kcp(x, n, heads):
    """The fp64 oracle of the same split: each shard's (P, R) from the token recurrence,
    then the fp64 fold and the forward from the folded states, on `heads`."""
    import numpy as np

    from oracle import oracle_fwd, oracle_shard_affine, oracle_shard_fold, oracle_threads

    cut = np.array([i * x.T // n for i in range(n + 1)], dtype=np.int32)
    t0 = time.perf_counter()
    P, R = oracle_shard_affine(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.A_log, x.dt_bias, x.lower_bound,
                               cu_seqlens=cut, heads=heads)
    starts, _ = oracle_shard_fold(P, R)
    sub = lambda t: t[:, :, heads].contiguous()  # noqa: E731
    oracle_fwd(sub(x.q), sub(x.k), sub(x.v), sub(x.raw_gate), x.raw_beta[:, :, heads].contiguous(), x.scale,
               x.A_log[heads], x.dt_bias[heads], x.lower_bound,
               __import__("torch").from_numpy(starts.astype(np.float32)), cut)
    dt = time.perf_counter() - t0
    ht = x.T * len(heads)
    return {"value": ht / dt, "unit": "head-tokens/s", "cores": oracle_threads(), "kind": "oracle",
            "sample": f"fp64 shard maps, fold and forward over heads 0..{len(heads) - 1} of {x.H}, all "
                      f"{x.T} tokens in {n} shards ({ht} head-tokens, {dt:.1f} s)"}


def bench_decode(args):
    """Token-by-token decode step: B = args.decode sequences, T = 1, H = args.H,
    fp32 states updated in place.  HBM-bound on the state: per (sequence, head)
    the algorithmic bytes are the 2 x 64 KiB state read and write plus the
    token's q, k, v, raw_gate, out (5 x 256 B) and raw_beta (2 B)."""
    import torch

    import chunked_gated_delta_amd as kda
    import workloads

    x = workloads.random_inputs("decode-bench", 5, args.decode, 1, args.H, init_std=0.1)
    dev = torch.device("cuda:0")
    d = lambda t: t.to(dev)  # noqa: E731
    q, k, v, g, b, al, dt, st = (d(t) for t in (x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.A_log, x.dt_bias,
                                                x.initial_state))
    out = torch.empty_like(v)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    ms = timed(lambda: kda.kda_decode(q, k, v, g, b, x.scale, out, al, dt, x.lower_bound, st, st, stream=sh),
               args.steps, args.warmup, stream)
    pairs = x.B * x.H
    alg = pairs * (2 * STATE_BYTES + 5 * 128 * 2 + 2)
    gbs = alg / (ms / 1e3) / 1e9
    print(json.dumps({
        "metric": "KDA decode step (T=1) sequence-heads/s", "value": pairs / (ms / 1e3),
        "unit": "sequence-heads/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "dtype": "fp32 state, bf16 io", "data": "synthetic",
        "config": {"workload": f"kda_decode B={x.B} T=1 H={x.H} K=V=128, in-place fp32 state"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": alg,
                     "traffic": measured_traffic("decode") if (x.B, x.H) == (64, 96) else None},
        "cpu_baseline": None if args.no_cpu_baseline else dict(
            cpu_baseline(x, list(range(x.H))), unit="sequence-heads/s"),
    }), flush=True)


def bench_bwd(args):
    """Backward pass (kda_bwd: the gradients of every input) on the --config
    workload, for a bf16 N(0,1) output gradient and an fp32 N(0,1) final-state
    gradient.  Roofline view: the algorithmic HBM bytes of the call are the
    inputs q, k, v, raw_gate, d_out (5 x 128 x 2 B per head-token) and raw_beta
    (2 B), the outputs dq, dk, dv, d_raw_gate (4 x 128 x 2 B) and d_raw_beta
    (2 B), plus the initial state, final-state gradient and initial-state
    gradient (3 x 64 KiB fp32 per (sequence, head)).  Workloads under 256 MB
    of those bytes (C2) run cold, as in the forward mode."""
    import torch

    import chunked_gated_delta_amd as kda
    import workloads

    if args.config == "c3":
        x = workloads.c3_headline(T=args.T, H=args.H)
        x.initial_state = torch.zeros(1, x.H, x.K, x.V, dtype=torch.float32)
    elif args.config == "c2":
        x = workloads.c2_tp_share()
    else:
        x = workloads.c4_varlen()
    dev = torch.device("cuda:0")
    d = lambda t: None if t is None else t.to(dev)  # noqa: E731
    q, k, v, g, b, al, dt, init, cu = (d(t) for t in (x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.A_log,
                                                      x.dt_bias, x.initial_state, x.cu_seqlens))
    gen = torch.Generator().manual_seed(9)
    d_out = d(torch.randn(x.B, x.T, x.H, x.V, generator=gen).to(torch.bfloat16))
    d_fin = d(torch.randn(x.N, x.H, x.K, x.V, generator=gen))
    dq, dk, dg = torch.empty_like(q), torch.empty_like(k), torch.empty_like(g)
    dv, db = torch.empty_like(v), torch.empty_like(b)
    dA, ddt, dinit = torch.empty_like(al), torch.empty_like(dt), torch.empty_like(init)
    ws = torch.empty(kda.kda_bwd_workspace_size(x.B * x.T, x.H, x.N), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    ht = x.B * x.T * x.H
    alg = ht * (9 * 128 * 2 + 2 * 2) + 3 * x.N * x.H * STATE_BYTES
    cold = alg < (256 << 20)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if cold else None
    evict = (lambda: flush.zero_()) if cold else (lambda: None)  # noqa: E731
    ms = timed(lambda: kda.kda_bwd(q, k, v, g, b, x.scale, d_out, dq, dk, dv, dg, db, dA, ddt, ws, al, dt,
                                   x.lower_bound, initial_state=init, d_final=d_fin, d_initial_state=dinit,
                                   cu_seqlens=cu, stream=sh), args.steps, args.warmup, stream, setup=evict)
    ms_reuse = None
    if not args.no_reuse:
        # the same gradients on the records a forward call left in this workspace
        out, fin = torch.empty_like(v), torch.empty_like(init)

        def forward_first():
            # the backward's factor record is written over the forward's records,
            # so every timed call gets a fresh forward first, outside its events
            kda.kda_fwd_ex(q, k, v, g, b, x.scale, out, ws, al, dt, x.lower_bound, init, fin, cu,
                           flags=kda.FLAG_KEEP_RECORDS, stream=sh)
            evict()

        ms_reuse = timed(lambda: kda.kda_bwd_ex(q, k, v, g, b, x.scale, d_out, dq, dk, dv, dg, db, dA, ddt, ws,
                                                al, dt, x.lower_bound, initial_state=init, d_final=d_fin,
                                                d_initial_state=dinit, cu_seqlens=cu,
                                                flags=kda.FLAG_REUSE_RECORDS, stream=sh),
                         args.steps, args.warmup, stream, setup=forward_first)
    gbs = alg / (ms / 1e3) / 1e9
    headline = args.config == "c3" and (x.T, x.H) == (32768, 96)
    workload = {"c3": f"kda_bwd B=1 T={x.T} H={x.H} K=V=128 chunk=64 lower_bound=-5",
                "c2": "kda_bwd B=2 T=4096 H=12 K=V=128 (one TP8 rank's share of H=96) lower_bound=-5, "
                      "initial state, run cold (MALL flushed between launches)",
                "c4": f"kda_bwd varlen: 16 packed sequences of U[1, 8192] tokens ({x.B * x.T} in all), H=32, "
                      "K=V=128, lower_bound=-5, per-sequence initial states"}[args.config]
    print(json.dumps({
        "metric": "KDA backward (all input gradients) head-tokens/s", "value": ht / (ms / 1e3),
        "ms_reusing_forward_records": ms_reuse,
        "unit": "head-tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "dtype": "fp32 compute, bf16 io", "data": "synthetic",
        "config": {"workload": workload + ", output and final-state gradients given",
                   "B": x.B, "T": x.T, "H": x.H, "N": x.N},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": alg,
                     "traffic": measured_traffic("bwd") if headline else None},
        "cold": cold,
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_bwd(x, 256, [0, 1]),
    }), flush=True)


def median(xs):
    ys = sorted(xs)
    n = len(ys)
    return ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])


def read_sclk():
    """(current, maximum) shader clock in MHz from the driver's DPM table in sysfs
    (the level marked '*' is the current one), or None where it is not readable."""
    import glob

    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            lines = open(path).read().strip().splitlines()
        except OSError:
            continue
        levels, cur = [], None
        for ln in lines:
            m = re.search(r"(\d+)\s*[Mm][Hh]z", ln)
            if not m:
                continue
            levels.append(int(m.group(1)))
            if "*" in ln:
                cur = int(m.group(1))
        if levels and cur is not None:
            return cur, max(levels), path
    return None


def loaded_clock(step, seconds=1.0):
    """Sample the shader clock while `step` runs back to back for about `seconds`."""
    import threading

    import torch

    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            r = read_sclk()
            if r is not None:
                samples.append(r)
            time.sleep(0.02)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            step()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    if not samples:
        return {"sclk_mhz": None, "max_mhz": None, "frac": None,
                "gate": "not measured: no readable pp_dpm_sclk"}
    cur = median([c for c, _, _ in samples])
    mx = max(m for _, m, _ in samples)
    frac = cur / mx
    return {"sclk_mhz": cur, "max_mhz": mx, "frac": frac, "samples": len(samples), "source": samples[0][2],
            "gate": "pass" if frac >= 0.70 else "FAIL: loaded clock below 0.70 of max, row not valid"}


CONFIGS = {
    "c3": "kda_fwd B=1 T={T} H={H} K=V=128 chunk=64 lower_bound=-5 zero initial state, final state written",
    "c2": "kda_fwd B=2 T=4096 H=12 K=V=128 (one TP8 rank's share of H=96) lower_bound=-5, initial and final "
          "states, run cold (MALL flushed between launches)",
    "c4": "kda_fwd varlen: 16 packed sequences of U[1, 8192] tokens ({T} in all), H=32, K=V=128, "
          "lower_bound=-5, per-sequence initial and final states",
}


def bench_forward(args):
    import torch

    import chunked_gated_delta_amd as kda
    import workloads

    if args.config == "c3":
        x = workloads.c3_headline(T=args.T, H=args.H)
        x.initial_state = torch.zeros(1, x.H, x.K, x.V, dtype=torch.float32)
        x.cu_seqlens = torch.tensor([0, x.T], dtype=torch.int32)
    elif args.config == "c2":
        x = workloads.c2_tp_share()
    else:
        x = workloads.c4_varlen()
    dev = torch.device("cuda:0")
    d = lambda t: None if t is None else t.to(dev)  # noqa: E731
    q, k, v, g, b = d(x.q), d(x.k), d(x.v), d(x.raw_gate), d(x.raw_beta)
    al, dt, init, cu = d(x.A_log), d(x.dt_bias), d(x.initial_state), d(x.cu_seqlens)
    out = torch.empty_like(v)
    fin = torch.empty_like(init)
    ws = torch.empty(kda.kda_workspace_size(x.B * x.T, x.H, x.N), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    head_tokens = x.B * x.T * x.H
    alg_bytes = head_tokens * BYTES_PER_HEAD_TOKEN + 2 * x.N * x.H * STATE_BYTES
    cold = alg_bytes < (256 << 20)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if cold else None

    def step():
        if args.single_launch:
            kda.kda_fwd_ex(q, k, v, g, b, x.scale, out, ws, al, dt, x.lower_bound, init, fin, cu,
                           flags=kda.FLAG_SINGLE_LAUNCH, stream=sh)
        else:
            kda.kda_fwd(q, k, v, g, b, x.scale, out, ws, al, dt, x.lower_bound, init, fin, cu, stream=sh)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if cold:
            flush.zero_()
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    med_s = median(kern_ms) / 1e3
    ms_per_step = wall / args.steps * 1e3
    value = head_tokens / (med_s if cold else wall / args.steps)
    clock = loaded_clock(step) if not args.no_clock else None

    achieved = alg_bytes / med_s / 1e9
    flops = head_tokens * algorithmic_flops_per_head_token()
    headline = args.config == "c3" and x.T == 32768 and x.H == 96
    line = {
        "metric": "KDA fwd head-tokens/s at H=96 T=32K bf16; % of MFMA/HBM roofline" if headline else
                  f"KDA fwd head-tokens/s ({args.config}); % of HBM roofline",
        "value": value,
        "unit": "head-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": CONFIGS[args.config].format(T=x.B * x.T, H=x.H) +
                   ("; single-launch schedule (KDA_FLAG_SINGLE_LAUNCH)" if args.single_launch else ""),
                   "B": x.B, "T": x.T, "H": x.H, "K": 128, "V": 128, "N": x.N},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic("single" if args.single_launch else "fwd") if headline else None,
                     "kernel": "kda_fwd (every kernel of one forward)",
                     "median_kernel_ms": med_s * 1e3,
                     "mean_kernel_ms": sum(kern_ms) / len(kern_ms),
                     "min_kernel_ms": min(kern_ms),
                     "algorithmic_bytes_per_launch": alg_bytes},
        "mfma": {"achieved_tflops": flops / med_s / 1e12, "peak_tflops": BF16_DENSE_TFLOPS,
                 "frac": flops / med_s / 1e12 / BF16_DENSE_TFLOPS,
                 "algorithmic_flops_per_launch": flops},
        "clock": clock,
        "cold": cold,
    }
    if not args.no_cpu_baseline:
        heads = list(range(min(args.cpu_heads, x.H)))
        line["cpu_baseline"] = cpu_baseline(x, heads)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--T", type=int, default=32768)
    ap.add_argument("--H", type=int, default=96)
    ap.add_argument("--config", choices=["c3", "c2", "c4"], default="c3",
                    help="workload of the forward (and of --bwd): c3 headline (default), c2 one TP8 rank's "
                         "share, c4 packed varlen")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true", help="skip the loaded-clock probe")
    ap.add_argument("--cpu-heads", type=int, default=96)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--decode", type=int, default=0,
                    help="time the decode step for this many sequences (T=1) instead")
    ap.add_argument("--bwd", action="store_true", help="time the backward pass (kda_bwd) instead")
    ap.add_argument("--kcp-shards", type=int, default=0,
                    help="time the split-sequence path with this many shards instead")
    ap.add_argument("--write-traffic", nargs=6, metavar=("MODE", "CALLS", "FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="rocprofv3 counter_collection.csv files of CALLS identical calls of MODE (fwd, single, "
                         "bwd, decode) and of --copy-calibration -> that mode's traffic file under profiles/")
    ap.add_argument("--no-reuse", action="store_true",
                    help="with --bwd: skip the second timing on a preceding forward's records")
    ap.add_argument("--single-launch", action="store_true",
                    help="time kda_fwd_ex with KDA_FLAG_SINGLE_LAUNCH (the one-launch producer/chain pipeline)")
    args = ap.parse_args()
    if args.write_traffic:
        mode, calls, *files = args.write_traffic
        write_traffic(*files, calls=int(calls), mode=mode)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: only --gpus 1 is supported; the library runs on one GPU (its forward "
              "would shard heads and sequences across GPUs with no exchange, which is not built)",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.kcp_shards:
        bench_kcp(args)
        return
    if args.decode:
        bench_decode(args)
        return
    if args.bwd:
        bench_bwd(args)
        return

    bench_forward(args)


if __name__ == "__main__":
    main()
