"""Benchmark of the KDA chunked forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one kda_fwd call (every kernel of the forward pass) over the
throughput headline workload: B=1, T=32768, H=96, K=V=128, bf16 q/k/v/raw_gate
and raw_beta ~N(0,1), A_log ~U(0, ln 16), dt_bias ~N(0, 0.1), lower_bound -5,
scale K^-0.5, a zero fp32 initial state, final state written.  Inputs are
synthetic (seeded, tests/workloads.py) and resident in HBM before timing
starts.  Prints one JSON line.

Roofline: the forward kernel is HBM-bound.  Its algorithmic traffic is
1282 bytes per head-token (q, k, v, raw_gate: 4 x 128 x 2 B; raw_beta 2 B;
out 128 x 2 B) plus 2 x 64 KiB of fp32 state I/O per (sequence, head); the
achieved rate is that byte count divided by the average device time of one
forward (its intra-chunk and inter-chunk kernels back to back), measured with
HIP events recorded on the launch stream around every timed launch.  ``traffic`` is the measured HBM bytes per launch from rocprofv3
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
KERNEL_SRCS = [os.path.join(ROOT, "chunked_gated_delta_amd", "csrc", f)
               for f in ("kda_common.h", "kda_host.h", "kda_intra.hip", "kda_inter.hip", "kda_api.hip")] + [
    os.path.join(ROOT, "chunked_gated_delta_amd", "build.py")]  # compile flags shape the kernels too
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kda_fwd_c3_traffic.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch from the committed counter summary, if still current."""
    try:
        with open(TRAFFIC_FILE) as f:
            doc = json.load(f)
    except (OSError, ValueError):
        return None
    if doc.get("kernel_source_sha256") != kernel_source_hash():
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


def write_traffic(fwd_fetch, fwd_write, copy_fetch, copy_write, copy_bytes=2 << 30):
    """Turn four rocprofv3 --pmc counter CSVs (FETCH_SIZE / WRITE_SIZE, KiB per
    dispatch) of this benchmark and of --copy-calibration into the traffic file.

    Each counter is scaled by what it reads for the plain copy of known size;
    the forward's figure is the average over its dispatches of each kernel."""
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
    for path, counter, fac, key in ((fwd_fetch, "FETCH_SIZE", ff, "read_bytes"),
                                    (fwd_write, "WRITE_SIZE", wf, "write_bytes")):
        for name, ks in per_kernel(path, counter).items():
            m = re.search(r"(kda_\w+_kernel)", name)
            if not m:
                continue
            short = m.group(1)
            kernels.setdefault(short, {})[key] = sum(ks) / len(ks) * 1024.0 * fac
    total = sum(v.get("read_bytes", 0.0) + v.get("write_bytes", 0.0) for v in kernels.values())
    doc = {"workload": "kda_fwd B=1 T=32768 H=96 K=V=128 (bench.py defaults)",
           "kernel_source_sha256": kernel_source_hash(),
           "hbm_bytes_per_launch": total,
           "kernels": kernels,
           "calibration": {"copy_bytes": copy_bytes, "fetch_size_factor": ff,
                           "write_size_factor": wf}}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print(json.dumps(doc))


def timed(fn, steps, warmup, stream):
    """Average device time (ms) of fn() over `steps` launches, HIP events on `stream`."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / steps


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
    }), flush=True)


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
                     "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": alg},
    }), flush=True)


def bench_bwd(args):
    """Backward pass (kda_bwd: the gradients of every input) on the headline
    workload, for a bf16 N(0,1) output gradient and an fp32 N(0,1) final-state
    gradient.  Roofline view: the algorithmic HBM bytes of the call are the
    inputs q, k, v, raw_gate, d_out (5 x 128 x 2 B per head-token) and raw_beta
    (2 B), the outputs dq, dk, dv, d_raw_gate (4 x 128 x 2 B) and d_raw_beta
    (2 B), plus the initial state, final-state gradient and initial-state
    gradient (3 x 64 KiB fp32 per (sequence, head))."""
    import torch

    import chunked_gated_delta_amd as kda
    import workloads

    x = workloads.c3_headline(T=args.T, H=args.H)
    x.initial_state = torch.zeros(1, x.H, x.K, x.V, dtype=torch.float32)
    dev = torch.device("cuda:0")
    d = lambda t: t.to(dev)  # noqa: E731
    q, k, v, g, b, al, dt, init = (d(t) for t in (x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.A_log, x.dt_bias,
                                                  x.initial_state))
    gen = torch.Generator().manual_seed(9)
    d_out = d(torch.randn(1, x.T, x.H, x.V, generator=gen).to(torch.bfloat16))
    d_fin = d(torch.randn(1, x.H, x.K, x.V, generator=gen))
    dq, dk, dg = torch.empty_like(q), torch.empty_like(k), torch.empty_like(g)
    dv, db = torch.empty_like(v), torch.empty_like(b)
    dA, ddt, dinit = torch.empty_like(al), torch.empty_like(dt), torch.empty_like(init)
    ws = torch.empty(kda.kda_bwd_workspace_size(x.T, x.H, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    ms = timed(lambda: kda.kda_bwd(q, k, v, g, b, x.scale, d_out, dq, dk, dv, dg, db, dA, ddt, ws, al, dt,
                                   x.lower_bound, initial_state=init, d_final=d_fin, d_initial_state=dinit,
                                   stream=sh), args.steps, args.warmup, stream)
    # the same gradients on the records a forward call left in this workspace
    out, fin = torch.empty_like(v), torch.empty_like(init)
    kda.kda_fwd(q, k, v, g, b, x.scale, out, ws, al, dt, x.lower_bound, init, fin, stream=sh)
    ms_reuse = timed(lambda: kda.kda_bwd_ex(q, k, v, g, b, x.scale, d_out, dq, dk, dv, dg, db, dA, ddt, ws, al,
                                            dt, x.lower_bound, initial_state=init, d_final=d_fin,
                                            d_initial_state=dinit, flags=kda.FLAG_REUSE_RECORDS, stream=sh),
                     args.steps, args.warmup, stream)
    ht = x.T * x.H
    alg = ht * (9 * 128 * 2 + 2 * 2) + 3 * x.H * STATE_BYTES
    gbs = alg / (ms / 1e3) / 1e9
    print(json.dumps({
        "metric": "KDA backward (all input gradients) head-tokens/s", "value": ht / (ms / 1e3),
        "ms_reusing_forward_records": ms_reuse,
        "unit": "head-tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "dtype": "fp32 compute, bf16 io", "data": "synthetic",
        "config": {"workload": f"kda_bwd B=1 T={x.T} H={x.H} K=V=128 chunk=64 lower_bound=-5, "
                               "output and final-state gradients given"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": alg},
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--T", type=int, default=32768)
    ap.add_argument("--H", type=int, default=96)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=96)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--decode", type=int, default=0,
                    help="time the decode step for this many sequences (T=1) instead")
    ap.add_argument("--bwd", action="store_true", help="time the backward pass (kda_bwd) instead")
    ap.add_argument("--kcp-shards", type=int, default=0,
                    help="time the split-sequence path with this many shards instead")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FWD_FETCH", "FWD_WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="rocprofv3 counter_collection.csv files -> profiles/kda_fwd_c3_traffic.json")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
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

    import torch

    import chunked_gated_delta_amd as kda
    import workloads

    x = workloads.c3_headline(T=args.T, H=args.H)
    x.initial_state = torch.zeros(1, x.H, x.K, x.V, dtype=torch.float32)
    dev = torch.device("cuda:0")
    d = lambda t: None if t is None else t.to(dev)  # noqa: E731
    q, k, v, g, b = d(x.q), d(x.k), d(x.v), d(x.raw_gate), d(x.raw_beta)
    al, dt, init = d(x.A_log), d(x.dt_bias), d(x.initial_state)
    cu = torch.tensor([0, x.T], dtype=torch.int32, device=dev)
    out = torch.empty_like(v)
    fin = torch.empty_like(init)
    ws = torch.empty(kda.kda_workspace_size(x.T, x.H, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream

    def step():
        kda.kda_fwd(q, k, v, g, b, x.scale, out, ws, al, dt, x.lower_bound, init, fin, cu,
                    stream=sh)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    avg_kern_s = sum(kern_ms) / len(kern_ms) / 1e3
    ms_per_step = wall / args.steps * 1e3
    head_tokens = x.B * x.T * x.H
    value = head_tokens / (wall / args.steps)

    alg_bytes = head_tokens * BYTES_PER_HEAD_TOKEN + 2 * x.N * x.H * STATE_BYTES
    achieved = alg_bytes / avg_kern_s / 1e9
    flops = head_tokens * algorithmic_flops_per_head_token()
    line = {
        "metric": "KDA fwd head-tokens/s at H=96 T=32K bf16; % of MFMA/HBM roofline",
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
        "config": {"workload": f"kda_fwd B=1 T={x.T} H={x.H} K=V=128 chunk=64 lower_bound=-5 "
                               "zero initial state, final state written",
                   "B": 1, "T": x.T, "H": x.H, "K": 128, "V": 128},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "kernel": "kda_fwd (intra-chunk + inter-chunk kernels, one forward)",
                     "avg_kernel_ms": avg_kern_s * 1e3,
                     "algorithmic_bytes_per_launch": alg_bytes},
        "mfma": {"achieved_tflops": flops / avg_kern_s / 1e12, "peak_tflops": BF16_DENSE_TFLOPS,
                 "frac": flops / avg_kern_s / 1e12 / BF16_DENSE_TFLOPS,
                 "algorithmic_flops_per_launch": flops},
    }
    if not args.no_cpu_baseline:
        heads = list(range(min(args.cpu_heads, x.H)))
        line["cpu_baseline"] = cpu_baseline(x, heads)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
