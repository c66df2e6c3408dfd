"""Throughput of the causal dot product on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

A step is one forward (writing the final state) plus one backward (reading
it) over the whole batch of the workload, inputs resident in HBM.  W untimed
steps, then K timed steps launched back to back between device
synchronisations: `value` is K * N*H*L over that wall time.  Per-kernel
durations come from a second pass of K steps in which every launch carries its
own start/end events on the stream it runs on (the library's timing hook,
which costs host time per launch and is therefore kept out of `value`).
Prints one JSON line with the whole-job tokens*heads/s, the roofline of the
dominant kernel (algorithmic bytes, and flops, per launch / its average launch
time), a plain device copy timed in the same run, and the fp64 CPU oracle
timed on a bounded sample of the same workload's own slices on this host's
cores (all of them, and one).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# dense matrix peaks (TFLOP/s) by the type a product is defined in
MFMA_PEAK_TFS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}
METRIC = "causal-product fwd+bwd tokens·heads/s and % HBM/MFMA roofline, L=4096 E=M=64"
UNIT = "tokens·heads/s"
COUNTERS = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = ("cp_device.hpp", "cp_fwd.hpp", "cp_fwd_launch.hpp", "cp_bwd.hpp", "cp_bwd_launch.hpp", "cp_tune.hpp",
                  "cp_launch.hpp", "cp_plan.hpp")
# the sweep kernel of each call; over few slices a call is two launches, the
# segment-increment pass and then the sweeps
SWEEP_KERNEL = {"fwd": "cp_fwd_kernel", "bwd": "cp_bwd_kernel", "linattn": "cp_fwd_kernel",
                "linattn_bwd": "cp_bwd_kernel"}


def kernel_name(kind: str, launches: int) -> str:
    """The kernels of one call: the sweep, after the segment-increment pass
    (over few slices) and, in the backward, the scan of its increments."""
    before = {1: [], 2: ["cp_seg_state_kernel"], 3: ["cp_seg_state_kernel", "cp_seg_scan_kernel"]}[launches]
    return " + ".join(before + [SWEEP_KERNEL[kind]])


def kernel_digest() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "prefix_sum_causal_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w, kind: str) -> int:
    """Bytes a launch must move at minimum: read every input once, write every
    output once (plus the fp32 final state passed from forward to backward)."""
    s = 4 if w.dtype == "f32" else 2
    th = w.N * w.H * w.L
    state = w.N * w.H * w.E * w.M * 4
    if kind == "fwd":
        return th * s * (2 * w.E + 2 * w.M) + state
    if kind == "bwd":
        return th * s * (4 * w.E + 3 * w.M) + state
    if kind == "linattn":
        return th * s * (2 * w.E + 2 * w.M)
    if kind == "linattn_bwd":
        # read q, k, v, out, dO and the fp32 denominators (and the final state);
        # write dq, dk, dv
        return th * (s * (4 * w.E + 4 * w.M) + 4) + state
    raise ValueError(kind)


def algorithmic_flops(w, kind: str) -> int:
    """Flops of the recurrence itself, per call: the forward's two products of
    E*M multiply-adds per token*head (state update k v^T, read-out q^T S),
    4EM flops; the backward's five (S again, dq, the suffix state R, dk, dv),
    10EM; the normaliser adds its running sum, dot product and division
    (3E + M), and its backward runs the causal-product backward on M + 1
    columns plus the per-row terms."""
    th = w.N * w.H * w.L
    E, M = w.E, w.M
    return th * {"fwd": 4 * E * M, "bwd": 10 * E * M, "linattn": 4 * E * M + 3 * E + M,
                 "linattn_bwd": 10 * E * (M + 1) + 3 * M}[kind]


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    try:
        with open(COUNTERS) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_digest") != kernel_digest():
        return None
    entry = rec.get("kernels", {}).get(f"{workload}:{kernel}")
    return None if entry is None else entry.get("hbm_bytes_per_launch")


def copy_rate(torch, mib: int = 1024, reps: int = 5) -> dict:
    """A plain device-to-device copy of `mib` MiB (read + write, larger than
    the caches), timed with events on the current stream: the practical
    streaming rate of this GPU in the same run."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, device="cuda", dtype=torch.float32)
    dst = torch.empty_like(src)
    dst.copy_(src)
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3)
    del src, dst
    t = sorted(ts)[len(ts) // 2]
    moved = 2 * mib * (1 << 20)
    return {"GBps": moved / t / 1e9, "bytes_moved": moved, "us": t * 1e6, "what": f"torch copy_ of {mib} MiB fp32, "
            f"median of {reps}"}


def cpu_baseline(w, host, target_seconds: float = 15.0) -> dict:
    """The fp64 oracle (the recurrences the workload's calls compute) on a
    bounded sample of the workload's own (n, h) slices, scaled to
    tokens*heads/s: as many slices as the oracle has threads (one slice per
    thread), repeated for about target_seconds; and one slice on one thread."""
    import numpy as np

    import oracle

    orc = oracle.default()
    threads = orc.num_threads()
    T = min(threads, w.N * w.H)

    def take(name, n):  # host[name] holds the first slices, [slices][L][features]
        return np.ascontiguousarray(host[name][:n])

    def run(n, seconds):
        d = {k: take(k, n) for k in host}
        slices, t0 = 0, time.perf_counter()
        while True:
            if w.op.startswith("linattn"):
                orc.linattn(d["Q"], d["K"], d["V"], 1e-6, 1)
                if w.op == "linattn+bwd":
                    orc.linattn_bwd(d["Q"], d["K"], d["V"], d["dO"], 1e-6, 1)
            else:
                orc.fwd(d["Q"], d["K"], d["V"])
                if w.op == "fwd+bwd":
                    orc.bwd(d["Q"], d["K"], d["V"], d["dO"])
            slices += n
            el = time.perf_counter() - t0
            if el >= seconds:
                return slices * w.L / el, slices, el

    value, slices, el = run(T, target_seconds)
    one, slices1, el1 = run(1, max(2.0, target_seconds / 3))
    return {"value": value, "unit": UNIT, "cores": threads, "kind": "oracle",
            "sample": f"the workload's first {T} (n,h) slices at full L={w.L}, one per thread, repeated "
                      f"({slices} slice passes in {el:.1f} s), fp64 recurrences ({w.op})",
            "one_thread": {"value": one, "unit": UNIT, "cores": 1,
                           "sample": f"slice (0,0), {slices1} passes in {el1:.1f} s"}}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-steps", type=int, default=5,
                    help="after the timed region, this many more steps with every call preceded by a 1 GiB "
                         "read that evicts the caches (the 256 MB MALL included); their per-call times are "
                         "reported as cold_cache")
    ap.add_argument("--settle-steps", type=int, default=300,
                    help="after the timed region, this many untimed steps back to back, then K more timed "
                         "ones, reported as steady_state; the per-call durations (and the roofline) are taken "
                         "right after them (the GPU's clocks dip for some milliseconds after a burst of load "
                         "starts, which is where a short timed region right after a few warm-up steps falls); "
                         "0 skips it")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run one plain device-to-device copy of this many MiB first (reference for the "
                         "HBM byte counters of a profiler run)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path shards over (n, h) slices "
              "with no communication, so run it per GPU.", file=sys.stderr)
        return 2

    import torch

    import prefix_sum_causal_amd as cp
    import workloads as W

    name = args.workload or W.HEADLINE
    w = W.WORKLOADS[name]
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.dtype]
    d = W.generate(w, need_do=w.op.endswith("bwd"))
    dev = {k: torch.from_numpy(v).to("cuda").to(tdt) for k, v in d.items()}
    # the host copies of the first slices stay for the CPU baseline
    keep = min(64, w.N * w.H)
    host = {k: v.reshape((w.N * w.H,) + v.shape[2:])[:keep].copy() for k, v in d.items()}
    del d
    q, k, v = dev["Q"], dev["K"], dev["V"]
    out = torch.empty_like(v)
    state = torch.empty((w.N, w.H, w.E, w.M), device="cuda", dtype=torch.float32)
    den = torch.empty((w.N, w.H, w.L), device="cuda", dtype=torch.float32)
    zfin = torch.empty((w.N, w.H, w.E), device="cuda", dtype=torch.float32)
    if w.op.endswith("bwd"):
        g = dev["dO"]
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    # one step = the calls below, in order; kinds[i] names call i
    def fwd_call():
        if w.op == "linattn":
            cp.linear_attn_fwd(q, k, v, 1e-6, 1, out=out)
        elif w.op == "linattn+bwd":
            cp.linear_attn_fwd(q, k, v, 1e-6, 1, out=out, state_out=state, z_out=zfin, den_out=den)
        else:
            cp.causal_product_fwd(q, k, v, out=out, state_out=state)

    def bwd_call():
        if w.op == "fwd+bwd":
            cp.causal_product_bwd(q, k, v, g, state_final=state, dq=dq, dk=dk, dv=dv)
        else:
            cp.linear_attn_bwd(q, k, v, out, g, den, 1, state_final=state, z_final=zfin, dq=dq, dk=dk, dv=dv)

    calls = [fwd_call] + ([bwd_call] if w.op.endswith("bwd") else [])
    kinds = {"fwd+bwd": ["fwd", "bwd"], "fwd": ["fwd"], "linattn": ["linattn"],
             "linattn+bwd": ["linattn", "linattn_bwd"]}[w.op]

    def step():
        for c in calls:
            c()

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, device="cuda", dtype=torch.float32)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    copy = copy_rate(torch)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K steps back to back, no timing hook.  Device time of the
    # region from two events on the stream the calls run on.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    device_s = ev0.elapsed_time(ev1) * 1e-3

    # Steady state: the same K steps once the load has lasted long enough for
    # the clocks to settle (about 50 ms at the headline workload; a short
    # region right after a few warm-up steps falls into a dip of the clocks
    # that follows the start of a burst of load).  Reported beside `value`,
    # which stays the K steps right after the W warm-up steps.  The per-call
    # durations below are taken right after it, at the same clocks.
    steady = None
    if args.settle_steps > 0:
        for _ in range(args.settle_steps):
            step()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for _ in range(args.steps):
            step()
        s1.record()
        torch.cuda.synchronize()
        sdev = s0.elapsed_time(s1) * 1e-3
        steady = {"settle_steps": args.settle_steps, "steps": args.steps,
                  "ms_per_step": sdev / args.steps * 1e3, "value": args.steps * w.token_heads / sdev}

    # Per-kernel durations: the same K steps again, each launch with its own
    # start/end events (the timestamps of its dispatch on the stream it runs
    # on, as a profiler's kernel trace reports them).  Launches per call: one,
    # or over few slices two (the segments' state increments, then the
    # sweeps); count them on one untimed step.
    n_launch = []
    for c in calls:
        cp.timing_begin(64)
        c()
        n_launch.append(len(cp.timing_end()))
    per_step = sum(n_launch)
    cp.timing_begin(args.steps * per_step)
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = cp.timing_end()
    assert len(ms) == args.steps * per_step, "every hooked launch is recorded"
    # a call's time is the sum of its launches
    times, launch_us, off = {}, {}, 0
    for kind, nl in zip(kinds, n_launch):
        times[kind] = sum(sum(ms[i * per_step + off:i * per_step + off + nl]) for i in range(args.steps)) \
            / args.steps * 1e-3
        launch_us[kind] = [sum(ms[i * per_step + off + j] for i in range(args.steps)) / args.steps * 1e3
                           for j in range(nl)]
        off += nl
    per_kernel = {}
    for kind in kinds:
        b = algorithmic_bytes(w, kind)
        f = algorithmic_flops(w, kind)
        per_kernel[kind] = {"avg_us": times[kind] * 1e6, "alg_bytes": b, "GBps": b / times[kind] / 1e9,
                            "alg_flops": f, "TFps": f / times[kind] / 1e12,
                            "launches": n_launch[kinds.index(kind)], "launch_us": launch_us[kind]}
    # Cold caches: each call again, after reading 1 GiB (more than L2 and
    # the MALL hold), so that no input is found in a cache.  The eviction is a
    # read, not a write: a write would leave the caches full of dirty lines
    # that the call would then have to write back.  Reported beside the
    # back-to-back figures; `value` and `roofline` stay the latter.
    cold = None
    if args.cold_steps > 0:
        flush = torch.ones(1 << 28, device="cuda", dtype=torch.float32)
        sink = torch.empty((), device="cuda", dtype=torch.float32)
        acc = {kind: 0.0 for kind in kinds}
        for i in range(args.cold_steps):
            for kind, c, nl in zip(kinds, calls, n_launch):
                torch.sum(flush, dim=0, out=sink)
                cp.timing_begin(nl)
                c()
                acc[kind] += sum(cp.timing_end()) * 1e-3
        torch.cuda.synchronize()
        del flush, sink
        cold = {kind: {"avg_us": acc[kind] / args.cold_steps * 1e6,
                       "GBps": algorithmic_bytes(w, kind) / (acc[kind] / args.cold_steps) / 1e9,
                       "frac": algorithmic_bytes(w, kind) / (acc[kind] / args.cold_steps) / 1e9 / HBM_PEAK_GBS}
                for kind in kinds}
    dom = max(kinds, key=lambda k: times[k])
    achieved = per_kernel[dom]["GBps"]
    hbm_frac = achieved / HBM_PEAK_GBS
    mfma_peak = MFMA_PEAK_TFS[w.dtype]
    mfma_frac = per_kernel[dom]["TFps"] / mfma_peak
    kname = kernel_name(dom, n_launch[kinds.index(dom)])
    hbm = {"bound": "hbm", "kernel": kname, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": hbm_frac, "traffic": traffic_for(dom, name), "frac_of_copy": achieved / copy["GBps"]}
    mfma = {"bound": "mfma", "kernel": kname, "achieved": per_kernel[dom]["TFps"], "peak": mfma_peak,
            "unit": "TFLOP/s", "frac": mfma_frac}
    roof = dict(hbm if hbm_frac >= mfma_frac else mfma)
    roof["other"] = mfma if roof["bound"] == "hbm" else hbm
    rec = {
        "metric": METRIC,
        "value": args.steps * w.token_heads / elapsed,
        "unit": UNIT,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "device_ms_per_step": device_s / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) draws; Q,K = elu(x)+1)" if w.qk == "elu1" else
                "synthetic (seeded N(0,1) draws; raw Q,K, feature map applied in the op)",
        "config": {"workload": name, "op": w.op, "N": w.N, "H": w.H, "L": w.L, "E": w.E, "M": w.M},
        "roofline": roof,
        "copy": copy,
        "kernels": per_kernel,
        "cold_cache": cold,
        "steady_state": steady,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, host)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
