#!/usr/bin/env python3
"""Benchmark the GDPA hot path on one MI355X and print one JSON line.

A step is one pass of the whole path over one batch of the workload: the jagged work
decomposition (gdpa_plan), the forward and the backward (dQ, dK, dV), with inputs resident in
HBM. The default workload is the personalized-FFN form in bf16, forward+backward: B=256
sequences with lengths uniform in [100, 1000], H=4, d=64, n=256 context-generated keys per
sample, SiLU, scale 1/1000 (seed 0 of the input recipe; synthetic data).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload pffn_train] [--no-cpu-baseline]
                      [--no-cold]

Besides the contract fields the line carries kernel_ms (mean per-kernel times), timing (p10 / p50
/ p90 of the step, the forward and the backward, and of a cold step that follows a 512 MiB write
flushing the Infinity Cache), roofline (the dominant kernel against its bound), mfma_reference (a
measured large bf16 library GEMM rate), hbm_reference (a measured 1 GiB copy rate) and
cpu_baseline (the oracle).
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

MFMA_PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 (256 CU x 2.4 GHz x 4096 flop/clk)
HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# Sources of each main kernel: the HBM-traffic counters of a kernel stay valid while these hash alike.
KERNEL_SOURCES = {
    "fwd": ["gdpa_device.hpp", "gdpa_launch.hpp", "gdpa_fwd.hpp", "gdpa_fwd.hip", "gdpa_fwd_any.hip"],
    "bwd": ["gdpa_device.hpp", "gdpa_launch.hpp", "gdpa_bwd.hpp", "gdpa_bwd.hip", "gdpa_bwd_pw.hip",
            "gdpa_bwd_sm.hip", "gdpa_bwd_agpr.hip", "gdpa_bwd_mix_d32.hip", "gdpa_bwd_mix_d64.hip",
            "gdpa_bwd_mix_d128.hip", "gdpa_bwd_mix_all.hip"],
}

WORKLOAD_TEXT = {
    "pffn_fwd": "PFFN-form GDPA bf16 forward: B=256, L~U[100,1000], H=4, d=64, n=256 context-generated "
            "keys/values, SiLU, scale 1/1000",
    "pffn_train": "PFFN-form GDPA bf16 forward+backward (dQ, dK, dV): B=256, L~U[100,1000], H=4, d=64, n=256 "
            "context-generated keys/values, SiLU, scale 1/1000, upstream gradient N(0,1)",
    "causal_gated": "gated-softmax self-attention bf16 forward+backward: B=128, L~U[200,2000], H=8, d=64, "
            "scale 1/8, log-sigmoid gate, causal window 128",
    "grouped10": "10 event groups in one launch, bf16 forward+backward: B=64 each, L~U[100,1000], n=32, "
            "groups 0-4 H=8 d=128, groups 5-9 H=2 d=32, GELU",
    "seed_pool": "seed-query pooling (PMA / hierarchical seed pooling form) bf16 forward+backward: S=256 "
            "learnable seed queries shared by B=256 sequences of L~U[100,1000] keys, H=4, d=64, softmax, "
            "scale 1/8, dQ summed over the sequences",
}


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "generalized_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they were taken on the
    current kernel sources; None otherwise."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    e = t.get(workload, {}).get(kernel)
    if not e or e.get("source_hash") != kernel_source_hash(kernel):
        return None
    return e.get("bytes_per_launch")


def percentiles(xs):
    """p10 / p50 / p90 of a list of per-step times (ms)."""
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"p10": float(np.percentile(a, 10)), "p50": float(np.percentile(a, 50)), "p90": float(np.percentile(a, 90))}


def measured_gemm_tflops(torch):
    """A reachable dense bf16 MFMA rate on this GPU: a large library GEMM (8192^3, hipBLASLt via
    torch.matmul), best of 10 runs. A reference point for the kernels, not part of the path."""
    n = 8192
    a = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.matmul(a, b)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    return 2.0 * n ** 3 / (best * 1e-3) / 1e12


def measured_hbm_gbps(torch):
    """A reachable HBM rate on this GPU for traffic that both reads and writes: a 1 GiB
    device-to-device copy, best of 5 (bytes read + written). A reference point, not part of the
    path: the GDPA kernels also both read and write."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)

    def best(fn):
        fn()
        torch.cuda.synchronize()
        t = float("inf")
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            t = min(t, e0.elapsed_time(e1))
        return t

    copy_ms = best(lambda: b.copy_(a))
    return {"copy_gbps": 2.0 * n / (copy_ms * 1e-3) / 1e9}


def cpu_model_name():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def host_threads() -> int:
    """The CPU threads the oracle runs on: this process's affinity set, at most 16 (the CPU share a
    GPU machine allots to one GPU, whatever count its host reports)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_baseline(workload, passes, seqs: int):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload (host cores)."""
    import numpy as np
    import oracle
    from gdpa_workloads import group_work

    threads = host_threads()
    rng = np.random.default_rng(123)
    flops = 0.0
    elapsed = 0.0
    picked = 0
    for g in workload.groups:
        k = max(1, min(g.spec.num_seqs, int(round(seqs * g.spec.num_seqs / sum(x.spec.num_seqs for x in workload.groups)))))
        sub = g.subset(sorted(rng.choice(g.spec.num_seqs, size=k, replace=False).tolist()))
        picked += k
        wk = group_work(sub)
        t0 = time.perf_counter()
        oracle.group_fwd(sub, nthreads=threads)
        if "bwd" in passes:
            oracle.group_bwd(sub, nthreads=threads)
        elapsed += time.perf_counter() - t0
        flops += wk["fwd_flops"] + (wk["bwd_flops"] if "bwd" in passes else 0.0)
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model_name(), "host_cpus_visible": os.cpu_count(),
            "sample": f"{picked} sequences drawn from the same workload (seeded), fwd{'+bwd' if 'bwd' in passes else ''}, "
                      f"{elapsed:.1f} s, {flops / 1e9:.2f} GFLOP of model work"}


def oracle_table():
    """Wall time of the fp64 oracle, as it stands, for each workload at full size: one forward and
    one backward call per group (the backward call recomputes its own row statistics), the median
    of 20 calls for the small fp32 workload. One JSON line per workload."""
    import numpy as np
    import oracle
    from gdpa_workloads import group_work, make_workload
    from gdpa_workloads.recipe import CONFIGS

    threads = host_threads()
    print(json.dumps({"oracle_threads": threads, "host_cpus_visible": os.cpu_count(),
                      "cpu_model": cpu_model_name()}), flush=True)
    for name in CONFIGS:
        w = make_workload(name, 0)
        reps = 20 if name == "tiny_fp32" else 1
        row = {"workload": name, "calls": reps}
        for pass_ in w.passes:
            times = []
            for _ in range(reps):
                t0 = time.perf_counter()
                for g in w.groups:
                    if pass_ == "fwd":
                        oracle.group_fwd(g, nthreads=threads)
                    else:
                        oracle.group_bwd(g, nthreads=threads, want_dg=g.g is not None)
                times.append(time.perf_counter() - t0)
            wall = float(np.median(times))
            gflop = sum(group_work(g)[f"{pass_}_flops"] for g in w.groups) / 1e9
            row[f"{pass_}_s"] = wall
            row[f"{pass_}_gflop"] = gflop
            row[f"{pass_}_gflops_per_s"] = gflop / wall
        print(json.dumps(row), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="pffn_train", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seqs", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-s", type=float, default=0.1,
                    help="seconds of untimed steps before the warm-up steps (clock settling)")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache steps (keeps a profiler's per-kernel averages to the warm steps)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 512 MiB device-to-device copy (scales HBM byte counters)")
    ap.add_argument("--oracle-table", action="store_true",
                    help="only time the fp64 oracle (fwd and bwd wall time) on every workload at full size")
    args = ap.parse_args()
    if args.oracle_table:
        oracle_table()
        return
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (got --gpus {args.gpus}); the GDPA path has no "
              f"cross-GPU step and is run per GPU on its share of the batch.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = 512 << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 3}))
        return
    import generalized_attention_amd as ga
    from gdpa_workloads import make_workload, workload_work

    w = make_workload(args.workload, args.seed)
    passes = w.passes
    work = workload_work(w)
    dev = torch.device("cuda:0")
    groups = []
    for g in w.groups:
        s = g.spec
        groups.append(ga.make_group(g.q.to(dev), g.k.to(dev), g.v.to(dev), g.q_offsets, g.kv_offsets, act=s.act,
                                    scale=s.scale, window=s.window, g=None if g.g is None else g.g.to(dev),
                                    self_attention=s.keys_per_seq is None and not s.shared_q, shared_q=s.shared_q,
                                    lengths_q=g.lengths_q.tolist(),
                                    lengths_kv=g.lengths_kv.tolist()))
    douts = [g.dout.to(dev) for g in w.groups]
    ws = ga.workspace(groups, 1 if "bwd" in passes else 0)
    planned = [ga.GroupArgs(**{**gr.__dict__, "planned": True}) for gr in groups]
    fwd_outs = [ga.ops._alloc_fwd(gr) for gr in groups]
    bwd_outs = [ga.ops._alloc_bwd(gr, want_dg=gr.g is not None) for gr in groups]
    single = len(groups) == 1

    def plan():
        ga.gdpa_plan(groups, ws)

    def fwd():
        if single:
            ga.gdpa_fwd(planned[0], o=fwd_outs[0][0], lse=fwd_outs[0][1], ws=ws)
        else:
            ga.gdpa_fwd_grouped(planned, outs=fwd_outs, ws=ws)

    def bwd():
        if single:
            ga.gdpa_bwd(planned[0], douts[0], o=fwd_outs[0][0], lse=fwd_outs[0][1], out=bwd_outs[0], ws=ws)
        else:
            ga.gdpa_bwd_grouped(planned, douts, fwd_outs=fwd_outs, outs=bwd_outs, ws=ws)

    def step():
        plan()
        fwd()
        if "bwd" in passes:
            bwd()

    # Reference rates first: a large library GEMM and a 1 GiB copy (reported in the line). They
    # also bring the GPU out of its idle clock before the warm-up steps, so a short warm-up does
    # not leave the first timed steps at a ramping clock.
    refs = {}
    try:
        refs["gemm"] = measured_gemm_tflops(torch)
    except RuntimeError as exc:  # a reference only: the line is printed without it
        refs["gemm_error"] = str(exc)[:200]
    try:
        refs["hbm"] = measured_hbm_gbps(torch)
    except RuntimeError as exc:
        refs["hbm_error"] = str(exc)[:200]
    torch.cuda.empty_cache()

    # Clock settling: the step itself, repeated for a fixed wall time before the W warm-up steps
    # (an idle or GEMM-loaded GPU runs the first memory-bound steps at a lower clock; a training
    # loop runs at the settled one). Untimed, reported as settle_steps.
    settle_steps = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(20):
            step()
        settle_steps += 20
        torch.cuda.synchronize()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # whole-step timing: events only at the ends of the timed region
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps

    # per-kernel timing: an event between consecutive launches (same stream as the kernels)
    n_ev = 4
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        evs[i][0].record()
        plan()
        evs[i][1].record()
        fwd()
        evs[i][2].record()
        if "bwd" in passes:
            bwd()
        evs[i][3].record()
    torch.cuda.synchronize()
    k_ms = {"plan": 0.0, "fwd": 0.0, "bwd": 0.0}
    for e in evs:
        k_ms["plan"] += e[0].elapsed_time(e[1]) / args.steps
        k_ms["fwd"] += e[1].elapsed_time(e[2]) / args.steps
        k_ms["bwd"] += e[2].elapsed_time(e[3]) / args.steps
    timing = {"step_ms": percentiles([e[0].elapsed_time(e[3]) for e in evs]),
              "fwd_ms": percentiles([e[1].elapsed_time(e[2]) for e in evs])}
    if "bwd" in passes:
        timing["bwd_ms"] = percentiles([e[2].elapsed_time(e[3]) for e in evs])
    if not args.no_cold:
        # cold: a 512 MiB write (twice the 256 MB Infinity Cache) between steps, outside the events
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        n_cold = min(args.steps, 50)
        cold = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_cold)]
        for i in range(n_cold):
            flush.zero_()
            cold[i][0].record()
            step()
            cold[i][1].record()
        torch.cuda.synchronize()
        timing["cold_step_ms"] = percentiles([c[0].elapsed_time(c[1]) for c in cold])
        del flush
    for o in fwd_outs + [tuple(b[:3]) for b in bwd_outs]:
        for t in o:
            if t is not None and not torch.isfinite(t).all():
                raise RuntimeError("non-finite output")

    flops = work["fwd_flops"] + (work["bwd_flops"] if "bwd" in passes else 0.0)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    dominant = "bwd" if ("bwd" in passes and k_ms["bwd"] >= k_ms["fwd"]) else "fwd"
    kbytes = work[f"{dominant}_bytes"]
    kflops = work[f"{dominant}_flops"]
    ridge = MFMA_PEAK_BF16_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    kms = k_ms[dominant]
    if kflops / kbytes < ridge:
        roof = {"bound": "hbm", "achieved": kbytes / (kms * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": kflops / (kms * 1e-3) / 1e12, "peak": MFMA_PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = load_traffic(args.workload, dominant)
    roof["kernel"] = (f"gdpa_{dominant} main kernel ("
                      + ("bwd_small_kernel / bwd_bf16_kernel" if dominant == "bwd" else "fwd_bf16_kernel") + ")")
    roof["kernel_ms"] = kms
    roof["algorithmic_bytes"] = kbytes
    roof["algorithmic_flops"] = kflops
    roof["mfma_frac"] = kflops / (kms * 1e-3) / 1e12 / MFMA_PEAK_BF16_TFLOPS

    out = {
        "metric": "GDPA fwd+bwd bf16 TFLOP/s and % of MI355X MFMA peak, jagged L<=1000",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {WORKLOAD_TEXT[args.workload]}",
                   "global_batch": sum(g.spec.num_seqs for g in w.groups),
                   "seq_len": "jagged", "total_rows": sum(g.total_q for g in w.groups),
                   "score_entries": work["entries"], "model_gflop_per_step": flops / 1e9,
                   "seed": args.seed},
        "pct_of_mfma_peak": 100.0 * tflops / MFMA_PEAK_BF16_TFLOPS,
        "hbm_gbps_step": (work["fwd_bytes"] + (work["bwd_bytes"] if "bwd" in passes else 0.0)) / (ms_per_step * 1e-3) / 1e9,
        "kernel_ms": k_ms,
        "timing": timing,
        "roofline": roof,
    }
    if "gemm" in refs:
        out["mfma_reference"] = {"measured_gemm_tflops": refs["gemm"], "step_frac_of_measured": tflops / refs["gemm"]}
    else:
        out["mfma_reference"] = {"error": refs.get("gemm_error")}
    if "hbm" in refs:
        hbm = dict(refs["hbm"])
        hbm["dominant_kernel_frac_of_copy"] = roof["achieved"] / hbm["copy_gbps"] if roof["unit"] == "GB/s" else None
        out["hbm_reference"] = hbm
    else:
        out["hbm_reference"] = {"error": refs.get("hbm_error")}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, passes, args.cpu_seqs)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
