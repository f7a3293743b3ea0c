"""Benchmark: fused diagonal-GMM EM iterations on one MI355X.

A step is one full EM iteration (parameter prologue, normaliser pass,
statistics pass, fixed-order reduction and M-step update) over the whole
synthetic data matrix, which is resident in HBM before timing starts. The
default workload is the headline one: N = 10,000,000 rows, D = 96, K = 1024,
fp32, non-negative integer descriptor-like data (planted means U[0,100]^D,
sd U[2,10], Zipf(1.1) weights), EM started from K seeded rows with unit
variances. Prints one JSON line.

Usage: python bench.py [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu-baseline] [--cpu-rows R] [--rows R]
                       [--mode em|kmeans|assign]

--mode kmeans times Lloyd (k-means) steps on the same data from the same
seeded centroids instead (the quantizer the GMM replaces); --mode assign
times the top-2 soft assignment pass followed by the IVF list construction.
Both print one JSON line of their own metric; the default is the EM step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP32_MFMA_TFLOPS = 157.3  # MI355X dense FP32 matrix peak (the metric's reference)
PEAK_FP64_MFMA_TFLOPS = 78.6   # MI355X dense FP64 matrix peak (the contractions' own dtype)

# HBM bytes per launch of the statistics kernel on the headline workload, from
# rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE runs of this bench (profiles/
# k_stats_descriptor_n10M_d96_k1024_hbm.md), each scaled by what the counter
# reads for a plain 3.84 GB device copy (FETCH_SIZE x2.0, WRITE_SIZE x1.0).
# Keyed by a hash of the kernel sources: a changed kernel reports null until
# it is profiled again.
MEASURED_TRAFFIC = {
    "45f21e27e4ec1449": {"workload": "descriptor", "kernel": "k_stats (pass 2)",
                         "bytes_per_launch": 1.6817e9},
}


def _kernel_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for name in ("gmm_kernels.hip", "gmm_device.h"):
        with open(os.path.join(ROOT, "gmm_em_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(workload: str, kernel: str):
    rec = MEASURED_TRAFFIC.get(_kernel_hash())
    if rec is None or rec["workload"] != workload or rec["kernel"] != kernel:
        return None
    return rec["bytes_per_launch"]


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="descriptor")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=3_000_000)
    ap.add_argument("--rows", type=int, default=0,
                    help="time a prefix of this many rows instead of the workload's N (the "
                         "JSON line then reports the prefix; EM cost is linear in N)")
    ap.add_argument("--mode", choices=("em", "kmeans", "assign"), default="em")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain device copy of the data matrix's size (calibrates the "
                         "HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the fused EM step runs on a single MI355X; "
              "multi-GPU runs are not part of this build", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from gmm_em_amd import datagen as dg
    from gmm_em_amd import ops

    W = dg.WORKLOADS[args.workload]
    if args.copy_probe:
        nbytes = W.n * W.d * (2 if W.dtype == "bf16" else 4)
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": nbytes, "copy_probe_bytes_written": nbytes,
                          "copies": 3}), flush=True)
        return 0
    t0 = time.time()
    n_rows = args.rows if 0 < args.rows < W.n else W.n
    x = dg.rows(W, n_rows)
    w0, m0, v0 = dg.init_params(W, x)
    print(f"# generated {W.key}: N={n_rows} D={W.d} K={W.k} in {time.time() - t0:.1f}s", file=sys.stderr,
          flush=True)
    dev = torch.device("cuda:0")
    if W.dtype == "bf16":
        xt = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        xt = torch.from_numpy(x).to(dev)
    ws = ops.workspace(W.d, W.k, dev)
    if args.mode != "em":
        return _other_mode(args, W, x, xt, w0, m0, v0, ws, n_rows)
    th0 = [torch.from_numpy(a).to(dev) for a in (w0, m0, v0)]
    w, mu, var = (t.clone() for t in th0)
    ll = torch.empty(max(args.steps, 1), dtype=torch.float64, device=dev)

    for _ in range(args.warmup):
        ops.em_step(xt, w, mu, var, W.var_floor, ws=ws, loglik=ll[0])
    torch.cuda.synchronize()
    for t, s in zip((w, mu, var), th0):
        t.copy_(s)
    torch.cuda.synchronize()

    chunk = 4096 if W.d > 128 else (1 << 22)  # rows per launch of each pass
    ops.profile_begin(args.steps * (-(-n_rows // chunk)) + 8)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        ops.em_step(xt, w, mu, var, W.var_floor, ws=ws, loglik=ll[i])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    prof = ops.profile_end()
    status = ops.device_status(ws, dev)
    if status != ops.GMM_OK:
        print(f"device status {status}", file=sys.stderr)
        return 1
    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / args.steps
    its = 1000.0 / ms_step
    flops_step = 8.0 * n_rows * W.d * W.k
    tflops = flops_step * its / 1e12
    hist = ll[: args.steps].cpu().numpy()

    # dominant kernel: the pass with the larger summed time (in the
    # cooperative single-pass schedule there is no pass 1 and the one kernel
    # does both contractions)
    (ms1, n1), (ms2, n2) = prof["pass1"], prof["pass2"]
    wide = W.d > 128  # rows past 128 dims run the D-sliced wide kernels
    if ms2 >= ms1:
        kname = ("k_wide statistics (pass 2)" if wide else "k_stats (pass 2)") if n1 > 0 \
            else "k_coop (single pass)"
        kms, kn, kflops = ms2, n2, 8.0 * W.d * W.k
    else:
        kname = "k_wide normaliser + k_wmerge (pass 1)" if wide else "k_lse (pass 1)"
        kms, kn, kflops = ms1, n1, 4.0 * W.d * W.k
    launches_per_step = kn / args.steps
    avg_ms = kms / kn
    alg_flops_launch = kflops * n_rows / launches_per_step
    achieved = alg_flops_launch / (avg_ms * 1e-3) / 1e12
    roofline = {
        "kernel": kname,
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": PEAK_FP64_MFMA_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_FP64_MFMA_TFLOPS, 4),
        "traffic": _traffic(W.key, kname),
        "schedule": "two-pass" if n1 > 0 else "cooperative single pass",
        "avg_launch_ms": round(avg_ms, 4),
        "launches_per_step": launches_per_step,
        "alg_flops_per_launch": alg_flops_launch,
        "pass1_ms_per_step": round(ms1 / args.steps, 3),
        "pass2_ms_per_step": round(ms2 / args.steps, 3),
    }

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import oracle

        nr = min(args.cpu_rows, n_rows)
        xs = x[:nr]
        t1 = time.perf_counter()
        oracle.em_step(xs, w0, m0, v0, W.var_floor)
        dt = time.perf_counter() - t1
        cpu = {
            "value": round(1.0 / (dt * n_rows / nr), 6),
            "unit": "EM it/s",
            "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"one EM step from the initial parameters on the first {nr} of {n_rows} rows "
                      f"({dt:.2f} s), scaled linearly to all rows",
        }

    headline = W.key == "descriptor" and n_rows == W.n
    out = {
        "metric": ("EM iterations/s and % MFMA roofline at N=10M,D=96,K=1024 (1 MI355X)" if headline
                   else f"EM iterations/s, {W.key} workload (1 MI355X)"),
        "value": round(its, 4),
        "unit": "EM it/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": f"{W.key}: N={n_rows} D={W.d} K={W.k} {W.dtype}, EM from seeded init"
                               + ("" if n_rows == W.n else f" (row prefix of N={W.n})"),
                   "n": n_rows, "d": W.d, "k": W.k, "x_dtype": W.dtype, "var_floor": W.var_floor},
        "x_dtype": W.dtype,
        "achieved_tflops": round(tflops, 2),
        # the metric's reference: 8*N*D*K flops per iteration against the
        # fp32-in/fp32-accumulate MFMA peak
        "pct_mfma_roofline": round(100.0 * tflops / PEAK_FP32_MFMA_TFLOPS, 2),
        # the same flops against the fp64 MFMA peak the contractions run on
        "pct_fp64_mfma_roofline": round(100.0 * tflops / PEAK_FP64_MFMA_TFLOPS, 2),
        "loglik_first_last": [float(hist[0]), float(hist[-1])],
        "wall_s": round(wall, 3),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


def _other_mode(args, W, x, xt, w0, m0, v0, ws, n_rows) -> int:
    """k-means steps or the soft-assignment pass + IVF lists (see the module doc)."""
    import torch

    from gmm_em_amd import ops

    dev = xt.device
    chunk = 4096 if W.d > 128 else (1 << 22)
    cfg = {"workload": f"{W.key}: N={n_rows} D={W.d} K={W.k} {W.dtype}"
                       + ("" if n_rows == W.n else f" (row prefix of N={W.n})"),
           "n": n_rows, "d": W.d, "k": W.k, "x_dtype": W.dtype}
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    extra = {}
    if args.mode == "kmeans":
        c0 = torch.from_numpy(m0).to(dev)
        c = c0.clone()
        for _ in range(args.warmup):
            ops.kmeans_step(xt, c, ws=ws, assign=False)
        c.copy_(c0)
        ops.profile_begin(args.steps * (-(-n_rows // chunk)) + 8)
        torch.cuda.synchronize()
        start.record()
        inertia = []
        for _ in range(args.steps):
            inertia.append(ops.kmeans_step(xt, c, ws=ws, assign=False)[0])
        stop.record()
        torch.cuda.synchronize()
        metric, unit = f"k-means (Lloyd) iterations/s, {W.key} workload (1 MI355X)", "k-means it/s"
        extra["inertia_first_last"] = [float(inertia[0].item()), float(inertia[-1].item())]
    else:
        w, mu, var = (torch.from_numpy(a).to(dev) for a in (w0, m0, v0))
        ops.em_step(xt, w, mu, var, W.var_floor, ws=ws)  # one EM step past the initial parameters
        for _ in range(args.warmup):
            ops.assign_topm(xt, w, mu, var, 2, ws=ws)
        ops.profile_begin(args.steps * (-(-n_rows // chunk)) + 8)
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.steps):
            idx, resp = ops.assign_topm(xt, w, mu, var, 2, ws=ws)
        stop.record()
        torch.cuda.synchronize()
        metric, unit = f"top-2 soft-assignment passes/s, {W.key} workload (1 MI355X)", "passes/s"
        # the IVF lists from the last assignment (threshold 0.1 for the border copies)
        ivf_ms = []
        for _ in range(3):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            off, rows, _ = ops.ivf_build(idx, resp, W.k, 0.1)
            b.record()
            torch.cuda.synchronize()
            ivf_ms.append(a.elapsed_time(b))
        extra["ivf_build_ms"] = round(min(ivf_ms), 3)
        extra["ivf_entries"] = int(rows.numel())
    prof = ops.profile_end()
    if ops.device_status(ws, dev) != ops.GMM_OK:
        print("device status not ok", file=sys.stderr)
        return 1
    ms_step = start.elapsed_time(stop) / args.steps
    (ms1, n1), (ms2, n2) = prof["pass1"], prof["pass2"]
    kname, kms, kn = ("k_wide normaliser + k_wmerge (pass 1)" if W.d > 128 else "k_lse (pass 1)"), ms1, n1
    if ms2 > ms1:
        kname, kms, kn = "k_stats (pass 2, one-hot)", ms2, n2
    flops_launch = 4.0 * W.d * W.k * n_rows / (kn / args.steps) if kname.endswith("(pass 1)") else None
    avg_ms = kms / kn
    achieved = flops_launch / (avg_ms * 1e-3) / 1e12 if flops_launch else None
    out = {
        "metric": metric, "value": round(1000.0 / ms_step, 4), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64",
        "data": "synthetic", "config": cfg,
        "roofline": {"kernel": kname, "bound": "mfma",
                     "achieved": round(achieved, 2) if achieved else None,
                     "peak": PEAK_FP64_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_FP64_MFMA_TFLOPS, 4) if achieved else None,
                     "traffic": None, "avg_launch_ms": round(avg_ms, 4),
                     "pass1_ms_per_step": round(ms1 / args.steps, 3),
                     "pass2_ms_per_step": round(ms2 / args.steps, 3)},
        "cpu_baseline": None,
        **extra,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
