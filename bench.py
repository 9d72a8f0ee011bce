"""Benchmark: one fused GMM EM iteration (gmm_em_step + gmm_finalize) on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line.  A step is one EM iteration over the whole synthetic
workload, already resident in HBM: the fused E+M kernel(s) over all points,
then the reduction / M-step kernel.  Workloads specified as a single EM
iteration time every step from the initial parameters (gmm_prepare is then
part of the step); the others chain the iterations.

The default workload is the diagonal fp32 mixture with 1e6 points, D=64,
K=16.  `value` is EM iterations/s; points*components/s and the achieved HBM
bandwidth are reported beside it.  `roofline` prices the dominant kernel
(gmm_em_step: the fused E+M kernel, or for more than 256 components the two
sweeps and the slice merge, plus the small scan / panel / LL-sum launches) with
its algorithmic work (8*D*K flops per point diagonal, 4*D*K isotropic)
against the dense peak of the contraction's operand type (fp32 matrix for the
fp32 family, fp16 for the large-K family), timed with HIP events recorded on
the stream the kernels run on.  `cpu_baseline` times the fp64
oracle on a bounded prefix of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, published
PEAK_TFLOPS = {                 # MI355X dense peaks, published
    "f32_matrix": 157.3,
    "bf16": 2500.0,
    "f16": 2500.0,
    "f32_vector": 157.3,
}
METRIC = "GMM EM iterations/sec & points·components/s at N,D,K; % of HBM or MFMA roofline"

# HBM traffic of one gmm_em_step (every launch it makes), measured with two
# rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE) over
#   bench.py --workload W --steps 2 --warmup 1 --no-cpu-baseline --copy-calibration
# summed over the em_step kernels' per-dispatch averages (KiB).  The same run
# copies a buffer of the size of X once (torch's copy kernel: reads and writes
# copy_bytes), and each counter is scaled by copy_bytes / (what it read for
# that copy).  "sources" is a digest of the kernel sources the figures were
# taken on: once they change, the figures are stale and traffic is reported
# as null.
TRAFFIC = {
    "diag-f32-n1e6-d64-k16": dict(
        sources="437d3889ed6ec5e7", fetch_kib=125183.4, write_kib=4144.3,
        copy_bytes=256e6, copy_fetch_kib=125021.25, copy_write_kib=250000.0),
    "iso-bf16-n1e7-d128-k256": dict(
        sources="027ea6c1b365e451", fetch_kib=1251255.1, write_kib=66743.4,
        copy_bytes=2.56e9, copy_fetch_kib=1250036.9375, copy_write_kib=2500000.0),
    "diag-bf16-n2e8-d128-k1024": dict(
        sources="027ea6c1b365e451", fetch_kib=114227215.7, write_kib=4043816.5,
        copy_bytes=51.2e9, copy_fetch_kib=25000258.0625, copy_write_kib=50000000.0),
    "full-f16-n1e6-d64-k16": dict(
        sources="481f08114fdf7145", fetch_kib=63933.1, write_kib=35528.6,
        copy_bytes=128e6, copy_fetch_kib=62514.9375, copy_write_kib=125000.0),
}
_SHARED_SOURCES = ("api.hip", "common.h", "plan.h", "../build.py")
FAMILY_SOURCES = {
    "diag_f32": ("diag_split.hip", "diag_params.hip", "diag_internal.h") + _SHARED_SOURCES,
    "largek": ("largek.hip", "largek_params.hip", "largek_internal.h") + _SHARED_SOURCES,
    "full": ("full_fused.hip", "full_params.hip", "full_internal.h") + _SHARED_SOURCES,
}


def sources_digest(family):
    """SHA-256 (first 16 hex digits) over the family's kernel sources."""
    import hashlib
    h = hashlib.sha256()
    for f in FAMILY_SOURCES[family]:
        with open(os.path.join(ROOT, "soft_clustering_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(w, family):
    """Calibrated HBM bytes per gmm_em_step, or None when no figures exist for
    this workload or the kernel sources changed since they were taken."""
    t = TRAFFIC.get(w.name)
    if t is None or t["sources"] != sources_digest(family):
        return None
    fetch = t["fetch_kib"] * t["copy_bytes"] / t["copy_fetch_kib"]
    write = t["write_kib"] * t["copy_bytes"] / t["copy_write_kib"]
    return {"bytes": fetch + write, "read_bytes": fetch, "write_bytes": write,
            "fetch_scale": t["copy_bytes"] / (1024 * t["copy_fetch_kib"]),
            "write_scale": t["copy_bytes"] / (1024 * t["copy_write_kib"])}


def algorithmic_work(w):
    """(flops, bytes) of one fused E+M pass: X read once; flops per point:
    diag 8DK (scores 4DK + statistics 4DK), iso 4DK, full (2 D(D+1) + 4D) K
    (whitening by the triangular inverse factor D(D+1)/2 FMA + symmetric outer
    product D(D+1)/2 FMA + 4D per point and component)."""
    es = 4 if w.x_dtype == "f32" else 2
    d = w.d
    per_pt = {"diag": 8 * d * w.k, "iso": 4 * d * w.k, "full": (2 * d * (d + 1) + 4 * d) * w.k}[w.cov]
    return float(per_pt) * w.n, float(w.n) * w.d * es


def cpu_baseline(w, x_dev, theta, target_s=12.0):
    """The oracle, as it stands, on a prefix of the workload; scaled to
    EM iterations/s of the whole workload."""
    import torch
    from threadpoolctl import threadpool_limits
    import oracle
    pi, mu, cov = theta
    p = oracle.Params(pi, mu, cov, w.cov)
    # calibration prefix of 1024 points, then a prefix sized to ~target_s
    m = min(1024, w.n)
    with threadpool_limits(limits=1):
        xs = x_dev[:m].double().cpu().numpy()
        t = time.perf_counter()
        oracle.em_step(xs, p)
        dt = time.perf_counter() - t
        m2 = int(min(w.n, max(m, m * target_s / max(dt, 1e-3))))
        m2 = max(m, (m2 // 256) * 256)
        xs = x_dev[:m2].double().cpu().numpy()
        t = time.perf_counter()
        oracle.em_step(xs, p)
        dt = time.perf_counter() - t
    it_s = (m2 / w.n) / dt
    return {"value": it_s, "unit": "EM iterations/s", "cores": 1, "kind": "oracle",
            "sample": f"first {m2} of {w.n} points, one em_step (fp64 numpy, 1 thread), "
                      f"{dt:.1f} s, scaled by {w.n}/{m2}",
            "points_components_per_s": m2 * w.k / dt}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="diag-f32-n1e6-d64-k16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--from-init", choices=("auto", "yes", "no"), default="auto",
                    help="time every step from the initial parameters (prepare + em_step + "
                         "finalize); auto: for workloads specified as one EM iteration")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, copy a buffer of the size of X once (a plain copy kernel "
                         "whose HBM counters calibrate FETCH_SIZE / WRITE_SIZE)")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU (asked for {a.gpus}); the fused EM "
              "iteration is single-GPU and multi-GPU sharding is not built.", file=sys.stderr)
        return 2

    import torch
    from soft_clustering_amd import gmm, synth

    w = synth.WORKLOADS[a.workload]
    from_init = a.from_init == "yes" or (a.from_init == "auto" and w.iters == 1)
    mix = synth.make_mixture(w)
    x = synth.sample_points(w, mix, device="cuda")
    pi0, mu0, cov0 = synth.init_params(w, x)
    gm = gmm.Gmm(w.n, w.d, w.k, w.cov, w.x_dtype)
    dev = lambda t: torch.as_tensor(t, dtype=torch.float32).cuda().contiguous()
    pi, mu, cov = dev(pi0), dev(mu0), dev(cov0)
    po, mo, co = torch.empty_like(pi), torch.empty_like(mu), torch.empty_like(cov)
    lls = torch.zeros(a.steps + a.warmup, dtype=torch.float64, device="cuda")
    stream = torch.cuda.current_stream()

    torch.cuda.synchronize()
    gm.prepare(pi, mu, cov)
    for i in range(a.warmup):
        if from_init:
            gm.prepare(pi, mu, cov)
        gm.em_step(x, lls[i:i + 1])
        gm.finalize(po, mo, co)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(a.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(a.steps):
        if from_init:
            gm.prepare(pi, mu, cov)
        ev[i][0].record(stream)
        gm.em_step(x, lls[a.warmup + i:a.warmup + i + 1])
        ev[i][1].record(stream)
        gm.finalize(po, mo, co)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    fused_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    ms_step = total_ms / a.steps
    fused_avg = float(np.mean(fused_ms))

    flops, nbytes = algorithmic_work(w)
    fp32_path = w.cov == "diag" and w.k <= 64          # fp32-accurate split-fp16 MFMA family
    full_path = w.cov == "full"                        # fp16 MFMA whitening + moments
    # every family runs its contractions on the fp16 matrix cores (the diagonal
    # family and the full family's whitening factor as fp16 hi + lo pairs):
    # the compute roof is the fp16 one
    peak_key = "f16"
    achieved_tflops = flops / (fused_avg * 1e-3) / 1e12
    hbm = nbytes / (fused_avg * 1e-3) / 1e9
    t_mfma = flops / (PEAK_TFLOPS[peak_key] * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBPS * 1e9)
    family = "diag_f32" if fp32_path else ("full" if full_path else "largek")
    traffic = measured_traffic(w, family)
    if t_mfma >= t_hbm:
        roof = {"bound": "mfma", "achieved": achieved_tflops,
                "peak": PEAK_TFLOPS[peak_key], "unit": "TFLOP/s",
                "frac": achieved_tflops / PEAK_TFLOPS[peak_key],
                "traffic": None if traffic is None else traffic["bytes"]}
    else:
        roof = {"bound": "hbm", "achieved": hbm, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": hbm / PEAK_HBM_GBPS, "traffic": None if traffic is None else traffic["bytes"]}
    if fp32_path:
        kname = "k_diag_split (the LL sum in its last workgroup)"
    elif full_path:
        kname = ("k_full_pipe (+ k_full_sum_ll)" if w.d > 32 else "k_full_fused (+ k_full_sum_ll)")
    elif w.k <= 256:
        kname = "k_lk<fused E+M> (+ k_lk_scan, k_lk_centre, k_lk_panel, k_lk_sum)"
    else:
        kname = ("k_lk<sweep 1> + k_lk_merge + k_lk<sweep 2> "
                 "(+ k_lk_scan, k_lk_centre, k_lk_panel, k_lk_sum)")
    roof.update({"kernel": kname, "timed": "gmm_em_step (all its launches), HIP events on its stream",
                 "avg_launch_ms": fused_avg,
                 "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": nbytes,
                 "hbm_GBps": hbm, "hbm_frac": hbm / PEAK_HBM_GBPS,
                 "traffic_unit": "bytes per gmm_em_step (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                 "copy-calibrated)",
                 "traffic_detail": traffic,
                 "sources_digest": sources_digest(family)})

    ll_hist = lls.cpu().numpy()
    out = {
        "metric": METRIC,
        "value": 1000.0 / ms_step,
        "unit": "EM iterations/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "split-f16/f32" if fp32_path else "f16",
        "math": ("products of fp16 hi/lo operand pairs on fp16 MFMA, fp32 accumulation, "
                 "fp32 exp/log/statistics" if fp32_path else
                 "fp16 MFMA whitening (inverse factor as fp16 hi + lo pairs) and second "
                 "moments, fp32 accumulation and softmax" if full_path else
                 "fp16 MFMA scores and statistics, fp32 accumulation and softmax"),
        "data": "synthetic",
        "config": {"workload": w.name, "n": w.n, "d": w.d, "k": w.k, "cov": w.cov,
                   "x_dtype": w.x_dtype, "parallelism": "single-gpu"},
        "steps_from": "initial parameters (every step)" if from_init else "previous step",
        "em_step_ms": fused_avg,
        "finalize_ms": ms_step - fused_avg,
        "points_components_per_s": w.n * w.k * 1000.0 / ms_step,
        "wall_s": wall,
        "ll_first_last": [float(ll_hist[0]), float(ll_hist[-1])],
        "roofline": roof,
        "cpu_baseline": None,
    }
    if a.copy_calibration:
        src = torch.empty(int(nbytes) // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = int(nbytes)
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, x, (pi0, mu0, cov0))
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
