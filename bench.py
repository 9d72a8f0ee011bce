"""Benchmark: one fused GMM EM iteration (gmm_em_step + gmm_finalize) on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line.  A step is one EM iteration over the whole synthetic
workload, already resident in HBM: the fused E+M kernel(s) over all points,
then the reduction / M-step kernel.  Workloads specified as a single EM
iteration time every step from the initial parameters (gmm_prepare is then
part of the step); the others chain the iterations.

The default workload is the largest one that fits a single GPU: the diagonal
mixture of 2e8 points, D=128, K=1024, stored in bf16 (51.2 GB), whose fused
iteration takes two sweeps over X.  `value` is EM iterations/s;
points*components/s and the achieved HBM bandwidth are reported beside it.
`roofline` prices gmm_em_step (all its launches) with its algorithmic work
(8*D*K flops per point diagonal, 4*D*K isotropic, (2 D(D+1) + 4D) K full)
against the dense fp16 matrix-core peak, timed with HIP events recorded on
the stream the kernels run on.  `calibration` measures the device's own
ceilings (a streaming read of X, register-resident fp16 MFMA chains) and
reports the fractions against them too.  `cpu_baseline` times the fp64
oracle, as it stands, on a bounded prefix of the same workload with one
worker process per host core.
"""
from __future__ import annotations

import argparse
import hashlib
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
DEFAULT_WORKLOAD = "diag-bf16-n2e8-d128-k1024"

# HBM traffic of one gmm_em_step (every launch it makes), measured with two
# rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE) over
#   bench.py --workload W --steps 3 --warmup 1 --no-cpu-baseline --no-digest
#            --no-calibration --copy-calibration
# summed over the em_step kernels' per-dispatch averages (KiB; a segmented
# pass's launches summed).  The same run copies a buffer of the size of X once
# (a device-to-device copy: reads and writes copy_bytes), and each counter is
# scaled by copy_bytes / (what it read for that copy).  "sources" is a digest of the kernel sources the figures were
# taken on: once they change, the figures are stale and traffic is reported
# as null.
TRAFFIC = {
    "diag-f32-n1e6-d64-k16": dict(
        sources="e577314d9fe4ccae", fetch_kib=125176.5, write_kib=4144.3,
        copy_bytes=2.56e+08, copy_fetch_kib=125011.5, copy_write_kib=250000.0),
    "iso-bf16-n1e7-d128-k256": dict(
        sources="1ddfc6385e023df2", fetch_kib=1251543.4, write_kib=78474.3,
        copy_bytes=2.56e+09, copy_fetch_kib=1250035.6875, copy_write_kib=2500000.0),
    "diag-bf16-n2e8-d128-k1024": dict(
        sources="1ddfc6385e023df2", fetch_kib=53762256.3, write_kib=7458634.4,
        copy_bytes=5.12e+10, copy_fetch_kib=25000253.125, copy_write_kib=50000000.0),
    "full-f16-n1e6-d64-k16": dict(
        sources="abdce93111c35cee", fetch_kib=66005.4, write_kib=39623.3,
        copy_bytes=1.28e+08, copy_fetch_kib=62511.5, copy_write_kib=125000.0),
    "full-f16-n1e6-d128-k16": dict(
        sources="abdce93111c35cee", fetch_kib=257789.8, write_kib=41404.2,
        copy_bytes=2.56e+08, copy_fetch_kib=125011.5, copy_write_kib=250000.0),
}
_SHARED_SOURCES = ("api.hip", "common.h", "plan.h", "../build.py")
FAMILY_SOURCES = {
    "diag_f32": ("diag_split.hip", "diag_params.hip", "diag_internal.h") + _SHARED_SOURCES,
    "largek": ("largek.hip", "largek_params.hip", "largek_exact.hip", "largek_internal.h") + _SHARED_SOURCES,
    "full": ("full_fused.hip", "full_params.hip", "full_internal.h") + _SHARED_SOURCES,
}


def sources_digest(family):
    """SHA-256 (first 16 hex digits) over the family's kernel sources."""
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


# ---- CPU baseline: the oracle on every host core -----------------------------
# The worker processes are started (spawned: a fresh interpreter each) before
# this process touches the GPU, and never use it; each runs the oracle's
# em_step, as it stands, over its share of a prefix of X.

def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _worker_init():
    from threadpoolctl import threadpool_limits
    global _LIMITS
    _LIMITS = threadpool_limits(limits=1)   # one thread per worker process


def _worker_step(args):
    import oracle
    xs, pi, mu, cov, cov_type = args
    t = time.perf_counter()
    oracle.em_step(xs, oracle.Params(pi, mu, cov, cov_type))
    return time.perf_counter() - t


def _worker_ready(_):
    import oracle  # noqa: F401  (imported before anything is timed)
    return os.getpid()


def start_cpu_pool(cores):
    import multiprocessing as mp
    ctx = mp.get_context("spawn")
    pool = ctx.Pool(cores, initializer=_worker_init)
    pool.map(_worker_ready, range(cores), chunksize=1)   # every worker up, oracle imported
    return pool


def cpu_baseline(pool, cores, w, x_dev, theta, target_s=15.0):
    """The oracle on a prefix of the workload, one share per worker; scaled
    to EM iterations/s and points*components/s of the whole workload."""
    pi, mu, cov = theta
    par = (np.asarray(pi, np.float64), np.asarray(mu, np.float64), np.asarray(cov, np.float64), w.cov)

    def run(m):
        xs = x_dev[:m].double().cpu().numpy()
        parts = np.array_split(xs, cores)
        t = time.perf_counter()
        pool.map(_worker_step, [(p, *par) for p in parts], chunksize=1)
        return time.perf_counter() - t, xs

    m = min(w.n, 64 * cores)
    dt, _ = run(m)                                          # calibration
    m2 = int(min(w.n, max(m, m * target_s / max(dt, 1e-3))))
    m2 = max(m, (m2 // (64 * cores)) * 64 * cores)
    dt, xs = run(m2)
    import torch
    digest = hashlib.sha256(x_dev[:m2].contiguous().cpu().view(-1).view(torch.uint8).numpy()).hexdigest()
    return {"value": (m2 / w.n) / dt, "unit": "EM iterations/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"first {m2} of {w.n} points (prefix), one fp64 numpy em_step per worker over "
                      f"{cores} equal shares, {cores} worker processes x 1 thread, {dt:.1f} s wall, "
                      f"scaled by {w.n}/{m2}",
            "points_components_per_s": m2 * w.k / dt,
            "sample_sha256": digest}


def x_digest(x, chunk_rows=1 << 20, workers=8):
    """SHA-256 over the SHA-256 digests of consecutive 2^20-row chunks of X's
    stored bytes (the chunks are hashed in parallel; hashlib releases the GIL)."""
    from concurrent.futures import ThreadPoolExecutor
    import torch
    n = x.shape[0]

    def one(lo):
        b = x[lo:lo + chunk_rows].contiguous().cpu().view(-1).view(torch.uint8).numpy()
        return hashlib.sha256(b).digest()

    with ThreadPoolExecutor(workers) as ex:
        ds = list(ex.map(one, range(0, n, chunk_rows)))
    return hashlib.sha256(b"".join(ds)).hexdigest()


def calibrate(gmm, x, reps=3):
    """Measured ceilings: streaming read of X, register-resident MFMA chains."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    grid_r = 8 * cus
    sink = gmm.calib_sink(grid_r)
    buf = x if x.is_contiguous() else x.contiguous()
    best_bw = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        nb = gmm.calib_read(buf, grid_r, sink)
        e1.record(stream)
        torch.cuda.synchronize()
        best_bw = max(best_bw, nb / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    grid_m = 2 * cus
    sinkm = gmm.calib_sink(grid_m)
    iters = 400_000
    best_tf = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fl = gmm.calib_mfma(iters, grid_m, sinkm)
        e1.record(stream)
        torch.cuda.synchronize()
        best_tf = max(best_tf, fl / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return {"hbm_read_GBps": best_bw, "hbm_read_bytes": int(nb),
            "mfma_f16_TFLOPs": best_tf, "mfma_instruction": "v_mfma_f32_32x32x16_f16",
            "kernels": "k_calib_read (16-byte grid-stride loads), k_calib_mfma (4 register chains per wave)",
            "best_of": reps}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-calibration", action="store_true")
    ap.add_argument("--no-digest", action="store_true", help="skip the SHA-256 digest of X")
    ap.add_argument("--from-init", choices=("auto", "yes", "no"), default="auto",
                    help="time every step from the initial parameters (prepare + em_step + "
                         "finalize); auto: for workloads specified as one EM iteration")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, copy a buffer of the size of X once (a plain copy kernel "
                         "whose HBM counters calibrate FETCH_SIZE / WRITE_SIZE)")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py: the benchmark runs on exactly one GPU (asked for {a.gpus}); the fused EM "
              "iteration is single-GPU and multi-GPU sharding is not built.", file=sys.stderr)
        return 2

    cores = host_cores()
    pool = None if a.no_cpu_baseline else start_cpu_pool(cores)   # before the GPU is touched

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
    torch.cuda.reset_peak_memory_stats()
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
    peak_mem = torch.cuda.max_memory_allocated()
    diag = gm.diagnostics()

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
        kname = ("k_full_wide_e + k_full_merge + one k_full_wide per quad of components "
                 "(+ k_full_sum_ll)" if w.d > 64 else
                 "k_full_pipe (+ k_full_sum_ll)" if w.d > 32 else "k_full_fused (+ k_full_sum_ll)")
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
        "peak_device_bytes": int(peak_mem),
        "x_bytes": int(w.x_bytes),
        "workspace_bytes": int(gm.ws_bytes),
        "nk_fp32_bytes": int(w.n * w.k * 4),
        "health": {"ill_cond": diag.ill_cond, "x_range": diag.x_range, "empty": diag.empty,
                   "nonfinite": diag.nonfinite, "bad_params": diag.bad_params},
        "roofline": roof,
        "calibration": None,
        "x_sha256": None,
        "cpu_baseline": None,
    }
    if a.copy_calibration:
        src = torch.empty(int(nbytes) // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        out["copy_calibration_bytes"] = int(nbytes)
    if not a.no_calibration:
        cal = calibrate(gmm, x)
        cal["frac_of_measured"] = (achieved_tflops / cal["mfma_f16_TFLOPs"] if roof["bound"] == "mfma"
                                   else hbm / cal["hbm_read_GBps"])
        out["calibration"] = cal
    if not a.no_digest:
        out["x_sha256"] = {"digest": x_digest(x), "recipe": "sha256 over the sha256 of consecutive "
                           "2^20-row chunks of X's stored bytes"}
    if pool is not None:
        out["cpu_baseline"] = cpu_baseline(pool, cores, w, x, (pi0, mu0, cov0))
        pool.close()
        pool.join()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
