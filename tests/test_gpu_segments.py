"""Bounded fp32 accumulation runs of the statistics passes.

Every family accumulates s0 / s1 / s2 in fp32 registers for at most a fixed
number of tiles per workgroup (or wave) and then closes the run into fp64
([Flash-GMM] Method: s0, s1, s2 accumulated on chip; [LP-GMM] 1.3 and 2.1:
statistics in fp32 or wider).  The pass is launched in segments of that
length; GMM_SEGMENT_TILES shortens the runs so that every workgroup closes
several of them at sizes the oracle finishes in seconds.

Per workload shape (the four benchmark workloads' D, K, covariance type and
storage type), at an N where the pass takes three or more segments:
  * s0, s1 and s2 element by element against the oracle's sums;
  * the same step run as one segment agrees with the segmented one to fp32
    accumulation rounding (only the order of the fp32 / fp64 sums differs).

Element-wise allowance |got - ref| <= rtol |ref| + atol max|ref|.  fp32 path:
the 1e-4 bar.  fp16-operand paths: a point's responsibility for k moves by
at most gamma (1 - gamma) dS <= dS / 4 under a score error dS, which the fp16
expanded form keeps near 0.1-0.2 nats for well-conditioned components, so a
component whose points are all contested can move by up to 5 % of its mass
(rtol 5e-2); the fp16 roundings of gamma and x add 2^-10 relative.
"""
import numpy as np
import pytest
import torch

from soft_clustering_amd import synth
from tests import metrics
from tests.gpu_common import (gpu_step, oracle_stats_chunked, params64, stats_elementwise, to_dev)

pytestmark = pytest.mark.gpu

CASES = [
    # workload, N, tiles per run, (rtol, atol as a fraction of the tensor's max)
    # diagonal fp32: 256 workgroups x 8 waves, 1 tile per wave and segment -> 5 segments
    ("diag-f32-n1e6-d64-k16", 300_000, 1, (1e-4, 1e-5)),
    # isotropic bf16, one sweep: 256 chunks x 2 tiles -> 3 segments
    ("iso-bf16-n1e7-d128-k256", 40_000, 2, (5e-2, 2e-3)),
    # diagonal bf16, K = 1024, sweep 2: 64 chunks x 1 tile -> 3 segments
    ("diag-bf16-n2e8-d128-k1024", 6_000, 1, (5e-2, 2e-3)),
    # full covariance fp16: 256 workgroups x 1 tile of 256 points -> 3 segments
    ("full-f16-n1e6-d64-k16", 140_000, 1, (5e-2, 2e-3)),
]


@pytest.mark.parametrize("name,n,seg,tol", CASES, ids=[c[0] for c in CASES])
def test_segmented_statistics(gmm_lib, monkeypatch, name, n, seg, tol):
    w = synth.WORKLOADS[name].with_n(n, f"-n{n}")
    mix = synth.make_mixture(w)
    x = synth.sample_points(w, mix)
    th0 = synth.init_params(w, x)
    xg = x.cuda()
    th = to_dev(*th0)
    gm = gmm_lib.Gmm(w.n, w.d, w.k, w.cov, w.x_dtype)
    print(f"{name} at N={n}: runs of {seg} tiles", flush=True)
    monkeypatch.setenv("GMM_SEGMENT_TILES", str(seg))
    ll, st, _ = gpu_step(gm, xg, *th)
    monkeypatch.setenv("GMM_SEGMENT_TILES", str(1 << 40))   # one segment
    ll1, st1, _ = gpu_step(gm, xg, *th)
    monkeypatch.delenv("GMM_SEGMENT_TILES")
    # segmentation only reorders the sums
    for a, b, nm in ((st.s0, st1.s0, "s0"), (st.s1, st1.s1, "s1"), (st.s2, st1.s2, "s2")):
        r = metrics.rel_inf(a.cpu().numpy(), b.cpu().numpy())
        print(f"   segmented vs one segment {nm}: {r:.2e}", flush=True)
        assert r <= 1e-5, (nm, r)
    assert metrics.rel(ll, ll1) <= 1e-9
    # element by element against the oracle
    xd = x.double().numpy()
    print("   oracle...", flush=True)
    ll_ref, s0, s1, s2 = oracle_stats_chunked(xd, params64(w.cov, *th))
    rtol, atol = tol
    print(f"   LL rel {metrics.rel(ll, ll_ref):.2e}", flush=True)
    assert metrics.rel(ll, ll_ref) <= (1e-4 if w.x_dtype == "f32" else 9e-3)
    stats_elementwise(st.s0.cpu().numpy(), s0, rtol, atol, "s0")
    stats_elementwise(st.s1.cpu().numpy(), s1, rtol, atol, "s1")
    stats_elementwise(st.s2.cpu().numpy(), s2, rtol, atol, "s2")
    assert abs(st.s0.sum().item() - n) <= 1e-4 * n
