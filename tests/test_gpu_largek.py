"""Parity of the large-K HIP path (isotropic / diagonal covariance, X stored
in bf16 or fp16, fp16 MFMA operands, fp32 softmax and statistics) against the
fp64 oracle.

Gate for reduced-precision storage (the operator write-up's acceptance bar,
section 2.3): LL(theta_t) relative error <= 9e-3 and argmax agreement
>= 99.5%.  The parameters are reported; as a guard against gross errors they
must also stay within loose bounds (SANITY) for components holding at least
MIN_MASS points.  The oracle takes the same stored X (bf16 / fp16 values
upcast) and the same fp32 parameters.
"""
import numpy as np
import pytest
import torch

import oracle
from soft_clustering_amd import synth
from tests import metrics
from tests.gpu_common import (check_params_bounded, gamma_error_bound, ill_conditioned, params64,
                              stats_elementwise, to_dev, workload_inputs)

pytestmark = pytest.mark.gpu

LL_TOL = 9e-3        # reduced-precision LL bar
ARGMAX_MIN = 0.995   # reduced-precision argmax-agreement bar
SANITY = {"s0": 1e-2, "pi": 1e-2, "mu": 2e-2, "cov": 5e-2}
MIN_MASS = 20.0


def gpu_step(gm, x, pi, mu, cov, prepare=True):
    if prepare:
        gm.prepare(pi, mu, cov)
    ll = torch.zeros(1, dtype=torch.float64, device="cuda")
    gm.em_step(x, ll)
    po, mo, co = torch.empty_like(pi), torch.empty_like(mu), torch.empty_like(cov)
    gm.finalize(po, mo, co)
    st = gm.get_stats()
    torch.cuda.synchronize()
    return float(ll.item()), st, (po, mo, co)


def gpu_loglik(gm, x, th):
    gm.prepare(*th)
    ll = torch.zeros(1, dtype=torch.float64, device="cuda")
    lse = torch.full((gm.n,), float("nan"), device="cuda")
    arg = torch.full((gm.n,), -1, dtype=torch.int32, device="cuda")
    gm.loglik(x, ll, lse, arg)
    torch.cuda.synchronize()
    return float(ll.item()), lse.cpu().numpy(), arg.cpu().numpy()


def check_reduced(ref, ll, st, theta, what=""):
    """Reduced-precision gate: LL and argmax bars of the pages, parameters and
    statistics within the SANITY bounds.  Nothing here reads a flag of the
    library under test."""
    heavy = np.asarray(ref.nk) >= MIN_MASS
    errs = {
        "ll": metrics.rel(ll, ref.ll),
        "s0": metrics.rel_inf(st.s0.cpu().numpy(), ref.nk),
        "pi": metrics.rel_inf(theta[0].cpu().numpy(), ref.params.pi),
        "mu": metrics.rel_inf(theta[1].cpu().numpy()[heavy], ref.params.mu[heavy]) if heavy.any() else 0.0,
        "cov": metrics.rel_inf(theta[2].cpu().numpy()[heavy], ref.params.cov[heavy]) if heavy.any() else 0.0,
        "s1": metrics.rel_inf(st.s1.cpu().numpy(), ref.s1),
        "s2": metrics.rel_inf(st.s2.cpu().numpy(), ref.s2),
    }
    print(what, " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if (k == "ll" and not v <= LL_TOL) or
           (k in SANITY and not v <= SANITY[k])}
    assert not bad, (what, bad)
    return errs


def check_later_step(ref, ll, st, theta_out, theta_in, xd, cov, what=""):
    """Gate of a step from the GPU's own theta_t (t >= 1).  The pages' bar
    for reduced precision holds as in the first step (LL relative error);
    the parameters are compared element by element within the error that
    the fp16 score precision propagates to them (gpu_common.gamma_error_bound,
    check_params_bounded): after a step, components crowd together and
    shrink, and the split of mass between two nearly identical components
    moves with score errors of a few tenths of a nat.  Components whose
    expanded-form score cannot be resolved (collapsed ones) are scored in
    the exact centred form by the library; the bound takes them as exact."""
    th_in = tuple(t.cpu().numpy() for t in theta_in)
    ill = ill_conditioned(th_in, xd, cov)
    if ill:
        print(f"{what}: {len(ill)} ill-conditioned components (first {ill[:8]})", flush=True)
    err = metrics.rel(ll, ref.ll)
    print(f"{what} ll={err:.2e}", flush=True)
    assert err <= LL_TOL, (what, err)
    p = params64(cov, *theta_in)
    B, g = gamma_error_bound(xd, p, th_in, cov)
    return check_params_bounded(ref, st, theta_out, xd, B, g, cov, what=what)


def check_argmax(xd, p, arg, what=""):
    _, lse_ref, arg_ref = oracle.loglik(xd, p)
    agree = float(np.mean(arg == arg_ref))
    print(what, f"argmax agreement {agree * 100:.3f}%", flush=True)
    assert agree >= ARGMAX_MIN, (what, agree)
    return lse_ref


def _make(n, d, k, cov, x_dtype, ldx_pad, misalign, seed, spread=6.0, offset=0.0):
    rng = np.random.default_rng(seed)
    kt = max(1, min(k, 64))
    mu_t = offset + rng.uniform(-spread, spread, size=(kt, d))
    z = rng.integers(0, kt, size=n)
    sd = rng.uniform(0.5, 1.5, size=(kt, d) if cov == "diag" else (kt, 1))
    xf = (mu_t[z] + rng.standard_normal((n, d)) * sd[z]).astype(np.float32)
    dt = synth.torch_dtype(x_dtype)
    ldx = d + ldx_pad
    off = 1 if misalign else 0
    buf = torch.zeros(n * ldx + off + 8, dtype=dt)
    xs = torch.as_strided(buf, (n, d), (ldx, 1), off)
    xs.copy_(torch.from_numpy(xf).to(dt))
    xg = torch.as_strided(buf.cuda(), (n, d), (ldx, 1), off)
    idx = rng.choice(n, size=k, replace=(k > n))
    mu0 = xs[torch.as_tensor(idx)].float().numpy()
    pi0 = rng.dirichlet(np.ones(k)).astype(np.float32)
    cov0 = rng.uniform(0.5, 2.0, size=(k, d) if cov == "diag" else (k,)).astype(np.float32)
    return xs.double().numpy(), xg, ldx, (pi0, mu0, cov0)


CASES = [
    # n, d, k, cov, x_dtype, ldx_pad, misalign
    (1, 8, 1, "iso", "bf16", 0, False),
    (33, 16, 5, "iso", "f16", 0, False),
    (1000, 24, 100, "iso", "bf16", 0, False),
    (3001, 128, 256, "iso", "bf16", 0, False),
    (2500, 100, 300, "iso", "f16", 4, False),
    (4097, 64, 257, "iso", "bf16", 8, True),
    (1500, 32, 65, "diag", "bf16", 0, False),
    (2047, 128, 256, "diag", "bf16", 0, False),
    (3000, 40, 513, "diag", "f16", 0, False),
    (999, 17, 200, "diag", "bf16", 3, True),
    (5003, 128, 1024, "diag", "bf16", 0, False),
    (2000, 64, 777, "diag", "f16", 16, False),
    (500, 1, 100, "diag", "bf16", 0, False),      # D = 1
    (777, 2, 300, "iso", "f16", 1, True),         # D = 2, two slices, element-wise loads
]


@pytest.mark.parametrize("n,d,k,cov,x_dtype,ldx_pad,misalign", CASES,
                         ids=[f"n{a}-d{b}-k{c}-{e}-{f}-pad{g}-mis{int(h)}" for a, b, c, e, f, g, h in CASES])
def test_ragged_shapes(gmm_lib, n, d, k, cov, x_dtype, ldx_pad, misalign):
    xd, xg, ldx, th0 = _make(n, d, k, cov, x_dtype, ldx_pad, misalign, seed=n * 13 + d * 5 + k)
    gm = gmm_lib.Gmm(n, d, k, cov, x_dtype, ldx=ldx)
    th = to_dev(*th0)
    p = params64(cov, *th)
    # E-step alone: LL, per-point log-normaliser and argmax
    ll_e, lse, arg = gpu_loglik(gm, xg, th)
    lse_ref = check_argmax(xd, p, arg, what=f"n{n} d{d} k{k} {cov} {x_dtype} loglik")
    print(f"   per-point lse max abs err {np.max(np.abs(lse - lse_ref)):.3e}", flush=True)
    # one EM step from well-conditioned parameters
    assert not ill_conditioned(th0, xd, cov)
    ll, st, th1 = gpu_step(gm, xg, *th)
    ref = oracle.em_step(xd, p)
    check_reduced(ref, ll, st, th1, what="  em step")
    assert abs(st.s0.sum().item() - n) <= 1e-3 * n
    assert metrics.rel(ll_e, ref.ll) <= LL_TOL
    assert abs(ll_e - ll) <= 1e-6 * abs(ll) + 1e-6   # same scores as the fused step
    # second iteration from the GPU's parameters (finalize prepared them)
    ll2, st2, th2 = gpu_step(gm, xg, *th1, prepare=False)
    ref2 = oracle.em_step(xd, params64(cov, *th1))
    check_later_step(ref2, ll2, st2, th2, th1, xd, cov, what="  second step")


@pytest.mark.parametrize("name,n", [("iso-bf16-n1e7-d128-k256", 60_000),
                                    ("diag-bf16-n2e8-d128-k1024", 9_000)])
def test_workload_shapes_subset(gmm_lib, name, n):
    """The benchmark workloads' mixtures at a size the oracle finishes in
    seconds: one step plus the E-step's argmax, then a second step."""
    w, x, th0 = workload_inputs(name, n=n)
    xd = x.double().numpy()
    xg = x.cuda()
    gm = gmm_lib.Gmm(w.n, w.d, w.k, w.cov, w.x_dtype)
    th = to_dev(*th0)
    p = params64(w.cov, *th)
    _, lse, arg = gpu_loglik(gm, xg, th)
    check_argmax(xd, p, arg, what=f"{name} loglik")
    assert not ill_conditioned(th0, xd, w.cov)
    ll, st, th1 = gpu_step(gm, xg, *th)
    ref = oracle.em_step(xd, p)
    check_reduced(ref, ll, st, th1, what="  em step")
    ll2, st2, th2 = gpu_step(gm, xg, *th1, prepare=False)
    p2 = params64(w.cov, *th1)
    ref2 = oracle.em_step(xd, p2)
    check_later_step(ref2, ll2, st2, th2, th1, xd, w.cov, what="  second step")
    _, _, arg2 = gpu_loglik(gm, xg, th1)
    check_argmax(xd, p2, arg2, what="  loglik at theta_1")


XC_CASES = [
    # n, d, k, cov, x_dtype, ldx_pad, misalign: one slice (fused kernel) and
    # several (two sweeps); vector and element-wise row loads
    (4000, 32, 100, "iso", "bf16", 0, False),
    (4000, 32, 100, "diag", "bf16", 0, False),
    (3000, 48, 300, "diag", "bf16", 0, False),
    (3000, 24, 520, "iso", "bf16", 0, False),
    (2000, 17, 300, "diag", "f16", 3, True),
    (2500, 40, 100, "iso", "f16", 0, False),
]


@pytest.mark.parametrize("n,d,k,cov,x_dtype,ldx_pad,misalign", XC_CASES,
                         ids=[f"n{a}-d{b}-k{c}-{e}-{f}-pad{g}-mis{int(h)}" for a, b, c, e, f, g, h in XC_CASES])
def test_exact_components(gmm_lib, n, d, k, cov, x_dtype, ldx_pad, misalign):
    """Components collapsed onto single points far from the data mean
    (variance 1e-4 at a stored point): their fp16 expanded-form score is off
    by thousands of nats, so the library takes them out of the panel and
    scores them in the exact centred form ([LP-GMM] 1.2, the density; 1.3,
    exp / log / statistics in fp32).  Against the oracle: LL, argmax, the
    E-step's per-point log-normaliser, the reduced-precision gate of the
    step, the collapsed components' s0 / s1 / s2 element by element, the
    top-m lists, and a second step from the GPU's own parameters."""
    xd, xg, ldx, (pi0, mu0, cov0) = _make(n, d, k, cov, x_dtype, ldx_pad, misalign, seed=7 * k + d)
    rng = np.random.default_rng(k + 1)
    pick = np.sort(rng.choice(k, size=6, replace=False))
    far = np.argsort(-np.abs(xd - xd.mean(0)).sum(1))[:6]   # the points furthest out
    mu0[pick] = xd[far].astype(np.float32)                    # stored values: exact
    cov0[pick] = 1e-4
    ill = ill_conditioned((pi0, mu0, cov0), xd, cov)
    assert set(pick.tolist()) <= set(ill), (pick, ill[:16])
    gm = gmm_lib.Gmm(n, d, k, cov, x_dtype, ldx=ldx)
    th = to_dev(pi0, mu0, cov0)
    p = params64(cov, *th)
    what = f"n{n} d{d} k{k} {cov} {x_dtype}"
    # E-step alone
    ll_e, lse, arg = gpu_loglik(gm, xg, th)
    assert gm.diagnostics().ill_cond >= len(pick)
    lse_ref = check_argmax(xd, p, arg, what=f"{what} loglik")
    for j, kk in zip(far, pick):   # each collapsed component owns its point
        assert arg[j] == kk, (j, arg[j], kk)
    err = np.abs(lse - lse_ref)
    print(f"   lse max abs err {np.max(err):.3e}, at the collapsed points {np.max(err[far]):.3e}", flush=True)
    assert np.max(err[far]) <= 1e-3 * np.max(np.abs(lse_ref[far])) + 1e-2
    # one EM step
    ll, st, th1 = gpu_step(gm, xg, *th)
    ref = oracle.em_step(xd, p)
    check_reduced(ref, ll, st, th1, what=f"  em step {what}")
    assert abs(ll_e - ll) <= 1e-6 * abs(ll) + 1e-6
    # the collapsed components' statistics, element by element: gamma =
    # exp2(S - lse) with fp32 scores |S| up to a few hundred (base 2), so a
    # relative error up to ~2^-24 * 300 * ln 2 ~ 1.2e-5; the bar is 1e-4
    for name, got, want in (("s0", st.s0, ref.nk), ("s1", st.s1, ref.s1), ("s2", st.s2, ref.s2)):
        stats_elementwise(got.cpu().numpy()[pick], np.asarray(want)[pick], 1e-4, 1e-6, what=f"{name} collapsed")
    # top-m lists: the collapsed component first on its point, responsibility ~1
    m = 4
    gm.prepare(*th)   # finalize moved the library's theta on
    idx, gam = gm.assign(xg, m)
    idx, gam = idx.cpu().numpy(), gam.cpu().numpy()
    ridx, rgam, _ = oracle.assign_topm(xd, p, m)
    assert np.array_equal(idx[:, 0], arg)
    for j, kk in zip(far, pick):
        assert idx[j, 0] == kk and abs(gam[j, 0] - rgam[j, 0]) <= 1e-4, (j, idx[j], gam[j], ridx[j], rgam[j])
    agree = float(np.mean(idx[:, 0] == ridx[:, 0]))
    assert agree >= ARGMAX_MIN, agree
    # second step from the GPU's parameters (the collapsed ones stay collapsed)
    ll2, st2, th2 = gpu_step(gm, xg, *th1)
    ref2 = oracle.em_step(xd, params64(cov, *th1))
    check_later_step(ref2, ll2, st2, th2, th1, xd, cov, what=f"  second step {what}")


def test_largest_k(gmm_lib):
    """K = 4096, the largest the large-K family takes (16 slices, the merge of
    17 rows with an exactly scored component among them): 4096 separated
    isotropic clusters of three points each in D = 8, the components started
    near them; the E-step argmax, one step and a second step against the
    oracle."""
    rng = np.random.default_rng(4096)
    n, d, k = 3 * 4096, 8, 4096
    mu_t = rng.uniform(-60.0, 60.0, size=(k, d))
    z = np.repeat(np.arange(k), 3)
    xf = (mu_t[z] + 0.5 * rng.standard_normal((n, d))).astype(np.float32)
    xs = torch.from_numpy(xf).to(torch.bfloat16)
    xd = xs.double().numpy()
    mu0 = (mu_t + 0.1 * rng.standard_normal((k, d))).astype(np.float32)
    cov0 = rng.uniform(0.2, 0.4, size=k).astype(np.float32)
    mu0[7], cov0[7] = xd[3 * 7], 1e-4   # one component collapsed onto a point: scored exactly
    pi0 = np.full(k, 1.0 / k, np.float32)
    gm = gmm_lib.Gmm(n, d, k, "iso", "bf16")
    xg = xs.cuda()
    th = to_dev(pi0, mu0, cov0)
    p = params64("iso", *th)
    _, lse, arg = gpu_loglik(gm, xg, th)
    assert gm.diagnostics().ill_cond >= 1
    check_argmax(xd, p, arg, what="k4096 loglik")
    ll, st, th1 = gpu_step(gm, xg, *th)
    ref = oracle.em_step(xd, p)
    check_reduced(ref, ll, st, th1, what="  k4096 em step")
    ll2, st2, th2 = gpu_step(gm, xg, *th1, prepare=False)
    ref2 = oracle.em_step(xd, params64("iso", *th1))
    check_later_step(ref2, ll2, st2, th2, th1, xd, "iso", what="  k4096 second step")


def test_determinism_bitwise(gmm_lib):
    w, x, th0 = workload_inputs("diag-bf16-n2e8-d128-k1024", n=50_001)
    xg = x.cuda()
    gm = gmm_lib.Gmm(w.n, w.d, w.k, w.cov, w.x_dtype)
    out = []
    for _ in range(2):
        ll, st, th = gpu_step(gm, xg, *to_dev(*th0))
        out.append((ll, st.s0.cpu(), st.s1.cpu(), st.s2.cpu(), *[t.cpu() for t in th]))
    assert out[0][0] == out[1][0]
    for a, b in zip(out[0][1:], out[1][1:]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("cov", ["iso", "diag"])
def test_degenerate_cases(gmm_lib, cov):
    """A far outlier (finite one-hot responsibility), an empty component
    (keeps mu and variance), data far from the origin (centring and the
    per-dimension power-of-two scale), K = 1 (sample mean and variance)."""
    rng = np.random.default_rng(11)
    n, d, k = 3000, 32, 300
    x = (1000.0 + 100.0 * rng.standard_normal((n, d))).astype(np.float32)
    x[7] = 5000.0
    xb = torch.from_numpy(x).to(torch.bfloat16)
    xd = xb.double().numpy()
    mu0 = xb[torch.as_tensor(rng.choice(n, k, replace=False))].float().numpy()
    mu0[5] = 3e4                                          # empty component
    cov0 = np.ones((k, d) if cov == "diag" else (k,), np.float32)
    pi0 = np.full(k, 1.0 / k, np.float32)
    gm = gmm_lib.Gmm(n, d, k, cov, "bf16")
    th = to_dev(pi0, mu0, cov0)
    ll, st, th1 = gpu_step(gm, xb.cuda(), *th)
    ref = oracle.em_step(xd, params64(cov, *th))
    assert np.isfinite(ll)
    check_reduced(ref, ll, st, th1, what=f"offset data {cov}")
    dg = gm.diagnostics()
    assert dg.empty >= 1 and dg.nonfinite == 0 and dg.bad_params == 0
    assert torch.equal(th1[1][5].cpu(), th[1][5].cpu()) and torch.equal(th1[2][5].cpu(), th[2][5].cpu())
    # K = 1
    g1 = gmm_lib.Gmm(n, d, 1, cov, "bf16")
    ll, st, t1 = gpu_step(g1, xb.cuda(), *to_dev(np.ones(1), np.zeros((1, d)),
                                                 np.ones((1, d) if cov == "diag" else 1)))
    np.testing.assert_allclose(t1[1].cpu().numpy()[0], xd.mean(0), rtol=1e-5)
    want_var = xd.var(0) if cov == "diag" else np.array([xd.var(0).mean()])
    np.testing.assert_allclose(t1[2].cpu().numpy().ravel(), np.ravel(want_var), rtol=2e-2)
    assert t1[0].item() == 1.0


def test_range_and_nan_flags(gmm_lib):
    """The fp16 scale comes from an evenly strided sample of rows (every
    second row at N = 8192); a value on an unsampled row far outside the
    sample's range cannot be staged in fp16: the pass fails visibly (LL is
    NaN, the range and non-finite flags are set, finalize keeps theta), and
    so does a NaN in X."""
    rng = np.random.default_rng(12)
    n, d, k = 8192, 16, 100
    x = rng.standard_normal((n, d)).astype(np.float32)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    th = to_dev(np.full(k, 1.0 / k), xb[:k].float().numpy(), np.ones((k, d)))
    gm = gmm_lib.Gmm(n, d, k, "diag", "bf16")
    ll, _, _ = gpu_step(gm, xb.cuda(), *th)
    dg = gm.diagnostics()
    assert dg.x_range == 0 and dg.nonfinite == 0 and np.isfinite(ll)
    xo = xb.clone()
    xo[3, 4] = 3000.0          # unsampled row; (y')^2 beyond the fp16 range
    ll, _, th1 = gpu_step(gm, xo.cuda(), *th)
    dg = gm.diagnostics()
    assert dg.x_range == 1 and dg.nonfinite == 1 and np.isnan(ll)
    for a, b in zip(th1, th):
        assert torch.equal(a.cpu(), b.cpu())   # theta kept
    xn = xb.clone()
    xn[9, 1] = float("nan")
    gpu_step(gm, xn.cuda(), *th)
    dg = gm.diagnostics()
    assert dg.x_range == 1 or dg.nonfinite == 1


@pytest.mark.parametrize("name", ["iso-bf16-n1e7-d128-k256", "diag-bf16-n2e8-d128-k1024"])
def test_full_size_workload(gmm_lib, name):
    """Full-size workload in the benchmark's launch configuration: properties
    that hold at any size (sum of s0 = N, LL = sum of per-point LSE, fused
    and E-only LL agree) and per-point LSE / argmax on sampled points against
    the oracle."""
    w = synth.WORKLOADS[name]
    mix = synth.make_mixture(w)
    print(f"sampling {w.n} points on the GPU...", flush=True)
    xg = synth.sample_points(w, mix, device="cuda")
    th0 = synth.init_params(w, xg)
    gm = gmm_lib.Gmm(w.n, w.d, w.k, w.cov, w.x_dtype)
    th = to_dev(*th0)
    ll, st, th1 = gpu_step(gm, xg, *th)
    s0 = st.s0.cpu().numpy()
    assert abs(s0.sum() - w.n) <= 1e-4 * w.n, s0.sum()
    ll_e, lse, arg = gpu_loglik(gm, xg, th)
    assert metrics.rel(ll_e, ll) <= 1e-6
    assert metrics.rel(np.sum(lse, dtype=np.float64), ll) <= 1e-5
    idx = np.sort(np.random.default_rng(0).choice(w.n, 3000, replace=False))
    xs = xg[torch.as_tensor(idx, device="cuda")].double().cpu().numpy()
    p = params64(w.cov, *th)
    ll_s, lse_ref, arg_ref = oracle.loglik(xs, p)
    err = np.abs(lse[idx] - lse_ref) / np.abs(lse_ref)
    agree = float(np.mean(arg[idx] == arg_ref))
    print(f"{name}: sampled lse rel err max {err.max():.2e}, argmax agreement {agree * 100:.2f}%",
          flush=True)
    assert metrics.rel(np.sum(lse[idx], dtype=np.float64), ll_s) <= LL_TOL
    assert agree >= ARGMAX_MIN
    assert np.all(np.isfinite(th1[1].cpu().numpy())) and np.all(th1[2].cpu().numpy() > 0)
