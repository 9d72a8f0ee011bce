"""gmm_em_iteration_noalloc (the entry point for callers that cannot
allocate) through the C ABI, against gmm_prepare + gmm_em_step +
gmm_finalize on a caller workspace: LL and the new parameters bit for bit, on
two calls in a row (the second with a smaller input, so the shared internal
workspace is reused with stale contents from the first), for each kernel
family; a descriptor whose workspace exceeds the internal one is refused."""
import ctypes

import numpy as np
import pytest
import torch

from tests.gpu_common import to_dev

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _inputs(n, d, k, cov, x_dtype, seed):
    rng = np.random.default_rng(seed)
    mu_t = rng.uniform(-5, 5, size=(k, d))
    x = (mu_t[rng.integers(0, k, n)] + rng.standard_normal((n, d))).astype(np.float32)
    xg = torch.from_numpy(x).to(DT[x_dtype]).cuda()
    mu0 = xg[torch.as_tensor(rng.choice(n, k, replace=False), device="cuda")].float().cpu().numpy()
    pi0 = np.full(k, 1.0 / k)
    cv = {"diag": np.ones((k, d)), "iso": np.ones(k), "full": np.tile(np.eye(d), (k, 1, 1))}[cov]
    return xg, to_dev(pi0, mu0, cv)


def _noalloc(gmm_lib, desc, th, xg):
    lib = gmm_lib._lib
    ll = torch.zeros(1, dtype=torch.float64, device="cuda")
    outs = [torch.full_like(t, float("nan")) for t in th]
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib.gmm_em_iteration_noalloc(ctypes.byref(desc), p(th[0]), p(th[1]), p(th[2]), p(xg), p(ll),
                                      p(outs[0]), p(outs[1]), p(outs[2]), None)
    assert st == gmm_lib.GMM_OK, gmm_lib.status_str(st)
    torch.cuda.synchronize()
    return ll.item(), [o.cpu() for o in outs]


def _reference(gmm_lib, n, d, k, cov, x_dtype, th, xg):
    gm = gmm_lib.Gmm(n, d, k, cov, x_dtype)
    gm.prepare(*th)
    ll = torch.zeros(1, dtype=torch.float64, device="cuda")
    gm.em_step(xg, ll)
    outs = [torch.empty_like(t) for t in th]
    gm.finalize(*outs)
    torch.cuda.synchronize()
    return ll.item(), [o.cpu() for o in outs]


@pytest.mark.parametrize("cov,x_dtype,d,k,n1,n2", [
    ("diag", "f32", 64, 16, 200_000, 3_001),
    ("iso", "bf16", 128, 256, 60_000, 5_000),
    ("diag", "bf16", 64, 600, 40_000, 777),
    ("full", "f16", 64, 16, 100_000, 2_000),
    ("full", "f16", 128, 20, 20_000, 1_500),   # D = 128: per-group LSE, statistics per quad
])
def test_noalloc_matches_workspace_path(gmm_lib, cov, x_dtype, d, k, n1, n2):
    for n in (n1, n2):   # two calls in a row, the second smaller
        xg, th = _inputs(n, d, k, cov, x_dtype, seed=n)
        desc = gmm_lib.make_desc(n, d, k, cov, x_dtype)
        assert gmm_lib.workspace_bytes(desc) <= gmm_lib._lib.gmm_noalloc_max_workspace()
        ll_a, th_a = _noalloc(gmm_lib, desc, th, xg)
        ll_b, th_b = _reference(gmm_lib, n, d, k, cov, x_dtype, th, xg)
        print(f"{cov} {x_dtype} n={n}: LL {ll_a:.10e} vs {ll_b:.10e}", flush=True)
        assert ll_a == ll_b
        for a, b in zip(th_a, th_b):
            assert torch.equal(a, b)


def test_noalloc_refuses_oversized_plan(gmm_lib):
    desc = gmm_lib.make_desc(2 * 10 ** 8, 128, 1024, "diag", "bf16")
    assert gmm_lib.workspace_bytes(desc) > gmm_lib._lib.gmm_noalloc_max_workspace()
    st = gmm_lib._lib.gmm_em_iteration_noalloc(ctypes.byref(desc), None, None, None, None, None, None,
                                               None, None, None)
    assert st == gmm_lib.GMM_E_WORKSPACE
