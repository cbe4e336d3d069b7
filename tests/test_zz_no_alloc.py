"""The allocation-free E-step (gmm_estep_stats_static) against gmm_estep_stats.

The static entry point runs the same plan and kernels as gmm_estep_stats on
the library's static per-GPU scratch, so its outputs must equal those of the
workspace entry point bit for bit. Calls follow each other on one stream:
the second is smaller than the first (fewer row chunks, so the scratch still
holds the first call's larger contents), the third takes another regime.
The smaller call is also held to the oracle's bars.
"""
import numpy as np
import pytest

import oracle
from soft_clustering_gmm_amd import datagen
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t):
    return t.detach().cpu().numpy()


def _same(a, b, what):
    for i, key in enumerate(("Nk", "Sx", "Sxx", "L", "l_n")):
        assert torch.equal(a[i], b[i]), f"{what}: {key} differs from gmm_estep_stats"


def test_static_matches_workspace_entry_point_on_successive_calls():
    from soft_clustering_gmm_amd import gmm
    gmm.lib()
    gmm.set_stats_precision(gmm.STATS_FP32)
    cases = [("ref", 300_000), ("ref", 70_001), ("smallk", 100_003)]
    for i, (name, N) in enumerate(cases):
        X, mu, var, logw = datagen.make_workload(name, N=N)
        info = gmm.plan_info(*X.shape, mu.shape[0])
        print(f"call {i}: {name} N={N} plan {info}", flush=True)
        args = (dev(X), dev(mu), dev(var), dev(logw))
        s = gmm.estep_stats_static(*args, want_point_loglik=True)
        w = gmm.estep_stats(*args, want_point_loglik=True)
        torch.cuda.synchronize()
        _same(s, w, f"call {i} ({name} N={N})")
        if i == 1:
            ref = oracle.estep(X, mu, var, logw, form="expanded", abs_x=True)
            parity.check_stats((host(s[0]), host(s[1]), host(s[2])), ref, None, ref["absx"], "static call 1")
            parity.check_total(host(s[3]), ref, "static call 1")
            parity.check_loglik_point(host(s[4]), ref["l"], "static call 1")
    # the oracle-sized case once more after the larger calls: still identical
    X, mu, var, logw = datagen.make_workload("tiny")
    args = (dev(X), dev(mu), dev(var), dev(logw))
    s = gmm.estep_stats_static(*args, want_point_loglik=True)
    w = gmm.estep_stats(*args, want_point_loglik=True)
    torch.cuda.synchronize()
    _same(s, w, "tiny after the larger calls")
