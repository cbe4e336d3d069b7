"""The C-ABI library loads, exports every symbol gmm.h declares, and rejects bad
arguments on the host before touching any GPU (these tests need no GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("gmm.h", "gmm_peaks.h")]
LIB = os.path.join(ROOT, "soft_clustering_gmm_amd", "libgmm_mi355x.so")

P = ctypes.c_void_p


def declared():
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == sorted(os.path.basename(h) for h in HEADERS)
    src = "\n".join(open(h).read() for h in HEADERS)
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gmm_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} not built: run __graft_entry__.build()")
    from soft_clustering_gmm_amd import gmm
    return gmm.lib()


def test_exports_every_declared_symbol(L):
    names = declared()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
    from soft_clustering_gmm_amd import gmm
    assert set(gmm.EXPORTS) == set(names)


def test_peak_probes_validate_on_the_host(L):
    assert L.gmm_peak_mfma(2, 10, 4, FAKE, None) == -1
    assert L.gmm_peak_mfma(0, 0, 4, FAKE, None) == -1
    assert L.gmm_peak_mfma(0, 10, 4, None, None) == -1
    assert L.gmm_peak_mfma_flops(0, 10, 4) == 8 * 4096 * 4 * 4 * 10
    assert L.gmm_peak_mfma_flops(1, 10, 4) == 8 * 2048 * 4 * 4 * 10
    assert L.gmm_peak_hbm_read(None, 1 << 20, 4, FAKE, None) == -1
    assert L.gmm_peak_hbm_read(ctypes.c_void_p(0x100004), 1 << 20, 4, FAKE, None) == -1  # misaligned
    assert L.gmm_peak_hbm_read(FAKE, 8, 4, FAKE, None) == -1
    for bad in ((-1, 10, 4, FAKE), (4, 10, 4, FAKE), (0, 0, 4, FAKE), (0, 10, 0, FAKE), (3, 10, 4, None)):
        assert L.gmm_peak_coissue(*bad, None) == -1


def test_version_and_error_strings(L):
    assert L.gmm_version() == 10000
    for code in (0, -1, -2, -3, -4, -5):
        assert len(L.gmm_error_string(code)) >= 2
    assert L.gmm_error_string(-99) == b"unknown status"


def test_stats_precision_setting(L):
    # host-only: the setting is validated and stored, nothing is enqueued
    assert L.gmm_set_stats_precision(7) == -1
    assert L.gmm_set_stats_precision(-1) == -1
    assert L.gmm_set_stats_precision(1) == 0
    assert L.gmm_set_stats_precision(0) == 0
    assert L.gmm_set_stats_precision(2) == 0  # the default (auto) mode


def test_workspace_bytes(L):
    assert L.gmm_workspace_bytes(0, 0, 8) == 0
    assert L.gmm_workspace_bytes(10, 129, 8) == 0
    assert L.gmm_workspace_bytes(10, 4, 70000) == 0
    small = L.gmm_workspace_bytes(4096, 16, 8)
    big = L.gmm_workspace_bytes(1 << 20, 128, 256)
    assert 0 < small < big
    assert L.gmm_workspace_bytes(1 << 20, 128, 256) % 256 == 0


def test_plan_info_launch_shapes(L):
    """Host-only launch-shape query: regime choice, slabs and tiles per block."""
    from soft_clustering_gmm_amd import gmm
    assert L.gmm_plan_info(10, 4, 3, 0, None) == -1
    buf = (ctypes.c_int64 * 7)()
    assert L.gmm_plan_info(10, 0, 3, 0, buf) == -1
    assert L.gmm_plan_info(10, 4, 300, 1, buf) == -2
    ref = gmm.plan_info(1 << 20, 128, 256)
    assert ref["regime"] == 1 and ref["waves"] == 8 and ref["kslabs"] == 1 and ref["tiles"] == 16384
    assert ref["chunks"] * ref["rows_per_chunk"] >= 1 << 20
    lk = gmm.plan_info(1 << 22, 128, 4096)
    assert lk["regime"] == 2 and lk["kslabs"] == 16
    assert gmm.plan_info(1 << 24, 32, 16)["regime"] == 3
    # the reduced-size cases of the multi-tile parity tests walk several tiles per block
    assert gmm.plan_info(65536, 128, 4096)["rows_per_chunk"] // 64 >= 32
    assert gmm.plan_info(131072, 96, 1024)["rows_per_chunk"] // 64 >= 16
    assert gmm.plan_info(65536, 96, 256)["rows_per_chunk"] // 64 >= 4


FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: every call below fails validation first


def test_static_entry_point_rejects_on_the_host(L):
    """The allocation-free E-step validates its arguments and rejects shapes whose
    plan needs more than the static scratch, before touching any device."""
    from soft_clustering_gmm_amd import gmm

    def call(X=FAKE, xt=0, N=100, d=4, K=3, nk=FAKE):
        return L.gmm_estep_stats_static(X, xt, N, d, FAKE, FAKE, FAKE, K, nk, FAKE, FAKE, FAKE, None, None)

    assert call(d=0) == -1 and call(xt=9) == -1 and call(X=None) == -1 and call(nk=None) == -1
    assert call(d=129) == -2
    cap = 128 << 20
    big = gmm.plan_info(1 << 22, 128, 4096)["scratch_bytes"]
    assert big > cap and call(N=1 << 22, d=128, K=4096) == -5
    assert b"static" in L.gmm_error_string(-5) and b"128 MiB" in L.gmm_error_string(-5)
    ref = gmm.plan_info(1 << 20, 128, 256)["scratch_bytes"]
    assert ref <= cap, ref  # the headline shape fits (the header quotes about 68 MiB)
    assert abs(ref / 2 ** 20 - 68) < 1.5
    assert gmm.plan_info(1 << 24, 32, 16)["scratch_bytes"] < 16 << 20  # small-K: no per-row region


def _estep(L, X=FAKE, xt=0, N=100, d=4, K=3, ws=FAKE, wsb=1 << 40, regime=0, nk=FAKE):
    return L.gmm_estep_stats_regime(X, xt, N, d, FAKE, FAKE, FAKE, K, nk, FAKE, FAKE, FAKE, None,
                                    ws, wsb, regime, None)


def test_estep_argument_validation(L):
    assert _estep(L, d=0) == -1
    assert _estep(L, N=-1) == -1
    assert _estep(L, K=0) == -1
    assert _estep(L, xt=7) == -1
    assert _estep(L, X=None) == -1
    assert _estep(L, nk=None) == -1
    assert _estep(L, d=129) == -2
    assert _estep(L, K=70000) == -2
    assert _estep(L, ws=None) == -3
    assert _estep(L, ws=ctypes.c_void_p(0x100010)) == -3   # misaligned
    assert _estep(L, wsb=16) == -3                         # too small
    assert _estep(L, K=300, regime=1) == -2                # single sweep needs K <= 256
    assert _estep(L, regime=5) == -1
    assert _estep(L, K=17, regime=3) == -2                 # small-K needs K <= 16
    assert _estep(L, d=65, regime=3) == -2                 # ... and d <= 64


def test_other_entry_points_validate(L):
    # mstep: N must be >= 1, floor >= 0
    assert L.gmm_mstep(FAKE, FAKE, FAKE, 0, 4, 3, ctypes.c_float(1e-6), FAKE, FAKE, FAKE, None) == -1
    assert L.gmm_mstep(FAKE, FAKE, FAKE, 10, 4, 3, ctypes.c_float(-1.0), FAKE, FAKE, FAKE, None) == -1
    assert L.gmm_mstep(None, FAKE, FAKE, 10, 4, 3, ctypes.c_float(1e-6), FAKE, FAKE, FAKE, None) == -1
    # em_iterate: N >= 1, iters >= 0, history pointer needed
    assert L.gmm_em_iterate(FAKE, 0, 0, 4, 3, 2, ctypes.c_float(1e-6), FAKE, FAKE, FAKE, FAKE, FAKE,
                            1 << 40, None) == -1
    assert L.gmm_em_iterate(FAKE, 0, 10, 4, 3, -1, ctypes.c_float(1e-6), FAKE, FAKE, FAKE, FAKE, FAKE,
                            1 << 40, None) == -1
    assert L.gmm_em_iterate(FAKE, 0, 10, 4, 3, 2, ctypes.c_float(1e-6), FAKE, FAKE, FAKE, None, FAKE,
                            1 << 40, None) == -1
    # top2 / resp: outputs needed, workspace checked
    assert L.gmm_assign_top2(FAKE, 0, 10, 4, FAKE, FAKE, FAKE, 3, None, FAKE, FAKE, 1 << 40, None) == -1
    assert L.gmm_assign_top2(FAKE, 0, 10, 4, FAKE, FAKE, FAKE, 3, FAKE, FAKE, FAKE, 8, None) == -3
    assert L.gmm_estep_resp(FAKE, 0, 10, 4, FAKE, FAKE, FAKE, 3, None, None, FAKE, 1 << 40, 0, None) == -1
    assert L.gmm_estep_resp(FAKE, 1, 10, 4, FAKE, FAKE, FAKE, 3, FAKE, None, FAKE, 1 << 40, 9, None) == -1


def _chunked(L, X=FAKE, xt=0, N=100, d=4, K=3, chunk=10, ws=FAKE, wsb=1 << 40):
    return L.gmm_estep_stats_chunked(X, xt, N, d, FAKE, FAKE, FAKE, K, FAKE, FAKE, FAKE, FAKE, None, chunk,
                                     ws, wsb, None)


def test_chunked_argument_validation(L):
    assert _chunked(L, chunk=0) == -1
    assert _chunked(L, chunk=-5) == -1
    assert _chunked(L, xt=3) == -1
    assert _chunked(L, X=None) == -1
    assert _chunked(L, d=129) == -2
    assert _chunked(L, ws=None) == -3
    assert _chunked(L, ws=ctypes.c_void_p(0x100010)) == -3
    assert _chunked(L, wsb=64) == -3


def test_chunked_workspace_bytes(L):
    assert L.gmm_workspace_bytes_chunked(100, 4, 3, 0, 0) == 0
    assert L.gmm_workspace_bytes_chunked(100, 4, 3, 10, 3) == 0
    assert L.gmm_workspace_bytes_chunked(100, 4, 3, 10, 2) > 0   # bfloat16 X
    assert L.gmm_workspace_bytes_chunked(100, 200, 3, 10, 0) == 0
    chunked = L.gmm_workspace_bytes_chunked(1 << 20, 128, 256, 1 << 16, 0)
    # the workspace holds chunk-sized regions only: it does not grow with N
    assert chunked > 2 * (1 << 16) * 128 * 4
    assert L.gmm_workspace_bytes_chunked(1 << 30, 128, 256, 1 << 16, 0) == chunked
    assert L.gmm_workspace_bytes_chunked(1 << 30, 128, 256, 1 << 16, 0) < L.gmm_workspace_bytes(1 << 30, 128, 256)
    assert L.gmm_workspace_bytes_chunked(1 << 20, 128, 256, 1 << 16, 1) < chunked  # fp16 staging
    assert chunked % 256 == 0


def test_border_lists_argument_validation(L):
    def call(idx=FAKE, resp=FAKE, N=100, K=8, off=FAKE, mem=FAKE, cap=200, ws=FAKE, wsb=1 << 40):
        return L.gmm_border_lists(idx, resp, N, K, 0.1, off, mem, cap, ws, wsb, None)
    assert call(N=-1) == -1
    assert call(K=0) == -1
    assert call(K=70000) == -2
    assert call(N=1 << 31) == -2                 # point indices are int32
    assert call(idx=None) == -1
    assert call(idx=ctypes.c_void_p(0x100004)) == -1   # not 8-byte aligned
    assert call(off=None) == -1
    assert call(cap=199) == -1                   # capacity must cover 2N entries
    assert call(ws=None) == -3
    assert call(wsb=8) == -3
    assert L.gmm_border_lists_workspace_bytes(100, 0) == 0
    assert L.gmm_border_lists_workspace_bytes(1 << 20, 1024) > L.gmm_border_lists_workspace_bytes(1 << 20, 256)


def test_kmeans_argument_validation(L):
    def assign(X=FAKE, xt=0, N=100, d=4, K=3, C=FAKE, out=FAKE, ws=FAKE, wsb=1 << 40):
        return L.gmm_kmeans_assign(X, xt, N, d, C, K, out, None, None, ws, wsb, None)
    assert assign(N=-1) == -1
    assert assign(xt=9) == -1
    assert assign(C=None) == -1
    assert assign(out=None) == -1
    assert assign(d=129) == -2
    assert assign(N=1 << 31) == -2
    assert assign(ws=None) == -3
    assert assign(wsb=100) == -3
    assert L.gmm_kmeans_update(FAKE, 0, 100, 4, None, 3, FAKE, None, FAKE, 1 << 40, None) == -1
    assert L.gmm_kmeans_iterate(FAKE, 0, 0, 4, 3, 2, FAKE, FAKE, FAKE, 1 << 40, None) == -1   # N >= 1
    assert L.gmm_kmeans_iterate(FAKE, 0, 10, 4, 3, 2, FAKE, None, FAKE, 1 << 40, None) == -1  # history needed
    assert L.gmm_kmeans_workspace_bytes(100, 4, 0) == 0
    assert L.gmm_kmeans_workspace_bytes(1000, 4, 3) > 0
