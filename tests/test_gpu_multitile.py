"""GPU parity at sizes where every block walks many 64-row tiles.

The fused kernels keep a block's statistics in registers across all the
tiles of its row chunk, double-buffer the X tiles (16-byte global->LDS
copies for fp32 rows, a register prefetch widened into LDS for half-precision
rows) and, in the two-pass regime, run one block per (chunk, 256-component
slab). At the small sizes of the element-wise tests every block takes a
single tile, so none of that machinery is reached there. These cases are
sized so that each block walks 4 to 64 tiles (asserted through the
launch-shape query), and compare against the float64 oracle:

  * all of Nk, Sx, Sxx and L (expanded form, BLAS) at the 1e-4 bars;
  * l_n of every row against the oracle;
  * the responsibilities of 256 seeded rows, taken from R materialised by a
    launch of the same shape (same N, d, K, regime: same plan);
  * with the split-bf16 statistics contraction: statistics against the
    oracle, l_n bitwise those of the fp32 contraction.

The IVF recipe's EM iterations are teacher-forced: each GPU E-step and
M-step is compared with the oracle on the GPU's own parameters.
"""
import numpy as np
import pytest

import oracle
from soft_clustering_gmm_amd import datagen
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture()
def G():
    from soft_clustering_gmm_amd import gmm
    gmm.lib()
    gmm.set_stats_precision(gmm.STATS_AUTO)  # the library's default
    yield gmm
    gmm.set_stats_precision(gmm.STATS_AUTO)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t):
    return t.detach().cpu().numpy()


def _xdev(X, xkind):
    """X on the device as float32, float16 or bfloat16, and the values the oracle sees."""
    if xkind == "f32":
        return dev(X.astype(np.float32)), X.astype(np.float32)
    if xkind == "f16":
        Xh = X.astype(np.float16)
        return dev(Xh), Xh.astype(np.float32)
    Xb = torch.from_numpy(np.ascontiguousarray(X, dtype=np.float32)).to(torch.bfloat16)
    return Xb.to("cuda"), Xb.float().numpy()


def _check_case(G, Xd, Xv, mu, var, logw, regime, what, min_tiles, split=(False,), sample=256):
    N, d = Xv.shape
    K = mu.shape[0]
    info = G.plan_info(N, d, K, regime)
    tiles = info["rows_per_chunk"] // 64
    print(f"{what}: N={N} d={d} K={K} plan {info}, {tiles} tiles per block", flush=True)
    assert tiles >= min_tiles, f"{what}: only {tiles} tiles per block"
    ref = oracle.estep(Xv, mu, var, logw, form="expanded", row_chunk=4096, abs_x=True)
    rows = np.sort(np.random.default_rng(99).choice(N, min(sample, N), replace=False))
    l_rows, R_rows = oracle.estep_rows(Xv, mu, var, logw, rows)
    args = (Xd, dev(mu), dev(var), dev(logw))
    l_fp32 = None
    for sp in split:  # False: fp32 products, True: split-bf16, "auto": the default mode
        G.set_stats_precision({False: G.STATS_FP32, True: G.STATS_SPLIT_BF16, "auto": G.STATS_AUTO}[sp])
        tag = f"{what} {'split-bf16' if sp is True else 'auto' if sp == 'auto' else 'fp32'}"
        Nk, Sx, Sxx, L, lp = G.estep_stats(*args, regime=regime, want_point_loglik=True)
        torch.cuda.synchronize()
        es = parity.check_stats((host(Nk), host(Sx), host(Sxx)), ref, None, ref["absx"], tag)
        parity.check_total(host(L), ref, tag)
        el = parity.check_loglik_point(host(lp), ref["l"], tag + " l_n (all rows)")
        parity.check_loglik_point(host(lp)[rows], l_rows, tag + " l_n (sampled, difference form)")
        if l_fp32 is None:
            l_fp32 = host(lp)
            R, lr = G.estep_resp(*args, regime=regime)
            torch.cuda.synchronize()
            assert np.array_equal(host(lr), l_fp32), f"{tag}: l_n of the resp launch differs"
            er = parity.check_resp(host(R[torch.from_numpy(rows).to("cuda")]), R_rows, tag + " sampled r")
            del R
        else:
            assert np.array_equal(host(lp), l_fp32), f"{tag}: l_n differs from the fp32 contraction"
            er = float("nan")
        print(f"{tag}: stats {es[0]:.1e}/{es[1]:.1e}/{es[2]:.1e}  l_n {el:.1e}  sampled |dr| {er:.1e}",
              flush=True)
        G.set_stats_precision(G.STATS_AUTO)
    return ref


@pytest.mark.parametrize("scale", [1.0, 0.1])
def test_two_pass_fp32_many_tiles(G, scale):
    """largek recipe at N = 65536: 16 slabs, 64 tiles per block, fp32 X through the
    asynchronous global->LDS tile copies (scale 0.1: dense responsibilities)."""
    X, mu, var, logw = datagen.make_workload("largek", N=65536, centre_scale=scale)
    Xd, Xv = _xdev(X, "f32")
    _check_case(G, Xd, Xv, mu, var, logw, 2, f"largek x{scale}", 32, split=(False, True))


def test_two_pass_fp16_prefetch_many_tiles(G):
    """ivf recipe at N = 131072, X in fp16: 4 slabs, 32 tiles per block, the
    half-precision register prefetch of the next tile; statistics as fp32
    products, split-bf16 products and (the default) exact fp16 splits."""
    X, mu, var, logw = datagen.make_workload("ivf", N=131072)
    Xd, Xv = _xdev(X, "f16")
    _check_case(G, Xd, Xv, mu, var, logw, 2, "ivf fp16", 16, split=(False, True, "auto"))


@pytest.mark.parametrize("xkind", ["bf16", "f16", "f32"])
def test_single_sweep_d96_many_tiles(G, xkind):
    """Single sweep, d = 96 (three feature tiles), K = 256, N = 65536: 4 tiles
    per block through the half-precision prefetch (bf16, fp16) or the
    asynchronous fp32 copies."""
    X, mu, var, logw = datagen.random_problem(4096, 65536, 96, 256)
    Xd, Xv = _xdev(X, xkind)
    _check_case(G, Xd, Xv, mu, var, logw, 1, f"single d=96 {xkind}", 4, split=(False, True))


@pytest.mark.parametrize("N,d,K", [(262144, 32, 64), (131072, 64, 128), (131072, 99, 200)])
def test_single_sweep_narrow_many_tiles(G, N, d, K):
    """Single sweep with one, two or four waves per block and one to four feature
    tiles (d = 99: ragged rows through the element-wise tile load), 4 tiles per block."""
    X, mu, var, logw = datagen.random_problem(5000 + d, N, d, K)
    Xd, Xv = _xdev(X, "f32")
    _check_case(G, Xd, Xv, mu, var, logw, 1, f"single N={N} d={d} K={K}", 4)


def test_ivf_em_teacher_forced_many_tiles(G):
    """Five EM iterations of the ivf recipe at N = 131072 (fp16 X, two-pass):
    each GPU E-step against the oracle on the GPU's own parameters, each
    M-step against the oracle's M-step on the GPU's statistics; then the
    on-device loop reproduces the step-by-step run bit for bit."""
    X, mu, var, logw = datagen.make_workload("ivf", N=131072)
    Xd, Xv = _xdev(X, "f16")
    N = Xv.shape[0]
    floor = 1e-6
    mud, vard, lwd = dev(mu.copy()), dev(var.copy()), dev(logw.copy())
    hist = []
    for t in range(5):
        m0, v0, w0 = host(mud), host(vard), host(lwd)
        Nk, Sx, Sxx, L, lp = G.estep_stats(Xd, mud, vard, lwd, want_point_loglik=True)
        torch.cuda.synchronize()
        ref = oracle.estep(Xv, m0, v0, w0, form="expanded", row_chunk=4096, abs_x=True)
        what = f"ivf EM iteration {t}"
        parity.check_loglik_point(host(lp), ref["l"], what)
        es = parity.check_stats((host(Nk), host(Sx), host(Sxx)), ref, None, ref["absx"], what)
        parity.check_total(host(L), ref, what)
        hist.append(float(L))
        G.mstep(Nk, Sx, Sxx, N, floor, mud, vard, lwd)
        torch.cuda.synchronize()
        rm, rv, rl = oracle.mstep(host(Nk), host(Sx), host(Sxx), N, floor, m0, v0)
        np.testing.assert_allclose(host(mud), rm.astype(np.float32), rtol=1e-6, atol=1e-6)
        np.testing.assert_allclose(host(vard), rv.astype(np.float32), rtol=1e-6, atol=1e-7)
        np.testing.assert_allclose(host(lwd), rl.astype(np.float32), rtol=1e-6, atol=1e-6)
        print(f"{what}: L {float(L):.6e}  stats {es[0]:.1e}/{es[1]:.1e}/{es[2]:.1e}", flush=True)
    hist = np.array(hist)
    assert (np.diff(hist) >= -1e-6 * np.abs(hist[:-1])).all(), hist
    mu2, var2, lw2 = dev(mu.copy()), dev(var.copy()), dev(logw.copy())
    h2 = G.em_iterate(Xd, mu2, var2, lw2, 5, floor)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(h2), hist)
    assert torch.equal(mu2, mud) and torch.equal(var2, vard) and torch.equal(lw2, lwd)


def test_two_pass_fp16_out_of_range_takes_fp32_products(G):
    """Half-precision X with rows of |x|^2 >= 225, where the fp16 split of (16 x)^2
    is not known to stay in the fp16 range: the default mode's second pass must hand
    the statistics to its fp32 twin, so that everything is bitwise what
    GMM_STATS_FP32 gives, and meets the oracle. (ivf recipe at N = 32768 scaled by
    20, so |x|^2 = 400 on every row; variances by 400.)"""
    X, mu, var, logw = datagen.make_workload("ivf", N=32768)
    X20 = (X.astype(np.float32) * 20.0).astype(np.float16)
    assert (X20.astype(np.float64) ** 2).sum(axis=1).max() >= 225.0
    mu20, var20 = (mu * 20.0).astype(np.float32), (var * 400.0).astype(np.float32)
    Xd, Xv = dev(X20), X20.astype(np.float32)
    args = (Xd, dev(mu20), dev(var20), dev(logw))
    G.set_stats_precision(G.STATS_AUTO)
    a = G.estep_stats(*args, regime=2, want_point_loglik=True)
    G.set_stats_precision(G.STATS_FP32)
    b = G.estep_stats(*args, regime=2, want_point_loglik=True)
    torch.cuda.synchronize()
    for i, key in enumerate(("Nk", "Sx", "Sxx", "L", "l_n")):
        assert torch.equal(a[i], b[i]), f"out-of-range fp16 X: {key} differs from the fp32 products"
    ref = oracle.estep(Xv, mu20, var20, logw, form="expanded", row_chunk=4096, abs_x=True)
    parity.check_stats((host(a[0]), host(a[1]), host(a[2])), ref, None, ref["absx"], "out-of-range fp16 X")
    parity.check_total(host(a[3]), ref, "out-of-range fp16 X")


@pytest.mark.parametrize("N,d,K,scale", [(1001, 37, 300, 0.25), (65, 1, 257, 1.0), (700, 64, 520, 0.25),
                                         (129, 96, 1024, 0.25), (2000, 40, 300, 2.0 ** -8)])
def test_two_pass_fp16_edge_shapes(G, N, d, K, scale):
    """Half-precision X through the two-pass regime at ragged shapes (N not a
    tile multiple, d not a multiple of the feature tile, K just past a
    256-component slab), with fp32 products and with the default fp16 splits:
    statistics, L and every l_n against the oracle, sampled r, and l_n bitwise
    equal between the two modes. Every row has |x|^2 < 225, so the default
    mode takes the fp16 splits. The 2^-8 case puts most |x| below 2^-6, where
    (16 x)^2 no longer splits exactly into two fp16 values."""
    X, mu, var, logw = datagen.random_problem(7000 + N + d + K, N, d, K)
    X = (X * scale).astype(np.float32)
    mu = (mu * scale).astype(np.float32)
    var = (var * scale * scale).astype(np.float32)
    Xd, Xv = _xdev(X, "f16")
    assert (Xv.astype(np.float64) ** 2).sum(axis=1).max() < 225.0
    if scale < 0.01:
        assert (np.abs(Xv) < 2.0 ** -6).mean() > 0.5
    _check_case(G, Xd, Xv, mu, var, logw, 2, f"fp16 two-pass N={N} d={d} K={K} scale={scale}", 0,
                split=(False, "auto"))
    # the default mode took the fp16 splits (not its fp32 twin): its products differ
    args = (Xd, dev(mu), dev(var), dev(logw))
    G.set_stats_precision(G.STATS_AUTO)
    a = G.estep_stats(*args, regime=2)
    G.set_stats_precision(G.STATS_FP32)
    b = G.estep_stats(*args, regime=2)
    torch.cuda.synchronize()
    assert not torch.equal(a[2], b[2]), "fp16 X in range: the default mode gave the fp32 products"
