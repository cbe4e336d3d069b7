"""The error model of the exact fp16-split statistics (half-precision X, the
second pass of the two-pass regime), checked on the CPU.

The kernel takes, per point and feature, x as fp16 (exact: X is fp16), q =
(16 x)^2 in fp32, q_hi = fp16(q) and q_lo = fp16(q - q_hi); per point and
component r' = 2^10 r, r_hi = fp16(r') and r_lo = fp16(r' - r_hi), all rounded
to nearest even with fp16 subnormals kept (the 32x32x16 f16 MFMA keeps
subnormal inputs). Sx gets r_hi x + r_lo x, Sxx gets r_hi q_hi + r_hi q_lo +
r_lo q_hi, and the partials are scaled back by 2^-10 and 2^-18. The library
states:
- q is exact in fp32 and q_hi never overflows while |x| < 15 (the range the
  device flag admits: every row has |x|^2 < 225);
- q = q_hi + q_lo exactly for |x| >= 2^-6, and within 2^-25 below;
- r' = r_hi + r_lo + d with |d| <= max(2^-22 r', 2^-25);
- every fp16 x fp16 product is exact in fp32;
- per term, Sx is off by <= 2^-22 r|x| + 2^-35 |x| and Sxx by
  <= 2^-21 r x^2 + 2^-35 x^2 + 2^-68, plus 2^-33 r where |x| < 2^-6,
  before the fp32 accumulation.
numpy's float32 -> float16 conversion rounds to nearest even and keeps
subnormals, as the device conversion does. The x side is checked over every
fp16 value below 15, the r side over random fp32 values of every magnitude.
"""
import numpy as np

F16_MAX = 65504.0
F16_MFMA_SAFE = 57600.0  # (16 * 15)^2: q stays at or below this for |x| < 15


def _all_x():
    """Every finite fp16 value with 0 < |x| < 15, both signs."""
    pos = np.arange(1, 0x4B80, dtype=np.uint16).view(np.float16)  # 0x4B80 is 15.0
    assert float(pos[-1]) < 15.0 and float(np.float16(15.0)) == 15.0
    return np.concatenate([pos, -pos])


def _split_q(x16):
    x32 = x16.astype(np.float32)
    q = (np.float32(16) * x32) * (np.float32(16) * x32)
    qh = q.astype(np.float16)
    ql = (q - qh.astype(np.float32)).astype(np.float16)
    return q, qh, ql


def _split_r(r32):
    rs = r32 * np.float32(1024)
    rh = rs.astype(np.float16)
    rl = (rs - rh.astype(np.float32)).astype(np.float16)
    return rs, rh, rl


def _rvals(rng, n):
    r = np.exp2(rng.uniform(-40.0, 0.0, n)).astype(np.float32)
    edge = np.array([0.0, 1.0, 2.0 ** -13, 2.0 ** -24, 2.0 ** -14, 0.5], dtype=np.float32)
    return np.concatenate([edge, r])


def f(v):
    return np.asarray(v).astype(np.float64)


def test_rounding_emulation_keeps_subnormals_and_ties_to_even():
    assert float(np.float32(2.0 ** -24).astype(np.float16)) == 2.0 ** -24  # smallest subnormal
    assert float(np.float32(2.0 ** -25).astype(np.float16)) == 0.0  # tie to even (zero)
    assert float(np.float32(1 + 2.0 ** -11).astype(np.float16)) == 1.0  # tie to even
    assert float(np.float32(1 + 3 * 2.0 ** -11).astype(np.float16)) == 1 + 2.0 ** -9


def test_square_split_over_every_fp16_x_below_15():
    x = _all_x()
    q, qh, ql = _split_q(x)
    q64 = (16.0 * f(x)) ** 2
    assert np.array_equal(f(q), q64)  # 22 significant bits: exact in fp32
    assert np.all(np.isfinite(qh)) and np.all(np.abs(f(qh)) <= F16_MFMA_SAFE)
    e = q64 - f(qh) - f(ql)
    big = np.abs(f(x)) >= 2.0 ** -6
    assert np.all(e[big] == 0.0)
    assert np.all(np.abs(e) <= 2.0 ** -25)
    # the threshold is tight: just below 2^-6 some squares do not split exactly
    assert np.any(e[~big] != 0.0)


def test_responsibility_split_residual():
    rng = np.random.default_rng(7)
    r = _rvals(rng, 1 << 20)
    rs, rh, rl = _split_r(r)
    assert np.array_equal(f(rs), 1024.0 * f(r))
    d = f(rs) - f(rh) - f(rl)
    assert np.all(np.abs(d) <= np.maximum(2.0 ** -22 * f(rs), 2.0 ** -25))
    normal = r >= 2.0 ** -13
    assert np.all(np.abs(d[normal]) <= 2.0 ** -22 * f(rs[normal]))


def test_products_exact_and_per_term_bounds():
    rng = np.random.default_rng(8)
    x = _all_x()
    q, qh, ql = _split_q(x)
    for _ in range(4):  # four random responsibilities per x
        r = _rvals(rng, x.size)[: x.size]
        rng.shuffle(r)
        rs, rh, rl = _split_r(r)
        xh = x
        pairs = ((rh, xh), (rl, xh), (rh, qh), (rh, ql), (rl, qh))
        for a, b in pairs:
            p = f(a) * f(b)
            assert np.array_equal(f(p.astype(np.float32)), p)  # 11 x 11 bits
        sx = 2.0 ** -10 * (f(rh) * f(xh) + f(rl) * f(xh))
        sxx = 2.0 ** -18 * (f(rh) * f(qh) + f(rh) * f(ql) + f(rl) * f(qh))
        ax, x2 = np.abs(f(x)), f(x) ** 2
        rx, rxx = f(r) * f(x), f(r) * x2  # exact in fp64 (35 and 46 bits)
        assert np.all(np.abs(sx - rx) <= 2.0 ** -22 * f(r) * ax + 2.0 ** -35 * ax)
        tiny = ax < 2.0 ** -6
        # the last term is the product of the two absolute residuals (2^-25
        # each, scaled back by 2^-18), met where both r' and q are subnormal
        bound = 2.0 ** -21 * rxx + 2.0 ** -35 * x2 + np.where(tiny, 2.0 ** -33 * f(r), 0.0) + 2.0 ** -68
        assert np.all(np.abs(sxx - rxx) <= bound)


def test_row_norm_rule_keeps_every_square_in_range():
    assert F16_MFMA_SAFE < F16_MAX
    # A fp32 sum of non-negative squares is monotone in each term under round
    # to nearest, so a row whose recorded |x|^2 is below 225 has every x_j^2
    # below 225, i.e. |x_j| < 15 and q = (16 x_j)^2 <= 57600 < F16_MAX.
    rng = np.random.default_rng(9)
    for _ in range(2000):
        d = int(rng.integers(1, 129))
        xr = (rng.standard_normal(d) * rng.uniform(0.1, 8.0)).astype(np.float16)
        sq = np.float32(0)
        for v in xr.astype(np.float32):
            sq = np.float32(sq + v * v)
        if sq < 225:
            assert np.all(np.abs(f(xr)) < 15.0)
            assert np.all(np.abs(f(_split_q(xr)[1])) <= F16_MFMA_SAFE)
