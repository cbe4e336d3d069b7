"""The error bound of the split-bf16 statistics contraction, checked on the CPU.

An fp32 value v is split as v = hi + lo + d with hi = bf16(v) and
lo = bf16(v - hi), both rounded to nearest even; a product a*b is then taken as
hi_a*hi_b + hi_a*lo_b + lo_a*hi_b. The library states |d| <= 2^-16 |v| and a
per-product error <= 3.0001 * 2^-16 |a b|. Both are checked here exhaustively over
random fp32 values of every magnitude the statistics meet, with bf16 rounding
emulated bit by bit (IEEE round to nearest even on the top 16 bits).

With 8 significant bits, |v - hi| <= 2^-8 |v|, so |lo| <= 2^-8 |v| and
|d| <= 2^-8 |v - hi| <= 2^-16 |v|; the dropped terms of a product are
lo_a lo_b and the d terms, together <= (3 + 2^-14) 2^-16 |a b|.
"""
import numpy as np


def bf16_rne(v: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even), returned as float32."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def split(v):
    hi = bf16_rne(v)
    lo = bf16_rne((v - hi).astype(np.float32))  # v - hi is exact in fp32
    return hi, lo


def _values(rng, n):
    mant = rng.uniform(1.0, 2.0, n)
    expo = rng.integers(-40, 40, n)
    sign = rng.choice([-1.0, 1.0], n)
    return (sign * mant * np.exp2(expo)).astype(np.float32)


def test_rounding_emulation_matches_known_values():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa wins (1.0);
    # 1 + 3*2^-8 ties between 1 + 2^-7 and 1 + 2^-6: rounds to 1 + 2^-6.
    v = np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -9, -3.0], dtype=np.float32)
    assert bf16_rne(v).tolist() == [1.0, 1.0, 1 + 2.0 ** -6, 1.0, -3.0]


def test_split_residual_bound():
    rng = np.random.default_rng(5)
    v = _values(rng, 1 << 20)
    hi, lo = split(v)
    d = v.astype(np.float64) - hi.astype(np.float64) - lo.astype(np.float64)
    assert np.all(np.abs(lo.astype(np.float64)) <= 2.0 ** -8 * np.abs(v.astype(np.float64)))
    assert np.all(np.abs(d) <= 2.0 ** -16 * np.abs(v.astype(np.float64)))


def test_split_product_bound():
    rng = np.random.default_rng(6)
    a = _values(rng, 1 << 20)
    b = _values(rng, 1 << 20)
    ah, al = split(a)
    bh, bl = split(b)
    f = lambda x: x.astype(np.float64)  # noqa: E731
    approx = f(ah) * f(bh) + f(ah) * f(bl) + f(al) * f(bh)
    exact = f(a) * f(b)
    assert np.all(np.abs(approx - exact) <= 3.0001 * 2.0 ** -16 * np.abs(exact))
    # and each of the three bf16 x bf16 products is exact in fp32 (8 + 8 bits)
    for x, y in ((ah, bh), (ah, bl), (al, bh)):
        p64 = f(x) * f(y)
        assert np.array_equal(p64.astype(np.float32).astype(np.float64), p64)
