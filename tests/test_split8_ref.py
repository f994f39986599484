"""CPU pins of the test-side split8 definitions (tests/split8_ref.py), checked
against exact rational arithmetic, so that the GPU tests that use them
compare the library with the documented fixed-point Gram matrix and not with
a restatement of their own mistakes."""
from fractions import Fraction

import numpy as np

from tests import split8_ref as R8


def _inputs(seed, n=40, d=5):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((n, d)) * np.exp(3.0 * rng.standard_normal(d))[None, :]
    X[:, 2] = 0.0
    X[7, 3] = 2.0 ** 5  # the column maximum is a power of two
    X[:, 3] = np.clip(X[:, 3], -2.0 ** 5, 2.0 ** 5)
    return X.astype(np.float32)


def _exact_fixed_point(X):
    """X~ as Fractions, from the definition: 2^e the smallest power of two
    above the column maximum, x rounded to a multiple of 2^(e - 30), ties to
    even."""
    n, d = X.shape
    out = [[None] * d for _ in range(n)]
    for f in range(d):
        col = [Fraction(float(v)) for v in X[:, f]]
        mx = max(abs(v) for v in col)
        e = 0
        if mx > 0:
            while Fraction(2) ** e <= mx:
                e += 1
            while Fraction(2) ** (e - 1) > mx:
                e -= 1
        step = Fraction(2) ** (e - 30)
        for k, v in enumerate(col):
            q = v / step
            fl = q.numerator // q.denominator
            r = q - fl
            m = fl + (1 if (r > Fraction(1, 2) or (r == Fraction(1, 2) and fl % 2)) else 0)
            assert abs(m) < 2 ** 30
            out[k][f] = m * step
    return out


def test_fixed_point_gram_is_the_exact_sum():
    X = _inputs(1)
    Xt = _exact_fixed_point(X)
    n, d = X.shape
    S, mag = R8.fixed_point_gram(X)
    for f in range(d):
        for g in range(d):
            ex = sum(Xt[k][f] * Xt[k][g] for k in range(n))
            assert abs(Fraction(float(S[f, g])) - ex) <= Fraction(2.0 ** -51) * Fraction(mag[f, g])
    dg = R8.fixed_point_diag(X)
    assert np.array_equal(dg, np.diag(S))
    m, e = R8.fixed_point_ints(X)
    assert e[2] == 0 and np.all(m[:, 2] == 0)
    assert e[3] == 6  # max 2^5 -> scale 2^6


def test_rounding_bound_holds_exactly():
    for seed in (2, 3):
        X = _inputs(seed)
        Xt = _exact_fixed_point(X)
        n, d = X.shape
        B = R8.rounding_bound(X)
        for f in range(d):
            for g in range(d):
                fixed = sum(Xt[k][f] * Xt[k][g] for k in range(n))
                exact = sum(Fraction(float(X[k, f])) * Fraction(float(X[k, g])) for k in range(n))
                assert abs(fixed - exact) <= Fraction(float(B[f, g]))


def test_subset_with_given_exponents_matches_full():
    X = _inputs(4, n=64, d=9)
    S, _ = R8.fixed_point_gram(X)
    cols = np.array([8, 0, 3])
    e = R8.col_exponent(X)[cols]
    Ss, _ = R8.fixed_point_gram(X[:, cols], e=e)
    assert np.array_equal(Ss, S[np.ix_(cols, cols)])


def _balanced_digits(m):
    """The digits of an integer m, |m| < 2^30, as plain Python integers:
    repeated division by 256 with remainders in [-128, 127]."""
    out = []
    for _ in range(3):
        r = (m + 128) % 256 - 128
        out.append(r)
        m = (m - r) // 256
    return [m] + out[::-1]


def test_digits_reconstruct_and_match_balanced_division():
    rng = np.random.default_rng(7)
    m = np.concatenate([rng.integers(-(2 ** 30) + 1, 2 ** 30, 2000),
                        [0, 1, -1, 127, 128, -128, -129, 2 ** 30 - 1, -(2 ** 30) + 1,
                         2 ** 29, -(2 ** 29), 0x7F7F7F, -0x808080]])
    d = R8.digits(m)
    rec = (d[0] << 24) + (d[1] << 16) + (d[2] << 8) + d[3]
    assert np.array_equal(rec, m)
    for a in (1, 2, 3):
        assert d[a].min() >= -128 and d[a].max() <= 127
    assert np.abs(d[0]).max() <= 64
    for k in range(len(m)):
        assert [int(x[k]) for x in d] == _balanced_digits(int(m[k]))


def test_split8_gram_is_the_exact_truncated_digit_sum():
    """Per entry, from the definition: sum over tokens and digit pairs with
    a + b <= 4 of d_a d_b 2^(48 - 8(a + b)), times 2^(e_f + e_g - 60), in
    exact rational arithmetic from balanced-division digits; and the left-out
    orders close the gap to the exact X~^T X~ and stay inside their bound."""
    for seed in (5, 6):
        X = _inputs(seed)
        m, e = R8.fixed_point_ints(X)
        n, d = X.shape
        dig = [[_balanced_digits(int(m[k, f])) for f in range(d)] for k in range(n)]
        S, mag = R8.split8_gram(X)
        Sfull, _ = R8.fixed_point_gram(X)
        Xt = _exact_fixed_point(X)
        B = R8.split8_bound(X)
        for f in range(d):
            for g in range(d):
                tr = 0
                for k in range(n):
                    for a in range(4):
                        for b in range(4):
                            if a + b <= 4:
                                tr += dig[k][f][a] * dig[k][g][b] * 2 ** (48 - 8 * (a + b))
                ex = Fraction(tr) * Fraction(2) ** int(e[f] + e[g] - 60)
                tol = Fraction(2.0 ** -51) * Fraction(mag[f, g])
                assert abs(Fraction(float(S[f, g])) - ex) <= tol, (f, g)
                full = sum(Xt[k][f] * Xt[k][g] for k in range(n))
                assert abs(Fraction(float(Sfull[f, g])) - full) <= tol
                exact = sum(Fraction(float(X[k, f])) * Fraction(float(X[k, g])) for k in range(n))
                assert abs(ex - exact) <= Fraction(float(B[f, g]))
        assert np.array_equal(R8.split8_diag(X), np.diag(S))
        assert not np.array_equal(S, Sfull)  # the left-out orders are not all zero
