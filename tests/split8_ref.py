"""Test-side definitions for the digit-sliced int8 Hessian (split8).

The library documents what split8 computes: per call (token chunk), column f
of X gets the scale 2^e_f, the smallest power of two above max_k |x_kf|, and
each value is rounded to the nearest multiple of 2^(e_f - 30) (ties to even);
the integer m = x~ 2^(30 - e_f) is written as d0 2^24 + d1 2^16 + d2 2^8 + d3
with d1..d3 signed bytes, and S += the digit-pair products of orders
a + b <= 4, that is X~^T X~ less 2^(e_f + e_g - 60) (2^8 (D2^T D3 + D3^T D2)
+ D3^T D3). These helpers restate that definition on the host, independently
of the HIP code, and sum it exactly: with m = hi 2^15 + lo (|hi| < 2^15,
0 <= lo < 2^15), every product of halves is an integer below 2^30 and every
sum over fewer than 2^22 tokens an integer below 2^52, so fp64 matrix
products of the halves (and of the digits) are exact; only the final
combination rounds (twice, relative 2^-53 each).
"""
from __future__ import annotations

import numpy as np


def col_exponent(X):
    """e_f with max_k |x_kf| = m 2^e_f, m in [0.5, 1) (0 for a zero column)."""
    X = np.asarray(X)
    mx = np.abs(X).max(axis=0).astype(np.float64)  # exact in X's own type
    return np.frexp(mx)[1].astype(np.int64)


def fixed_point_ints(X, e=None):
    """(m, e): X~ = m 2^(e - 30), m integer (int64), |m| < 2^30. ``e`` may be
    given (the exponents of the full call when X holds some of its columns)."""
    e = col_exponent(X) if e is None else np.asarray(e, dtype=np.int64)
    m = np.rint(np.ldexp(np.asarray(X, dtype=np.float64), (30 - e)[None, :])).astype(np.int64)
    assert np.abs(m).max(initial=0) < 2 ** 30
    return m, e


def _halves(m):
    hi = m >> 15
    lo = m - (hi << 15)
    return hi.astype(np.float64), lo.astype(np.float64)


def digits(m):
    """[d0, d1, d2, d3] with m = d0 2^24 + d1 2^16 + d2 2^8 + d3, d1..d3 in
    [-128, 127] (int64 arrays of m's shape)."""
    m = np.asarray(m, dtype=np.int64)
    d = [None] * 4
    for a in (3, 2, 1):
        low = m & 0xFF
        d[a] = low - ((low >= 128).astype(np.int64) << 8)
        m = (m - d[a]) >> 8
    d[0] = m
    return d


def dropped_orders(m_a, m_b):
    """(2^8 (D2^T D3 + D3^T D2) + D3^T D3, its bound with |d| in place of d):
    the digit orders 5 and 6 that split8 leaves out, in units of
    2^(e_f + e_g - 60); exact integers (fewer than 2^22 tokens)."""
    da, db = digits(m_a), digits(m_b)
    f = [x.astype(np.float64) for x in da]
    g = [x.astype(np.float64) for x in db]
    v = 256.0 * (f[2].T @ g[3] + f[3].T @ g[2]) + f[3].T @ g[3]
    af, ag = [np.abs(x) for x in f], [np.abs(x) for x in g]
    b = 256.0 * (af[2].T @ ag[3] + af[3].T @ ag[2]) + af[3].T @ ag[3]
    return v, b


def split8_gram(X, cols_a=None, cols_b=None, e=None):
    """(what split8 adds for one call, restricted to cols_a x cols_b, and
    |X~|^T |X~| on the same block): X~^T X~ without the digit orders 5 and 6.
    Exact integer sums, one combination; requires fewer than 2^22 tokens."""
    X = np.asarray(X)
    assert X.shape[0] < 2 ** 22
    m, e = fixed_point_ints(X, e)
    ca = np.arange(X.shape[1]) if cols_a is None else np.asarray(cols_a)
    cb = ca if cols_b is None else np.asarray(cols_b)
    ha, la = _halves(m[:, ca])
    hb, lb = _halves(m[:, cb])
    drop, _ = dropped_orders(m[:, ca], m[:, cb])
    T = (ha.T @ hb) * 2.0 ** 30 + ((ha.T @ lb) + (la.T @ hb)) * 2.0 ** 15 + (la.T @ lb - drop)
    scale = np.ldexp(1.0, e[ca][:, None] + e[cb][None, :] - 60)
    am = np.abs(m).astype(np.float64)
    mag = (am[:, ca].T @ am[:, cb]) * scale
    return T * scale, mag


def split8_diag(X, e=None, block=1024):
    """diag of split8_gram for one call's X (column blocks, to bound the
    temporaries)."""
    X = np.asarray(X)
    e = col_exponent(X) if e is None else np.asarray(e, dtype=np.int64)
    out = np.empty(X.shape[1])
    for c0 in range(0, X.shape[1], block):
        m, eb = fixed_point_ints(X[:, c0:c0 + block], e[c0:c0 + block])
        hi, lo = _halves(m)
        d = digits(m)
        d2, d3 = d[2].astype(np.float64), d[3].astype(np.float64)
        drop = 512.0 * (d2 * d3).sum(axis=0) + (d3 * d3).sum(axis=0)
        t = (hi * hi).sum(axis=0) * 2.0 ** 30 + 2.0 * (hi * lo).sum(axis=0) * 2.0 ** 15 \
            + ((lo * lo).sum(axis=0) - drop)
        out[c0:c0 + block] = t * np.ldexp(1.0, 2 * eb - 60)
    return out


def split8_bound(X, cols_a=None, cols_b=None, e=None):
    """Bound on |split8 - X^T X| for one call: the rounding of X
    (rounding_bound) plus the digit orders left out."""
    X = np.asarray(X)
    m, e = fixed_point_ints(X, e)
    ca = np.arange(X.shape[1]) if cols_a is None else np.asarray(cols_a)
    cb = ca if cols_b is None else np.asarray(cols_b)
    _, b = dropped_orders(m[:, ca], m[:, cb])
    scale = np.ldexp(1.0, e[ca][:, None] + e[cb][None, :] - 60)
    return rounding_bound(X, ca, cb, e) + b * scale


def fixed_point_gram(X, cols_a=None, cols_b=None, e=None):
    """(X~^T X~ restricted to cols_a x cols_b, |X~|^T |X~| on the same block)
    for one call's X. Exact integer sums; requires fewer than 2^23 tokens."""
    X = np.asarray(X)
    assert X.shape[0] < 2 ** 23
    m, e = fixed_point_ints(X, e)
    ca = np.arange(X.shape[1]) if cols_a is None else np.asarray(cols_a)
    cb = ca if cols_b is None else np.asarray(cols_b)
    ha, la = _halves(m[:, ca])
    hb, lb = _halves(m[:, cb])
    T = (ha.T @ hb) * 2.0 ** 30 + ((ha.T @ lb) + (la.T @ hb)) * 2.0 ** 15 + la.T @ lb
    scale = np.ldexp(1.0, e[ca][:, None] + e[cb][None, :] - 60)
    am = np.abs(m).astype(np.float64)
    mag = (am[:, ca].T @ am[:, cb]) * scale
    return T * scale, mag


def fixed_point_diag(X, e=None, block=1024):
    """diag(X~^T X~) for one call's X, exact integer sums then one rounding
    (column blocks, to bound the temporaries)."""
    X = np.asarray(X)
    e = col_exponent(X) if e is None else np.asarray(e, dtype=np.int64)
    out = np.empty(X.shape[1])
    for c0 in range(0, X.shape[1], block):
        m, eb = fixed_point_ints(X[:, c0:c0 + block], e[c0:c0 + block])
        hi, lo = _halves(m)
        d = (hi * hi).sum(axis=0) * 2.0 ** 30 + 2.0 * (hi * lo).sum(axis=0) * 2.0 ** 15 \
            + (lo * lo).sum(axis=0)
        out[c0:c0 + block] = d * np.ldexp(1.0, 2 * eb - 60)
    return out


def rounding_bound(X, cols_a=None, cols_b=None, e=None):
    """Bound on |X~^T X~ - X^T X| for one call: |x~ - x| <= 2^(e_f - 31), so
    2^-31 (s_f sum|x_g| + s_g sum|x_f|) + n 2^-62 s_f s_g."""
    X = np.asarray(X, dtype=np.float64)
    ca = np.arange(X.shape[1]) if cols_a is None else np.asarray(cols_a)
    cb = ca if cols_b is None else np.asarray(cols_b)
    s = np.ldexp(1.0, col_exponent(X) if e is None else np.asarray(e, dtype=np.int64))
    a = np.abs(X).sum(axis=0)
    n = X.shape[0]
    return 2.0 ** -31 * (s[ca][:, None] * a[cb][None, :] + s[cb][None, :] * a[ca][:, None]) \
        + n * 2.0 ** -62 * np.outer(s[ca], s[cb])
