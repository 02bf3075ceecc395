"""Numerical rules the kernels rely on, checked on the host in binary64
(no GPU): the TriAttention z reciprocal rule."""
import numpy as np


def test_tri_z_reciprocal_rule_agrees_with_the_division():
    # The TriAttention reduce forms z = (float)((s - mu) / sigma) as
    # q = (s - mu) * RN(1 / sigma) and keeps (float)q unless q lies within
    # 3 binary64 ulps of a binary32 rounding midpoint, or below binary32's
    # normal range.  Check that rule against the correctly rounded division
    # where it matters most: quotients placed a few ulps from midpoints.
    rs = np.random.default_rng(71)
    n = 200000
    sigma = np.exp(rs.uniform(-8, 8, n))
    f = (rs.standard_normal(n) * np.exp2(rs.integers(-30, 20, n))).astype(np.float32)
    nxt = np.nextafter(f, np.float32(np.inf), dtype=np.float32)
    mid = (f.astype(np.float64) + nxt.astype(np.float64)) / 2          # exact midpoints
    d = mid * sigma
    d = d + np.ldexp(rs.integers(-8, 9, n).astype(np.float64), np.frexp(d)[1] - 53)
    d = np.concatenate([d, rs.standard_normal(n) * np.exp2(rs.integers(-30, 20, n)),
                        np.ldexp(rs.uniform(1, 2, 1000), rs.integers(-160, -127, 1000))])   # below 2^-126
    sigma = np.concatenate([sigma, sigma, np.ones(1000)])
    q = d * (1.0 / sigma)
    b = q.view(np.uint64)
    low = (b & np.uint64(0x1FFFFFFF)).astype(np.int64)
    ex = ((b >> np.uint64(52)) & np.uint64(0x7FF)).astype(np.int64)
    safe = (np.abs(low - (1 << 28)) > 3) & (ex >= 1023 - 126)
    exact = (d / sigma).astype(np.float32)
    fast = q.astype(np.float32)
    assert np.array_equal(fast[safe].view(np.uint32), exact[safe].view(np.uint32))
    # the rule sends the near-midpoint and tiny quotients to the division
    assert (~safe[:n]).sum() > n // 10
    assert not safe[-1000:].any()
