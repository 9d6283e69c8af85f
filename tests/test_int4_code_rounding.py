"""The int4 encoder's fast code rounding, checked on the host in binary32.

The encoder computes code = rint(x / scale) (binary32 division) as
rint(RN(x * RN(1 / scale))) and falls back to the division when that product
lies within 2^-18 of a half-integer (|t - rint(t)| >= 1/2 - 2^-18).  This
replays exactly that arithmetic in
numpy float32 on values packed around every code boundary, at scales from
2^-100 to 2^100, and requires it to equal division-then-rint everywhere; the
same values without the fallback must show mismatches (so the fallback is
what makes it exact).  Host only: no GPU."""

import numpy as np

F32 = np.float32


def _values(rng, scale, amax, n=4000):
    k = rng.integers(-7, 7, n)
    base = ((k + 0.5) * np.float64(scale)).astype(F32)
    near = (base.view(np.int32) + rng.integers(-40, 41, n).astype(np.int32)).view(F32)
    rand = (rng.uniform(-1, 1, n) * amax).astype(F32)
    x = np.concatenate([near, rand, [amax, -amax, F32(0)]]).astype(F32)
    return x[np.abs(x) <= amax]


def test_fast_rounding_equals_division():
    rng = np.random.default_rng(0)
    unguarded_mismatches = 0
    for _ in range(120):
        amax = F32(rng.uniform(0.5, 1.0) * 2.0 ** int(rng.integers(-100, 100)))
        scale = F32(amax / F32(7))
        r = F32(F32(1) / scale)
        x = _values(rng, scale, amax)
        want = np.rint(x / scale)
        t = (x * r).astype(F32)
        q = np.rint(t)
        near = np.abs(t - q) >= F32(0.5) - F32(2.0 ** -18)  # the kernel's form of the test
        assert np.array_equal(np.where(near, want, q), want)
        unguarded_mismatches += int(np.sum(q != want))
    assert unguarded_mismatches > 0
