"""The quantizer kernels take rne(w / s) in the clip search from
t = w * fl(1 / s) and fall back to the division only when t lies within
2^-20 |t| of a half-integer.  This checks that rule in IEEE binary32 (numpy)
on quotients placed a few ulps from half-integers and on ordinary ones: where
the rule does not flag a value, rint(t) equals rint(fl(w / s)) exactly."""
import numpy as np


def _fast(w, s):
    f32 = np.float32
    inv = (f32(1) / s).astype(np.float32)
    tq = (w * inv).astype(np.float32)
    t = np.rint(tq)
    with np.errstate(invalid="ignore"):
        near = ~(np.abs(np.abs((tq - t).astype(np.float32)) - f32(0.5)) > np.abs(tq) * f32(2.0 ** -20))
    return t, near


def test_fast_quotient_rounding_rule():
    rng = np.random.default_rng(5)
    n = 1_000_000
    # fp16 scales, as the search uses
    s = (2.0 ** rng.uniform(-14, 4, n)).astype(np.float16).astype(np.float32)
    # quotients within a few ulps of half-integers ...
    q = rng.integers(-40, 40, n).astype(np.float32)
    w_near = ((q + np.float32(0.5)) * s).astype(np.float32)
    steps = rng.integers(-3, 4, n)
    for k in range(1, 4):
        w_near = np.where(steps >= k, np.nextafter(w_near, np.float32(np.inf)), w_near)
        w_near = np.where(steps <= -k, np.nextafter(w_near, np.float32(-np.inf)), w_near)
    # ... and ordinary ones, with NaN and zero weights
    w_any = (rng.standard_normal(n) * rng.uniform(0.001, 50, n) * s).astype(np.float32)
    w_any[:7] = [np.nan, 0.0, -0.0, 1e-30, -1e-30, 65504.0, -65504.0]
    for w in (w_near.astype(np.float32), w_any):
        with np.errstate(invalid="ignore"):
            exact = np.rint((w / s).astype(np.float32))
        t, near = _fast(w, s)
        ok = near | (t == exact)
        assert ok.all(), f"{(~ok).sum()} values round differently without a flag"
    # the flag is rare on ordinary quotients (it only costs time)
    _, near = _fast(w_any, s)
    assert near.mean() < 1e-3
