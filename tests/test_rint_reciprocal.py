"""The sweep kernel decides q = rint(w / s) (fp32 quotient, correctly rounded)
as rint(w * (1/s)) unless w * (1/s) lies near a half-integer (or 1/s is zero
or not finite); such a step is swept again with true divisions.  This checks
the claim behind it on the CPU with IEEE fp32 arithmetic (NumPy): whenever
the fast test passes, the two integers agree.  The check emulates the
kernel's instruction sequence: y = fl(w * r) with r = fl(1 / s);
t = fl(w * r - rint(y)) (one fused rounding); m = fl(|y| 2^-20 + |t|) (one
fused rounding); the fast path stands when m < 1/2.
"""
import numpy as np

f32 = np.float32


def fast_decision(w, s):
    r = (f32(1.0) / s).astype(f32)
    y = (w * r).astype(f32)
    qr = np.rint(y)
    t = (w.astype(np.float64) * r.astype(np.float64) - qr.astype(np.float64)).astype(f32)
    m = (np.abs(y).astype(np.float64) * 2.0 ** -20 + np.abs(t).astype(np.float64)).astype(f32)
    ok = (m < f32(0.5)) & np.isfinite(r) & (r != 0)
    return qr, ok


def exact_decision(w, s):
    return np.rint((w / s).astype(f32))


def test_reciprocal_rint_agrees_when_not_near_half():
    rng = np.random.default_rng(0)
    n = 2_000_000
    s = (rng.uniform(1e-4, 1.0, n) * 10.0 ** rng.integers(-3, 2, n)).astype(f32)
    w = (rng.normal(0.0, 1.0, n) * s * rng.uniform(0, 20, n)).astype(f32)
    qr, ok = fast_decision(w, s)
    ex = exact_decision(w, s)
    assert np.array_equal(qr[ok], ex[ok])
    assert ok.mean() > 0.999  # the divide path is rare


def test_ties_and_neighbours_take_the_division():
    # w = (k + 1/2) s rounded, and its fp32 neighbours: quotients at or next
    # to a rounding boundary
    rng = np.random.default_rng(1)
    s = rng.uniform(1e-3, 1.0, 20000).astype(f32)
    k = rng.integers(-300, 300, 20000).astype(f32)
    base = ((k + f32(0.5)) * s).astype(f32)
    for steps in range(-3, 4):
        w = base
        for _ in range(abs(steps)):
            w = np.nextafter(w, np.inf if steps > 0 else -np.inf).astype(f32)
        qr, ok = fast_decision(w, s)
        ex = exact_decision(w, s)
        assert np.array_equal(qr[ok], ex[ok]), steps
        # exact ties in the quotient never pass the fast test
        tie = (w / s).astype(f32) == (k + f32(0.5))
        assert not np.any(ok & tie)


def test_degenerate_scales_take_the_division():
    # 1/s zero or not finite (s = 0, a subnormal s whose reciprocal
    # overflows, s = inf): the fast path never stands
    s = np.array([0.0, 1e-40, np.inf, 2.0 ** -127], dtype=f32)
    w = np.array([0.3, 1e-41, 5.0, 2.0 ** -128], dtype=f32)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        _, ok = fast_decision(w, s)
    assert not np.any(ok[:3])
