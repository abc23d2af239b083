"""The sweep kernel decides q = rint(w / s) (fp32 quotient, correctly rounded)
as rint(w * (1/s)) unless w * (1/s) lies within |y| 2^-21 of a half-integer,
where it divides.  This checks the claim behind it on the CPU with IEEE fp32
arithmetic (NumPy): whenever the fast test passes, the two integers agree.
The check emulates the kernel's instruction sequence: y = fl(w * r) with
r = fl(1 / s); t = fl(w * r - rint(y)) (one fused rounding); the distance
0.5 - |t| against fl(|y| 2^-21 + 2^-126) (one fused rounding).
"""
import numpy as np

f32 = np.float32


def fast_decision(w, s):
    r = (f32(1.0) / s).astype(f32)
    y = (w * r).astype(f32)
    qr = np.rint(y)
    t = (w.astype(np.float64) * r.astype(np.float64) - qr.astype(np.float64)).astype(f32)
    dist = (f32(0.5) - np.abs(t)).astype(f32)
    delta = (np.abs(y).astype(np.float64) * 2.0 ** -21 + 2.0 ** -126).astype(f32)
    ok = dist >= delta
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
