"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these re-types the oracle's formula: each checks it against a closed
form, a brute force, an independent formulation (exact rationals, the
Schur-complement form of the update, the optimality of the remaining weights)
or an invariant that a plausible mistake (dropped factor 2, wrong sign,
transposed operand, off-by-one group boundary, wrong rounding) would break.
"""
from fractions import Fraction
import itertools
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads


# ----------------------------------------------------------------- Hessian --
def test_hessian_brute_force_integer_exact():
    rng = np.random.default_rng(0)
    X = rng.integers(-8, 9, size=(64, 16)).astype(np.float16)
    H = O.hessian([X[:40], X[40:]])
    Hb = np.zeros((16, 16))
    for i in range(16):
        for j in range(16):
            acc = 0
            for t in range(64):
                acc += int(X[t, i]) * int(X[t, j])
            Hb[i, j] = 2 * acc
    assert np.array_equal(H, Hb)


def test_hessian_symmetric_psd():
    X = workloads.x_tokens(workloads.get("c0"), 0, 1).numpy()
    H = O.hessian(X)
    assert np.array_equal(H, H.T)
    ev = np.linalg.eigvalsh(H)
    assert ev.min() >= -1e-12 * np.abs(H).max()


def test_hessian_is_second_difference_of_layer_loss():
    """L(V) = ||X (V - W0)^T||_F^2 is quadratic; its second difference along E
    is t^2 * sum_r e_r^T H e_r exactly (this fixes the factor 2 and the operand order)."""
    rng = np.random.default_rng(1)
    X = rng.standard_normal((50, 12))
    W0 = rng.standard_normal((3, 12))
    E = rng.standard_normal((3, 12))
    t = 0.125

    def L(V):
        return float(np.sum((X @ (V - W0).T) ** 2))

    lhs = L(W0 + t * E) - 2 * L(W0) + L(W0 - t * E)
    H = O.hessian(X)
    rhs = t * t * float(np.sum((E @ H) * E))
    assert math.isclose(lhs, rhs, rel_tol=1e-12)


# ---------------------------------------------------------- damp / order --
def test_condition_closed_form_with_dead_feature():
    H = np.diag([4.0, 0.0, 2.0]) + np.array([[0, 0, 1], [0, 0, 0], [1, 0, 0]], float)
    Hd, mu = O.condition(H, 0.01)
    assert mu == pytest.approx((4 + 1 + 2) / 3)  # dead feature counted as 1
    assert np.allclose(np.diag(Hd), [4 + 0.07 / 3, 1 + 0.07 / 3, 2 + 0.07 / 3])
    assert Hd[0, 2] == 1.0 and Hd[2, 0] == 1.0 and Hd[0, 1] == 0.0


def test_column_order_desc_stable():
    H = np.diag([3.0, 5.0, 3.0, 7.0, 5.0, 0.0])
    assert list(O.column_order(H, True)) == [3, 1, 4, 0, 2, 5]
    assert list(O.column_order(H, False)) == [0, 1, 2, 3, 4, 5]
    assert list(O.column_order(np.eye(5), True)) == [0, 1, 2, 3, 4]


# ------------------------------------------------------------------ factor --
T1_H = np.array([[2.0, 1, 0], [1, 2, 1], [0, 1, 2]])
T1_W = np.array([[0.4, 1.4, 3.0]])


def test_factor_t1_closed_form():
    U = O.hinv_chol(T1_H, np.arange(3))
    r3 = math.sqrt(3.0)
    want = np.array([[r3 / 2, -1 / r3, 1 / (2 * r3)],
                     [0, math.sqrt(2 / 3), -1 / math.sqrt(6)],
                     [0, 0, 1 / math.sqrt(2)]])
    assert np.allclose(U, want, atol=1e-14, rtol=0)


def test_factor_two_routes_and_residual():
    X = workloads.x_tokens(workloads.get("c0"), 0, 1).numpy()
    H = O.hessian(X)
    Hd, _ = O.condition(H, 0.01)
    perm = O.column_order(H, True)
    U = O.hinv_chol(Hd, perm)
    U2 = O.hinv_chol_reverse(Hd, perm)
    assert np.allclose(np.tril(U, -1), 0)
    assert np.all(np.diag(U) > 0)
    assert np.abs(U - U2).max() <= 1e-10 * np.abs(U).max()
    Hp = Hd[np.ix_(perm, perm)]
    assert np.abs(U.T @ U @ Hp - np.eye(128)).max() < 1e-9


def test_factor_not_pd_raises():
    with pytest.raises(O.NotPositiveDefinite):
        O.hinv_chol(-np.eye(4), np.arange(4))
    with pytest.raises(O.NotPositiveDefinite):
        O.hinv_chol(np.zeros((3, 3)), np.arange(3))


# ---------------------------------------------------- sweep: toy traces --
def test_t1_trace():
    """1x3 layer, 2-bit asym, one group, damp 0.

    Hand derivation (exact rationals): range of the original row [0, 3]
    (zero included) -> s = 1, z = 0.  U' = U / diag(U) = [[1, -2/3, 1/3],
    [0, 1, -1/2], [0, 0, 1]].  Step 0: 0.4 -> q 0, e = 2/5, w1 = 5/3,
    w2 = 43/15.  Step 1: 5/3 -> q 2, e = -1/3, w2 = 27/10.  Step 2: q 3.
    """
    res = O.gptq(T1_W, T1_H, bits=2, group_size=-1, sym=False, damp_percent=0.0,
                 desc_act=False)
    assert res.codes.tolist() == [[0, 2, 3]]
    assert res.scales.tolist() == [[1.0]] and res.zeros.tolist() == [[0]]
    rt = O.rtn(T1_W, 2, -1, False)
    assert rt.codes.tolist() == [[0, 1, 3]]
    d_g = T1_W - res.what
    d_r = T1_W - rt.what
    assert float(np.sum((d_g @ T1_H) * d_g)) == pytest.approx(14 / 25, abs=1e-12)
    assert float(np.sum((d_r @ T1_H) * d_r)) == pytest.approx(24 / 25, abs=1e-12)


def test_t1_brute_force_optimum():
    """GPTQ is greedy: for T1 it reaches the best of all 64 code triples on the
    grid s = 1, z = 0 (the optimum value 14/25 is attained by [0,2,3] and [1,1,3])."""
    best = min(
        (float(((T1_W[0] - np.array(c)) @ T1_H @ (T1_W[0] - np.array(c)))), c)
        for c in itertools.product(range(4), repeat=3))
    assert best[0] == pytest.approx(14 / 25)
    res = O.gptq(T1_W, T1_H, 2, -1, False, 0.0, False)
    d = T1_W[0] - res.what[0]
    assert float(d @ T1_H @ d) == pytest.approx(best[0])


T2_H = np.array([[2.0, 1, 0, 0], [1, 5, 2, 0], [0, 2, 3, 1], [0, 0, 1, 4]])
T2_W = np.array([[1.0, 1.0, -0.2, -0.6], [-0.2, 0.8, 1.0, -0.2]])


def test_t2_trace_desc_act_groups():
    """2x4 layer, 2-bit asym, group_size 2, desc_act, damp 0.

    diag = [2,5,3,4] -> perm [1,3,2,0]; groups in quantization order are
    {1,3} and {2,0} -> g_idx [1,0,1,0].  Row 0: group {1,3} from [1, -3/5]:
    s = 8/15, z = 1; col 1: 23/8 -> 3; col 3: -9/88 -> 0.  Group {2,0} from
    [-4/15, 29/30]: s = 37/90, z = 1; col 2: 13/37 -> 0; col 0: 124/37 -> 3.
    Row 1: s = 1/3, z = 1; col 1: 17/5 -> 3; col 3: 18/55 -> 0.  Next group
    from [17/15, -2/15]: s = 19/45, z = 0; col 2: 51/19 -> 3; col 0: -6/19 -> 0.
    """
    res = O.gptq(T2_W, T2_H, 2, 2, False, 0.0, True)
    assert res.perm.tolist() == [1, 3, 2, 0]
    assert res.g_idx.tolist() == [1, 0, 1, 0]
    assert res.codes.tolist() == [[3, 3, 0, 0], [0, 3, 3, 0]]
    assert res.zeros.tolist() == [[1, 1], [1, 0]]
    assert np.allclose(res.scales, np.array([[8 / 15, 1 / 3], [37 / 90, 19 / 45]]),
                       rtol=1e-14, atol=0)
    # quality: sum_r d^T H d = 511/1620 for GPTQ
    d = T2_W - res.what
    assert float(np.sum((d @ T2_H) * d)) == pytest.approx(511 / 1620, rel=1e-12)
    # RTN, natural-order groups {0,1}, {2,3}; row 0 by hand: [1, 1] -> s = 1/3,
    # z = 0 -> codes 3, 3; [-1/5, -3/5] -> s = 1/5, z = 3 -> codes 2, 0.
    # (Row 1 lands on exact rounding ties and is not pinned.)
    rt = O.rtn(T2_W, 2, 2, False)
    assert rt.codes[0].tolist() == [3, 3, 2, 0]
    d = T2_W - rt.what
    assert float(np.sum((d @ T2_H) * d)) > 511 / 1620


# ------------------------------------- sweep: independent exact formulation --
def _round_half_even(x: Fraction) -> int:
    f = math.floor(x)
    r = x - f
    if r > Fraction(1, 2):
        return f + 1
    if r < Fraction(1, 2):
        return f
    return f if f % 2 == 0 else f + 1


def _solve(A, b):
    """Exact Gaussian elimination on Fractions."""
    n = len(b)
    M = [list(A[i]) + [b[i]] for i in range(n)]
    for c in range(n):
        p = next(r for r in range(c, n) if M[r][c] != 0)
        M[c], M[p] = M[p], M[c]
        for r in range(n):
            if r != c and M[r][c] != 0:
                f = M[r][c] / M[c][c]
                M[r] = [a - f * bb for a, bb in zip(M[r], M[c])]
    return [M[i][n] / M[i][i] for i in range(n)]


def _schur_gptq_row(w, Hp, bits, gs, sym):
    """One row, quantization order, exact rationals, OBS re-fit form:
    after fixing column j with error e, the remaining set F moves by
    + e * H_FF^-1 H_Fj.  Returns (codes, min distance of any pre-rounding value
    to a rounding boundary)."""
    n = len(w)
    maxq = 2 ** bits - 1
    w = list(w)
    codes = []
    mind = Fraction(10)
    s = z = None
    for j in range(n):
        if j % gs == 0:
            grp = w[j:min(j + gs, n)]
            lo, hi = min(min(grp), 0), max(max(grp), 0)
            if sym:
                hi = max(-lo, hi)
                lo = -hi
            if lo == hi:
                lo, hi = Fraction(-1), Fraction(1)
            s = (hi - lo) / maxq
            if sym:
                z = 2 ** (bits - 1)
            else:
                zp = -lo / s
                mind = min(mind, abs(zp - math.floor(zp) - Fraction(1, 2)))
                z = _round_half_even(zp)
        p = w[j] / s
        mind = min(mind, abs(p - math.floor(p) - Fraction(1, 2)))
        q = min(max(_round_half_even(p) + z, 0), maxq)
        codes.append(q)
        e = w[j] - s * (q - z)
        F = list(range(j + 1, n))
        if F:
            HFF = [[Hp[a][b] for b in F] for a in F]
            HFj = [Hp[a][j] for a in F]
            delta = _solve(HFF, HFj)
            for t, k in enumerate(F):
                w[k] += e * delta[t]
    return codes, mind


@pytest.mark.parametrize("case", range(6))
def test_sweep_matches_exact_schur_form(case):
    rng = np.random.default_rng(100 + case)
    n = 6
    bits = [2, 3, 4, 8, 4, 3][case]
    gs = [-1, 2, 3, 2, 6, -1][case]
    sym = case in (2, 4)
    desc = case % 2 == 1
    A = rng.integers(-3, 4, size=(n + 2, n))
    Hint = 2 * (A.T @ A) + np.diag(rng.integers(1, 4, size=n))
    Wq = rng.integers(-40, 41, size=(3, n))  # multiples of 1/32
    W = Wq / 32.0
    res = O.gptq(W, Hint.astype(float), bits, gs, sym, 0.0, desc)
    perm = res.perm
    Hp = [[Fraction(int(Hint[perm[a], perm[b]])) for b in range(n)] for a in range(n)]
    gse = n if gs == -1 else gs
    for r in range(3):
        wr = [Fraction(int(Wq[r, perm[j]]), 32) for j in range(n)]
        codes, mind = _schur_gptq_row(wr, Hp, bits, gse, sym)
        if mind < Fraction(1, 10 ** 6):
            continue  # a value on a boundary: both roundings are correct
        assert res.codes_perm[r].tolist() == codes


def test_prefix_optimality_reconstructs_codes():
    """Before column j is quantized, the remaining weights of a row are the
    optimum of the layer loss with the prefix fixed:
        w_F = w0_F - (q^_P - w0_P) H_PF H_FF^-1.
    Rebuilding every step of C0 from that characterization (fp64, no sweep)
    gives the oracle's codes wherever a value is not on a rounding boundary."""
    cfg = workloads.get("c0")
    W = workloads.weight(cfg).numpy().astype(np.float64)[:8]
    X = workloads.x_tokens(cfg, 0, 1).numpy()
    H = O.hessian(X)
    res = O.gptq(W, H, cfg.bits, cfg.group_size, cfg.sym, cfg.damp, cfg.desc_act)
    Hd, _ = O.condition(H, cfg.damp)
    perm = res.perm
    Hp = Hd[np.ix_(perm, perm)]
    W0 = W[:, perm]
    n = W.shape[1]
    Q = res.what[:, perm]
    gs = cfg.group_size
    checked = 0
    for j in range(n):
        P, F = slice(0, j), slice(j, n)
        if j == 0:
            cur = W0.copy()
        else:
            corr = (Q[:, P] - W0[:, P]) @ Hp[P, F] @ np.linalg.inv(Hp[F, F])
            cur = np.concatenate([Q[:, P], W0[:, F] - corr], axis=1)
        if j % gs == 0:
            g = j // gs
            grp = cur[:, j:j + gs]
            s, z, _ = O.group_params(grp.min(1), grp.max(1), cfg.bits, cfg.sym)
            assert np.allclose(s, res.scales[g], rtol=1e-6)
        s = res.scales[j // gs].astype(np.float64)
        z = res.zeros[j // gs]
        pre = cur[:, j] / s + z
        dist = np.abs(pre - np.floor(pre) - 0.5)
        q = np.clip(np.rint(cur[:, j] / s) + z, 0, 2 ** cfg.bits - 1)
        ok = dist > 1e-6
        assert np.array_equal(q[ok], res.codes_perm[ok, j])
        checked += int(ok.sum())
    assert checked > 0.99 * W.size


# ------------------------------------------ grid: degenerate range, ties --
@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_all_zero_group_row_hand_trace(bits):
    """An all-zero group-row has lo = hi = 0, so its range becomes [-1, 1]:
    s = 2 / maxq and z = rint(1 / s) = rint(maxq / 2), an exact tie that
    round-half-to-even sends to 2^(b-1) (1.5 -> 2, 3.5 -> 4, 7.5 -> 8,
    127.5 -> 128); every code is then z and every w^ exactly 0.  The group is
    the row's first, so no earlier error reaches it, and its own errors are 0,
    so nothing moves inside it even with a correlated H."""
    maxq = 2 ** bits - 1
    cfg, W, H = _c0_problem(rows=4)
    W = W.copy()
    W[1, :32] = 0.0
    res = O.gptq(W, H, bits, 32, False, 0.01, False)
    want_z = {2: 2, 3: 4, 4: 8, 8: 128}[bits]
    assert want_z == 2 ** (bits - 1)
    assert res.zeros[0, 1] == want_z
    assert res.scales[0, 1] == pytest.approx(2.0 / maxq, rel=1e-15)
    assert res.codes[1, :32].tolist() == [want_z] * 32
    assert np.all(res.what[1, :32] == 0.0)
    # symmetric: the zero is 2^(b-1) by definition and the scale the same
    rs = O.gptq(W, H, bits, 32, True, 0.01, False)
    assert rs.zeros[0, 1] == want_z and rs.codes[1, :32].tolist() == [want_z] * 32
    assert rs.scales[0, 1] == pytest.approx(2.0 / maxq, rel=1e-15)


def test_exact_ties_round_half_to_even():
    """Values that land exactly on a half-integer (H = I: nothing propagates).

    Row 0, 4-bit asym, one group: lo = -2, hi = 1.75 -> s = 3.75 / 15 = 1/4,
    z = rint(8) = 8.  w / s = 2.5, -1.5, 0.5, 3.5, -0.5 round (half to even)
    to 2, -2, 0, 4, -0 -> codes 10, 6, 8, 12, 8.  Half-up would give
    11, 7, 9, 12, 8 and half-away-from-zero 11, 6, 9, 12, 7.
    Row 1: lo = -0.625, hi = 3.125 -> s = 1/4 and -lo / s = 2.5 -> z = 2
    (half-up: 3); w / s = -2.5, 12.5, 1.5, -2.5 -> rint -2, 12, 2, -2 ->
    codes 0, 14, 4, 0 (half-up: 12.5 -> 13 -> code 15).
    """
    W = np.array([[-2.0, 1.75, 0.625, -0.375, 0.125, 0.875, -0.125, 0.0],
                  [-0.625, 3.125, 0.375, -0.625, 0.0, 0.0, 0.0, 0.0]])
    res = O.gptq(W, np.eye(8), 4, -1, False, 0.01, False)
    assert res.scales[0].tolist() == [0.25, 0.25]
    assert res.zeros[0].tolist() == [8, 2]
    assert res.codes[0].tolist() == [0, 15, 10, 6, 8, 12, 8, 8]
    assert res.codes[1].tolist() == [0, 14, 4, 0, 2, 2, 2, 2]
    assert np.array_equal(O.rtn(W, 4, -1, False).codes, res.codes)


def test_layer_error_is_output_error_on_explicit_tokens():
    """layer_error(W, W^, 2 X^T X) equals the squared Frobenius norm of the
    layer's output error X (W - W^)^T, summed here token by token and output
    by output with scalar loops."""
    rng = np.random.default_rng(3)
    t, n, out = 7, 5, 3
    X = rng.normal(size=(t, n))
    W = rng.normal(size=(out, n))
    Wh = W + rng.normal(size=(out, n)) * 0.1
    want = 0.0
    for tt in range(t):
        for r in range(out):
            y = sum(X[tt, k] * (W[r, k] - Wh[r, k]) for k in range(n))
            want += y * y
    assert O.layer_error(W, Wh, O.hessian(X)) == pytest.approx(want, rel=1e-13)
    assert O.layer_error(W, W, O.hessian(X)) == 0.0


# ------------------------------------------------------------ invariants --
def _c0_problem(rows=None):
    cfg = workloads.get("c0")
    W = workloads.weight(cfg).numpy().astype(np.float64)
    if rows is not None:
        W = W[:rows]
    H = O.hessian(workloads.x_tokens(cfg, 0, 1).numpy())
    return cfg, W, H


def test_h_identity_reduces_to_rtn_bit_exact():
    for bits, gs, sym in [(4, 32, False), (2, 32, False), (3, -1, False), (8, 64, False),
                          (4, 64, True), (3, 32, True)]:
        W = workloads.boundary_safe_weight(16, 128, bits, gs, sym).numpy().astype(np.float64)
        g = O.gptq(W, np.eye(128), bits, gs, sym, 0.01, True)
        r = O.rtn(W, bits, gs, sym)
        assert np.array_equal(g.codes, r.codes)
        assert np.array_equal(g.scales, r.scales) and np.array_equal(g.zeros, r.zeros)
        assert np.array_equal(g.perm, np.arange(128))
        # RTN inside the grid range: every weight is within s/2 of its code point
        s = r.scales[r.g_idx, :].T.astype(np.float64)
        assert np.all(np.abs(W - r.what) <= 0.5 * s)
        assert np.all(np.log2(r.scales) == np.round(np.log2(r.scales)))


def test_scale_invariance_bit_identical():
    cfg, W, H = _c0_problem()
    a = O.gptq(W, H, 4, 32, False, 0.01, True)
    b = O.gptq(W, 4.0 * H, 4, 32, False, 0.01, True)
    assert np.array_equal(a.codes, b.codes)
    assert np.array_equal(a.scales, b.scales) and np.array_equal(a.zeros, b.zeros)


def test_permutation_equivariance():
    cfg, W, H = _c0_problem()
    a = O.gptq(W, H, 3, 32, False, 0.01, True)
    p = a.perm
    b = O.gptq(W[:, p], H[np.ix_(p, p)], 3, 32, False, 0.01, False)
    assert np.array_equal(a.codes_perm, b.codes)
    assert np.array_equal(a.scales, b.scales)
    assert np.array_equal(a.codes[:, p], b.codes)


def test_row_independence():
    cfg, W, H = _c0_problem()
    a = O.gptq(W, H, 4, 32, True, 0.01, False)
    rows = [3, 17, 40]
    b = O.gptq(W[rows], H, 4, 32, True, 0.01, False)
    assert np.array_equal(a.codes[rows], b.codes)
    assert np.array_equal(a.scales[:, rows], b.scales)


def test_gptq_beats_rtn_on_correlated_inputs():
    cfg, W, H = _c0_problem()
    for bits, gs, sym, desc in [(4, 32, False, False), (3, 32, False, True),
                                (2, -1, False, False), (4, 64, True, True)]:
        g = O.gptq(W, H, bits, gs, sym, 0.01, desc)
        r = O.rtn(W, bits, gs, sym)
        assert O.layer_error(W, g.what, H) < O.layer_error(W, r.what, H)


def test_dequantize_matches_sweep_output():
    cfg, W, H = _c0_problem()
    g = O.gptq(W, H, 4, 32, False, 0.01, True)
    assert np.array_equal(O.dequantize(g.codes, g.scales, g.zeros, g.g_idx), g.what)


def test_replay_records_and_follows_forced_codes():
    cfg, W, H = _c0_problem(rows=4)
    Hd, _ = O.condition(H, 0.01)
    perm = O.column_order(H, False)
    U = O.hinv_chol(Hd, perm)
    base = O.gptq_sweep(W, U, perm, 4, 32, False)
    forced = base.codes_perm.copy()
    forced[1, 5] = (forced[1, 5] + 1) % 16
    rep = O.gptq_sweep(W, U, perm, 4, 32, False, forced_codes=forced)
    kinds = [(m[0], m[1], m[2]) for m in rep.mismatches]
    assert ("code", 1, 5) in kinds
    assert np.array_equal(rep.codes_perm[:, 5], forced[:, 5])
    assert np.array_equal(rep.codes_perm[[0, 2, 3]], base.codes_perm[[0, 2, 3]])


# ------------------------------------------------------------------ packing --
def _words(codes, bits):
    q = O.pack(np.array([codes]), bits)
    return [int(v) & 0xFFFFFFFF for v in q[:, 0]]


def test_pack_words_from_layout_definition():
    # 4-bit codes 1..8, then zeros: first word 0x87654321
    assert _words(list(range(1, 9)) + [0] * 24, 4)[0] == 0x87654321
    # 2-bit codes k mod 4 for k < 16: every byte is 0b11100100
    assert _words([k % 4 for k in range(32)], 2) == [0xE4E4E4E4, 0xE4E4E4E4]
    # 8-bit codes 1..4
    assert _words([1, 2, 3, 4] + [0] * 28, 8)[0] == 0x04030201
    # 3-bit codes k mod 8: 32 codes -> 3 words, codes straddle word boundaries
    assert _words([k % 8 for k in range(32)], 3) == [0x88FAC688, 0xC688FAC6, 0xFAC688FA]
    assert _words([7] * 32, 3) == [0xFFFFFFFF] * 3


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_pack_roundtrip(bits):
    rng = np.random.default_rng(bits)
    c = rng.integers(0, 2 ** bits, size=(5, 96))
    q = O.pack(c, bits)
    assert q.shape == (96 * bits // 32, 5) and q.dtype == np.int32
    assert np.array_equal(O.unpack(q, bits, 96), c)


def test_g_index():
    assert O.g_index([1, 3, 2, 0], 2).tolist() == [1, 0, 1, 0]
    assert O.g_index([0, 1, 2], -1).tolist() == [0, 0, 0]


# ----------------------------------------------------------- dequant_matmul --
def test_dequant_matmul_worked_example():
    # One output row, 32 inputs, 4-bit: word 0 = 0x87654321 holds codes
    # 1..8 for inputs 0..7, the other words are 0.  Groups of 16: group 0
    # scale 0.5 zero 1, group 1 scale 2 zero 0.  W^ = 0.5 k for k < 8,
    # -0.5 for 8 <= k < 16, 0 above.  Token 1 (all ones): 0.5*28 - 0.5*8 = 10;
    # token 2 (x_k = k): 0.5*140 - 0.5*92 = 24.
    qw = np.zeros((4, 1), dtype=np.int64)
    qw[0, 0] = 0x87654321
    qw = qw.astype(np.uint32).view(np.int32)
    scales = np.array([[0.5], [2.0]], dtype=np.float32)
    zeros = np.array([[1], [0]], dtype=np.int32)
    g_idx = np.array([0] * 16 + [1] * 16, dtype=np.int32)
    x = np.stack([np.ones(32), np.arange(32.0)])
    y = O.dequant_matmul(x, qw, scales, zeros, g_idx, 4)
    assert y.shape == (2, 1)
    assert y[:, 0].tolist() == [10.0, 24.0]


def _bit_loop_codes(qweight, bits, n):
    """Codes by walking the bit stream one bit at a time (independent of
    O.unpack's vectorized form)."""
    q = np.asarray(qweight).astype(np.int64) & 0xFFFFFFFF
    out = q.shape[1]
    codes = np.zeros((out, n), dtype=np.int64)
    for r in range(out):
        for k in range(n):
            v = 0
            for i in range(bits):
                pos = k * bits + i
                v |= ((int(q[pos // 32, r]) >> (pos % 32)) & 1) << i
            codes[r, k] = v
    return codes


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_dequant_matmul_brute_force(bits):
    rng = np.random.default_rng(10 + bits)
    out, n, t, gs = 3, 64, 2, 16
    codes = rng.integers(0, 2 ** bits, size=(out, n))
    qw = O.pack(codes, bits)
    perm = rng.permutation(n)
    g_idx = O.g_index(perm, gs)
    scales = rng.uniform(0.1, 1.0, size=(n // gs, out)).astype(np.float32)
    zeros = rng.integers(0, 2 ** bits, size=(n // gs, out)).astype(np.int32)
    x = rng.normal(size=(t, n)).astype(np.float16).astype(np.float64)
    y = O.dequant_matmul(x, qw, scales, zeros, g_idx, bits)
    c2 = _bit_loop_codes(qw, bits, n)
    ref = np.zeros((t, out))
    for a in range(t):
        for r in range(out):
            ref[a, r] = sum(x[a, k] * float(scales[g_idx[k], r]) * (c2[r, k] - int(zeros[g_idx[k], r]))
                            for k in range(n))
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_dequant_matmul_input_permutation_invariant():
    # Reordering the input features (X columns, the codes' positions in the
    # stream, g_idx) together leaves Y unchanged.
    rng = np.random.default_rng(3)
    out, n, gs, bits = 5, 96, 32, 4
    codes = rng.integers(0, 16, size=(out, n))
    g_idx = O.g_index(rng.permutation(n), gs)
    scales = rng.uniform(0.1, 1.0, size=(n // gs, out)).astype(np.float32)
    zeros = rng.integers(0, 16, size=(n // gs, out)).astype(np.int32)
    x = rng.normal(size=(4, n))
    y = O.dequant_matmul(x, O.pack(codes, bits), scales, zeros, g_idx, bits)
    p = rng.permutation(n)
    y2 = O.dequant_matmul(x[:, p], O.pack(codes[:, p], bits), scales, zeros, g_idx[p], bits)
    assert np.allclose(y, y2, rtol=1e-12, atol=1e-12)


def test_group_order_hand_example():
    # g_idx 2 0 1 0 2 1 over 32 inputs (pattern repeated): sorted by group with
    # ties in input order, the first group-0 inputs are 1, 3, 7, 9, ...
    g_idx = np.array([2, 0, 1, 0, 2, 1] * 5 + [0, 1], dtype=np.int32)
    codes = np.arange(32).reshape(1, 32) % 16
    qs, gs, order = O.group_order(O.pack(codes, 4), g_idx, 4)
    zeros_at = [k for k in range(32) if g_idx[k] == 0]
    ones_at = [k for k in range(32) if g_idx[k] == 1]
    twos_at = [k for k in range(32) if g_idx[k] == 2]
    assert order.tolist() == zeros_at + ones_at + twos_at
    assert order[:4].tolist() == [1, 3, 7, 9]
    assert gs.tolist() == [0] * len(zeros_at) + [1] * len(ones_at) + [2] * len(twos_at)
    # position p of the re-packed stream holds the code of input order[p]
    assert _bit_loop_codes(qs, 4, 32)[0].tolist() == [int(codes[0, k]) for k in order]


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_group_order_same_product_exactly(bits):
    # Integer X and power-of-two scales: every term and partial sum is exact
    # in fp64, so the re-ordered layer must give the identical Y.
    rng = np.random.default_rng(20 + bits)
    out, n, gs = 4, 128, 32
    codes = rng.integers(0, 2 ** bits, size=(out, n))
    g_idx = O.g_index(rng.permutation(n), gs)
    scales = (2.0 ** rng.integers(-6, 0, size=(n // gs, out))).astype(np.float32)
    zeros = rng.integers(0, 2 ** bits, size=(n // gs, out)).astype(np.int32)
    x = rng.integers(-8, 9, size=(3, n)).astype(np.float64)
    qw = O.pack(codes, bits)
    qs, gsrt, order = O.group_order(qw, g_idx, bits)
    assert sorted(order.tolist()) == list(range(n))
    assert np.all(np.diff(gsrt) >= 0)
    y = O.dequant_matmul(x, qw, scales, zeros, g_idx, bits)
    y2 = O.dequant_matmul(x, qs, scales, zeros, gsrt, bits, x_order=order)
    assert np.array_equal(y, y2)
    # the ordered layer's chunks of 32 inputs each hold one group
    assert all(len(set(gsrt[c:c + 32].tolist())) == 1 for c in range(0, n, 32))


def test_silu_mul_closed_forms():
    # SiLU(0) = 0; SiLU(ln 3) = ln 3 / (1 + 1/3) = 0.75 ln 3; SiLU(-ln 3) =
    # -ln 3 / 4; large |g|: g or 0; the up factor multiplies.
    l3 = np.log(3.0)
    g = np.array([0.0, l3, -l3, 40.0, -40.0, l3])
    u = np.array([5.0, 1.0, 1.0, 1.0, 1.0, -2.0])
    want = np.array([0.0, 0.75 * l3, -0.25 * l3, 40.0, 0.0, -1.5 * l3])
    got = O.silu_mul(g, u)
    assert np.allclose(got, want, rtol=1e-15, atol=1e-15)


def _silu_scalar(g):
    return g / (1.0 + math.exp(-g))


def test_mlp_block_down_hessian_from_quantized_gate_up():
    """The down projection's Hessian comes from activations computed with the
    gate and up layers already quantized.  Rebuilt here token by token with
    scalar loops from the dequantized weights (w^ = s (q - z), read from the
    returned codes, scales, zeros and g_idx), and checked to differ from the
    Hessian the unquantized gate and up layers would give."""
    rng = np.random.default_rng(5)
    d, inter, t = 8, 12, 40
    X = rng.normal(size=(t, d)).astype(np.float16).astype(np.float64)
    Wg = (rng.normal(size=(inter, d)) * 0.3).astype(np.float32)
    Wu = (rng.normal(size=(inter, d)) * 0.3).astype(np.float32)
    Wd = (rng.normal(size=(d, inter)) * 0.3).astype(np.float32)
    r = O.mlp_block(X, Wg, Wu, Wd, 3, 4, False, 0.01, True)

    def wq(res, i, k):
        g = int(res.g_idx[k])
        return float(res.scales[g, i]) * (int(res.codes[i, k]) - int(res.zeros[g, i]))

    def act(Wgate, Wup):
        A = [[0.0] * inter for _ in range(t)]
        for tt in range(t):
            for i in range(inter):
                gv = sum(X[tt, k] * Wgate(i, k) for k in range(d))
                uv = sum(X[tt, k] * Wup(i, k) for k in range(d))
                A[tt][i] = _silu_scalar(gv) * uv
        return A

    A = act(lambda i, k: wq(r.gate, i, k), lambda i, k: wq(r.up, i, k))
    Hd = np.zeros((inter, inter))
    for a in range(inter):
        for b in range(inter):
            Hd[a, b] = 2.0 * sum(A[tt][a] * A[tt][b] for tt in range(t))
    assert np.allclose(r.H_down, Hd, rtol=1e-12, atol=1e-12)
    A0 = act(lambda i, k: float(Wg[i, k]), lambda i, k: float(Wu[i, k]))
    H0 = 2.0 * np.array(A0).T @ np.array(A0)
    assert np.linalg.norm(H0 - r.H_down) > 1e-3 * np.linalg.norm(H0)
    # gate and up use the block input's Hessian: same as quantizing them alone
    ref = O.gptq(Wg, 2.0 * X.T @ X, 3, 4, False, 0.01, True)
    assert np.array_equal(ref.codes, r.gate.codes)
    # the down layer's calibration error beats round-to-nearest on its inputs
    Wd64 = Wd.astype(np.float64)
    e = O.layer_error(Wd64, r.down.what, r.H_down)
    e_rtn = O.layer_error(Wd64, O.rtn(Wd64, 3, 4, False).what, r.H_down)
    assert e < e_rtn


def _attn_scalar(Q, K, V, seq_len, heads, causal):
    """Attention with scalar loops and math.exp (no max subtraction)."""
    tokens, w = len(Q), len(Q[0])
    hd = w // heads
    O = [[0.0] * w for _ in range(tokens)]
    for t in range(tokens):
        b0 = (t // seq_len) * seq_len
        for h in range(heads):
            keys = range(b0, t + 1) if causal else range(b0, b0 + seq_len)
            sc = {s_: math.exp(sum(Q[t][h * hd + i] * K[s_][h * hd + i] for i in range(hd))
                               / math.sqrt(hd)) for s_ in keys}
            z = sum(sc.values())
            for i in range(hd):
                O[t][h * hd + i] = sum(sc[s_] * V[s_][h * hd + i] for s_ in keys) / z
    return np.array(O)


@pytest.mark.parametrize("causal", [True, False])
def test_attention_brute_force(causal):
    rng = np.random.default_rng(21)
    seq_len, heads, hd = 4, 2, 3
    Q, K, V = (rng.normal(size=(2 * seq_len, heads * hd)) for _ in range(3))
    got = O.attention(Q, K, V, seq_len, heads, causal)
    want = _attn_scalar(Q.tolist(), K.tolist(), V.tolist(), seq_len, heads, causal)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_attention_closed_forms():
    rng = np.random.default_rng(22)
    seq_len, heads, hd = 5, 2, 4
    Q = rng.normal(size=(2 * seq_len, heads * hd))
    V = rng.normal(size=(2 * seq_len, heads * hd))
    # equal scores (K = 0): causal attention is the running mean of V within
    # each sequence, full attention the sequence mean
    Oc = O.attention(Q, np.zeros_like(Q), V, seq_len, heads, True)
    Of = O.attention(Q, np.zeros_like(Q), V, seq_len, heads, False)
    for b in range(2):
        blk = V[b * seq_len:(b + 1) * seq_len]
        run = np.cumsum(blk, axis=0) / np.arange(1, seq_len + 1)[:, None]
        assert np.allclose(Oc[b * seq_len:(b + 1) * seq_len], run, rtol=1e-13, atol=1e-14)
        assert np.allclose(Of[b * seq_len:(b + 1) * seq_len], blk.mean(axis=0), rtol=1e-13)
    # the first token of a causal sequence attends to itself only
    Oq = O.attention(Q, rng.normal(size=Q.shape), V, seq_len, heads, True)
    assert np.allclose(Oq[[0, seq_len]], V[[0, seq_len]], rtol=1e-14)


def test_residual_rmsnorm_closed_forms():
    rng = np.random.default_rng(23)
    X = rng.normal(size=(3, 6))
    A = rng.normal(size=(3, 6))
    g = rng.normal(size=6)
    Hs, U = O.residual_rmsnorm(X, A, g, 1e-5)
    assert np.array_equal(Hs, X + A)
    for r in range(3):
        ms = sum(v * v for v in Hs[r]) / 6
        for c in range(6):
            assert U[r, c] == pytest.approx(Hs[r, c] / math.sqrt(ms + 1e-5) * g[c], rel=1e-13)
    # a constant row c with eps = 0 normalizes to sign(c) * gamma
    _, Uc = O.residual_rmsnorm(np.full((2, 6), -2.5), np.zeros((2, 6)), g, 0.0)
    assert np.allclose(Uc, -g[None, :], rtol=1e-15)


def test_decoder_block_hessians_through_quantized_layers():
    """The output projection's Hessian is 2 O^T O with O the attention of the
    quantized q, k, v; the MLP's is 2 U^T U with U the normalized residual
    stream after the quantized o.  Rebuilt with scalar loops from the
    dequantized weights (codes, scales, zeros, g_idx) of the returned
    layers; the unquantized path gives a different H_o."""
    rng = np.random.default_rng(24)
    d, inter, heads, seq_len, seqs = 8, 12, 2, 5, 2
    X = rng.normal(size=(seqs * seq_len, d)).astype(np.float16).astype(np.float64)
    Ws = [(rng.normal(size=(d, d)) * 0.3) for _ in range(4)]
    gamma = 1.0 + 0.1 * rng.normal(size=d)
    Wg, Wu = rng.normal(size=(inter, d)) * 0.3, rng.normal(size=(inter, d)) * 0.3
    Wd = rng.normal(size=(d, inter)) * 0.3
    r = O.decoder_block(X, *Ws, gamma, Wg, Wu, Wd, heads, seq_len, 1e-6, 3, 4, False, 0.01, True)

    def wq(res, i, k):
        g = int(res.g_idx[k])
        return float(res.scales[g, i]) * (int(res.codes[i, k]) - int(res.zeros[g, i]))

    def proj(Xl, res):
        return [[sum(Xl[t][k] * wq(res, i, k) for k in range(len(Xl[0])))
                 for i in range(res.codes.shape[0])] for t in range(len(Xl))]

    Xl = X.tolist()
    Oat = _attn_scalar(proj(Xl, r.q), proj(Xl, r.k), proj(Xl, r.v), seq_len, heads, True)
    assert np.allclose(r.O, Oat, rtol=1e-11, atol=1e-12)
    Ho = np.array([[2.0 * sum(Oat[t, a] * Oat[t, b] for t in range(len(Xl)))
                    for b in range(d)] for a in range(d)])
    assert np.allclose(r.H_o, Ho, rtol=1e-11, atol=1e-12)
    O0 = _attn_scalar((X @ Ws[0].T).tolist(), (X @ Ws[1].T).tolist(), (X @ Ws[2].T).tolist(),
                      seq_len, heads, True)
    H0 = 2.0 * O0.T @ O0
    assert np.linalg.norm(H0 - r.H_o) > 1e-4 * np.linalg.norm(H0)
    AO = proj(Oat.tolist(), r.o)
    U = np.zeros((len(Xl), d))
    for t in range(len(Xl)):
        hs = [Xl[t][c] + AO[t][c] for c in range(d)]
        rr = 1.0 / math.sqrt(sum(v * v for v in hs) / d + 1e-6)
        U[t] = [hs[c] * rr * gamma[c] for c in range(d)]
    assert np.allclose(r.U, U, rtol=1e-11, atol=1e-12)
    assert np.allclose(r.mlp.H_in, 2.0 * U.T @ U, rtol=1e-11, atol=1e-12)


def test_pack_zeros_hand_example():
    # 4-bit zeros 1..8 of one group row -> one word 0x87654321; 3-bit zeros
    # 7, 0, 5 start a stream whose low bits are 0b101_000_111 = 0x147;
    # 8-bit zeros 0x11, 0x22, 0x33, 0x44 -> 0x44332211.
    z4 = np.arange(1, 9).reshape(1, 8)
    assert (O.pack_zeros(z4, 4).view(np.uint32) == [[0x87654321]]).all()
    z3 = np.zeros((1, 32), dtype=np.int64)
    z3[0, :3] = [7, 0, 5]
    w3 = O.pack_zeros(z3, 3).view(np.uint32)
    assert w3.shape == (1, 3) and int(w3[0, 0]) == 0x147 and int(w3[0, 1]) == 0
    z8 = np.array([[0x11, 0x22, 0x33, 0x44]])
    assert (O.pack_zeros(z8, 8).view(np.uint32) == [[0x44332211]]).all()


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_pack_zeros_round_trip_bitwise(bits):
    rng = np.random.default_rng(bits)
    z = rng.integers(0, 2 ** bits, size=(3, 64))
    q = O.pack_zeros(z, bits)
    assert q.shape == (3, 64 * bits // 32)
    assert np.array_equal(O.unpack_zeros(q, bits, 64), z)
    # bit by bit: zero r of row g occupies stream bits [r b, (r+1) b)
    qu = q.view(np.uint32).astype(np.int64)
    for g in range(3):
        for r in range(0, 64, 7):
            v = 0
            for i in range(bits):
                pos = r * bits + i
                v |= ((int(qu[g, pos // 32]) >> (pos % 32)) & 1) << i
            assert v == z[g, r]
