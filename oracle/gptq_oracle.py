"""Plain, slow, obviously-correct CPU oracle for GPTQ layer-wise weight quantization.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import this
module.  The product path (the HIP library and its Python binding) never calls
it, and this module shares no code with that path.

Everything is NumPy in float64.  Inputs are upcast exactly from the bytes the
GPU receives (fp16 / bf16 / fp32 are all exactly representable in fp64).

Sources (web pages, cited by title and passage):
  [GLOSS]  "gptq" glossary entry (chipfoundryservices.com): paragraphs
           "Method", "Key innovation", "Algorithm", "Quantization targets",
           "Group quantization".
  [SKILL]  "gptq" agent skill page (nethave.com): section "Group-wise
           quantization" (per-group scale/zero-point, the [1024, 4096] g128
           example) and "Quantization configurations".
  [HANDB]  "GPTQ > Using AutoGPTQ in Practice" (Language AI Handbook):
           "Key Parameters" list (bits, group_size, desc_act, damp_percent).
  [AGPTQ]  "AutoGPTQ" catalogue page (unfragile.ai): calibration paragraph
           (symmetric and asymmetric schemes, reconstruction error).

Where the pages leave a step open, the reading taken is stated at the step.

Every step, including the ones that decide an integer (a group's zero-point,
a code), runs in float64.  A second implementation that decides in a lower
precision can land on the other side of a rounding boundary when its value
sits within rounding of it; ``gptq_sweep``'s replay mode records the distance
of each such disagreement so that a caller can check exactly that.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "NotPositiveDefinite",
    "hessian",
    "condition",
    "column_order",
    "hinv_chol",
    "hinv_chol_reverse",
    "group_params",
    "quantize_codes",
    "SweepResult",
    "gptq_sweep",
    "gptq",
    "rtn",
    "g_index",
    "pack",
    "unpack",
    "dequantize",
    "dequant_matmul",
    "group_order",
    "pack_zeros",
    "unpack_zeros",
    "silu_mul",
    "BlockResult",
    "mlp_block",
    "attention",
    "residual_rmsnorm",
    "DecoderResult",
    "decoder_block",
    "layer_error",
]


class NotPositiveDefinite(ValueError):
    """The damped, permuted Hessian (or its inverse) has no Cholesky factor."""


# ---------------------------------------------------------------------------
# Hessian.  [GLOSS] "Algorithm" step (1): H = d^2 L / dW^2 of the layer loss,
# approximated from calibration data.  For the layer reconstruction loss
# L(W^) = sum_r || X (w_r - w^_r) ||^2 over calibration tokens x_t (rows of X),
# the Hessian with respect to each output row is exactly 2 X^T X.
# Reading: a sum over tokens, not a mean (codes are invariant to H -> cH).
# ---------------------------------------------------------------------------
def hessian(x_chunks) -> np.ndarray:
    """H = 2 * sum_t x_t x_t^T over every calibration token, float64, symmetric.

    ``x_chunks`` is an iterable of [tokens x features] arrays (or one array).
    The upper triangle is computed and mirrored, so H is symmetric bitwise.
    """
    if isinstance(x_chunks, np.ndarray):
        x_chunks = [x_chunks]
    H = None
    for X in x_chunks:
        X64 = np.asarray(X, dtype=np.float64)
        part = 2.0 * (X64.T @ X64)
        H = part if H is None else H + part
    if H is None:
        raise ValueError("no calibration tokens")
    upper = np.triu(H)
    return upper + np.triu(upper, 1).T


# ---------------------------------------------------------------------------
# Damping.  [HANDB] "damp_percent": a fraction of the mean of diag(H) is added
# to the diagonal; the default 0.01 means 1 %.
# Reading (pages silent): a feature whose diagonal entry is exactly 0 (never
# active in the calibration data) gets H_ii := 1 first, then the mean is taken.
# ---------------------------------------------------------------------------
def condition(H: np.ndarray, damp_percent: float):
    """Return (H_damped, mu) with mu = mean(diag H) after the dead-feature fix."""
    Hd = np.array(H, dtype=np.float64, copy=True)
    idx = np.arange(Hd.shape[0])
    dead = Hd[idx, idx] == 0.0
    Hd[idx[dead], idx[dead]] = 1.0
    mu = float(np.mean(Hd[idx, idx]))
    Hd[idx, idx] += float(damp_percent) * mu
    return Hd, mu


# ---------------------------------------------------------------------------
# Column order.  [HANDB] "desc_act": columns are processed by decreasing
# Hessian diagonal.  Reading: the raw diagonal of H (damping shifts every entry
# by the same amount, so it cannot change the order), ties broken by the lower
# original index first (a stable sort).
# ---------------------------------------------------------------------------
def column_order(H: np.ndarray, desc_act: bool) -> np.ndarray:
    n = H.shape[0]
    if not desc_act:
        return np.arange(n, dtype=np.int64)
    d = np.diag(np.asarray(H, dtype=np.float64))
    # A stable ascending sort of the negated keys is a stable descending sort.
    return np.argsort(-d, kind="stable").astype(np.int64)


# ---------------------------------------------------------------------------
# The factor of the inverse Hessian that drives the sweep.  [GLOSS]
# "Algorithm" step (2) adjusts the remaining weights "using H^-1"; [HANDB]
# (introductory paragraph) names the Cholesky factorization as part of the
# work.  The object used is U, the upper-triangular Cholesky factor of
# H_p^-1 (U^T U = H_p^-1), with H_p the damped Hessian in quantization order.
# This is the textbook route: invert, then factor.
# ---------------------------------------------------------------------------
def hinv_chol(Hd: np.ndarray, perm: np.ndarray) -> np.ndarray:
    Hp = np.asarray(Hd, dtype=np.float64)[np.ix_(perm, perm)]
    try:
        np.linalg.cholesky(Hp)
        Hinv = np.linalg.inv(Hp)
        L = np.linalg.cholesky(Hinv)
    except np.linalg.LinAlgError as exc:
        raise NotPositiveDefinite(str(exc)) from exc
    return np.ascontiguousarray(L.T)


def hinv_chol_reverse(Hd: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """Second route to the same U, used only to pin ``hinv_chol``.

    Factor the index-reversed matrix J H_p J = L L^T (lower), so that
    R = J L J is upper with H_p = R R^T; then H_p^-1 = R^-T R^-1 and
    U = R^-1 is upper with positive diagonal: the unique upper Cholesky
    factor of H_p^-1.
    """
    Hp = np.asarray(Hd, dtype=np.float64)[np.ix_(perm, perm)]
    try:
        L = np.linalg.cholesky(Hp[::-1, ::-1])
    except np.linalg.LinAlgError as exc:
        raise NotPositiveDefinite(str(exc)) from exc
    R = L[::-1, ::-1]
    n = R.shape[0]
    # Back substitution column by column: R U = I.
    U = np.zeros_like(R)
    for c in range(n):
        e = np.zeros(n)
        e[c] = 1.0
        x = np.zeros(n)
        for i in range(n - 1, -1, -1):
            x[i] = (e[i] - R[i, i + 1:] @ x[i + 1:]) / R[i, i]
        U[:, c] = x
    return U


# ---------------------------------------------------------------------------
# Group quantization grid.  [SKILL] "Group-wise quantization": each group has
# its own scale / zero-point; [HANDB] "group_size": the number of weights
# sharing quantization parameters; [AGPTQ]: symmetric and asymmetric schemes.
# Readings (pages silent on the formulas):
#   * the range always includes 0: lo = min(0, min w), hi = max(0, max w);
#   * symmetric: hi = max(-lo, hi), lo = -hi, zero fixed at 2^(b-1);
#   * a degenerate range lo == hi becomes [-1, +1];
#   * scale s = (hi - lo) / (2^b - 1); asymmetric zero z = rint(-lo / s);
#   * rint is round-half-to-even.
# ---------------------------------------------------------------------------
def group_params(lo, hi, bits: int, sym: bool):
    """Per-row (scale, zero, pre-rounding zero value) for one group, float64.

    ``lo`` / ``hi`` are the per-row minimum / maximum of the group's current
    values.  Returns float64 scales, int64 zeros and the float64 value the
    zero was rounded from (for boundary checks).
    """
    maxq = (1 << bits) - 1
    lo = np.minimum(np.asarray(lo, dtype=np.float64), 0.0)
    hi = np.maximum(np.asarray(hi, dtype=np.float64), 0.0)
    if sym:
        hi = np.maximum(-lo, hi)
        lo = -hi
    same = lo == hi
    lo = np.where(same, -1.0, lo)
    hi = np.where(same, 1.0, hi)
    scale = (hi - lo) / maxq
    if sym:
        zero_pre = np.full(scale.shape, float(1 << (bits - 1)))
    else:
        zero_pre = -lo / scale
    zero = np.rint(zero_pre).astype(np.int64)
    return scale, zero, zero_pre


def quantize_codes(w, scale, zero, bits: int):
    """q = clamp(rint(w / s) + z, 0, 2^b - 1), float64.

    Returns (codes int64, dequantized w^ = s (q - z) float64, pre-rounding
    value w / s + z float64).
    """
    maxq = (1 << bits) - 1
    w = np.asarray(w, dtype=np.float64)
    s = np.asarray(scale, dtype=np.float64)
    z = np.asarray(zero, dtype=np.int64)
    ratio = w / s
    q = np.clip(np.rint(ratio).astype(np.int64) + z, 0, maxq)
    what = s * (q - z).astype(np.float64)
    return q, what, ratio + z


def _boundary_distance(pre):
    """Distance, in code units, of a pre-rounding value to the nearest half-integer."""
    return np.abs(pre - np.floor(pre) - 0.5)


@dataclass
class SweepResult:
    codes: np.ndarray          # int64 [out x in], ORIGINAL column order
    codes_perm: np.ndarray     # int64 [out x in], quantization order
    scales: np.ndarray         # float64 [n_groups x out]
    zeros: np.ndarray          # int64 [n_groups x out]
    g_idx: np.ndarray          # int64 [in], original column -> group
    perm: np.ndarray           # int64 [in]
    what: np.ndarray           # float64 [out x in], dequantized, original order
    # Replay bookkeeping: (kind, row, column-or-group, forced, own, distance)
    mismatches: list = field(default_factory=list)


# ---------------------------------------------------------------------------
# The sweep.  [GLOSS] "Algorithm" step (2): for each weight in order, quantize
# it, compute the error, and adjust the remaining weights using H^-1 to
# compensate ("Key innovation").  With U the upper Cholesky factor of H_p^-1,
# the adjustment after fixing column j (error e = w_j - w^_j) is
#     w_k -= (e / U_jj) * U_jk      for every k > j,
# which is the optimal re-fit of the remaining weights (the row of U is the
# Schur-complement row of H_p^-1).  Rows of W are independent: every update
# uses only the row's own error.  Groups ([SKILL] "Group-wise quantization"):
# group_size consecutive columns in quantization order; the group's scale and
# zero are taken when its first column comes up, from the group's current
# (already error-updated) values.  group_size = -1 means one group per row.
# ---------------------------------------------------------------------------
def gptq_sweep(W, U, perm, bits: int, group_size: int, sym: bool,
               forced_codes=None, forced_zeros=None) -> SweepResult:
    """Column-by-column GPTQ sweep of W (original column order) with factor U.

    ``U`` is the upper Cholesky factor of the inverse damped Hessian in
    quantization order (as from ``hinv_chol``).  Unblocked: exactly the
    pages' per-weight order.

    Replay (optional; for checking a second implementation's output): when
    ``forced_codes`` ([out x in], quantization order) / ``forced_zeros``
    ([n_groups x out]) are given and differ from this oracle's own decision,
    the mismatch is recorded with the distance of this oracle's pre-rounding
    value to the rounding boundary, and the forced value is used from then
    on.  Several results are correct only where a value sits on a boundary
    within rounding; the recorded distance lets the caller check exactly that.
    """
    if bits not in (2, 3, 4, 8):
        raise ValueError("bits must be 2, 3, 4 or 8")
    W64 = np.asarray(W, dtype=np.float64)
    out, n = W64.shape
    U64 = np.asarray(U, dtype=np.float64)
    perm = np.asarray(perm, dtype=np.int64)
    Wp = W64[:, perm].copy()
    gs = n if group_size == -1 else int(group_size)
    n_groups = 1 if group_size == -1 else -(-n // gs)
    scales = np.zeros((n_groups, out), dtype=np.float64)
    zeros = np.zeros((n_groups, out), dtype=np.int64)
    codes_perm = np.zeros((out, n), dtype=np.int64)
    what_perm = np.zeros((out, n), dtype=np.float64)
    mismatches = []
    s = z = None
    for j in range(n):
        if j % gs == 0:
            g = j // gs
            cols = slice(j, min(j + gs, n))
            lo = Wp[:, cols].min(axis=1)
            hi = Wp[:, cols].max(axis=1)
            s, z, z_pre = group_params(lo, hi, bits, sym)
            if forced_zeros is not None:
                fz = np.asarray(forced_zeros[g], dtype=np.int64)
                for r in np.nonzero(fz != z)[0]:
                    mismatches.append(("zero", int(r), g, int(fz[r]), int(z[r]),
                                       float(_boundary_distance(z_pre[r]))))
                z = fz
            scales[g] = s
            zeros[g] = z
        q, what, pre = quantize_codes(Wp[:, j], s, z, bits)
        if forced_codes is not None:
            fq = np.asarray(forced_codes[:, j], dtype=np.int64)
            for r in np.nonzero(fq != q)[0]:
                mismatches.append(("code", int(r), j, int(fq[r]), int(q[r]),
                                   float(_boundary_distance(pre[r]))))
            q = fq
            what = s * (q - z).astype(np.float64)
        codes_perm[:, j] = q
        what_perm[:, j] = what
        err = Wp[:, j] - what
        # Compensation: adjust every not-yet-quantized weight of the row.
        Wp[:, j + 1:] -= np.outer(err / U64[j, j], U64[j, j + 1:])
    codes = np.empty_like(codes_perm)
    codes[:, perm] = codes_perm
    what_orig = np.empty_like(what_perm)
    what_orig[:, perm] = what_perm
    return SweepResult(codes=codes, codes_perm=codes_perm, scales=scales,
                       zeros=zeros, g_idx=g_index(perm, group_size), perm=perm,
                       what=what_orig, mismatches=mismatches)


def g_index(perm, group_size: int) -> np.ndarray:
    """g_idx[perm[j]] = j // group_size (0 for one group per row)."""
    perm = np.asarray(perm, dtype=np.int64)
    n = perm.shape[0]
    g = np.zeros(n, dtype=np.int64)
    if group_size != -1:
        g[perm] = np.arange(n) // group_size
    return g


def gptq(W, H, bits: int, group_size: int, sym: bool, damp_percent: float,
         desc_act: bool) -> SweepResult:
    """The whole layer: condition, order, factor, sweep."""
    Hd, _ = condition(H, damp_percent)
    perm = column_order(H, desc_act)
    U = hinv_chol(Hd, perm)
    return gptq_sweep(W, U, perm, bits, group_size, sym)


def rtn(W, bits: int, group_size: int, sym: bool) -> SweepResult:
    """Round-to-nearest baseline ("blind" quantization in [AGPTQ]'s words):
    the same grid, natural-order groups, parameters from the original W and
    no error compensation."""
    W64 = np.asarray(W, dtype=np.float64)
    out, n = W64.shape
    gs = n if group_size == -1 else int(group_size)
    n_groups = 1 if group_size == -1 else -(-n // gs)
    scales = np.zeros((n_groups, out), dtype=np.float64)
    zeros = np.zeros((n_groups, out), dtype=np.int64)
    codes = np.zeros((out, n), dtype=np.int64)
    what = np.zeros((out, n), dtype=np.float64)
    for g in range(n_groups):
        cols = slice(g * gs, min((g + 1) * gs, n))
        s, z, _ = group_params(W64[:, cols].min(axis=1), W64[:, cols].max(axis=1), bits, sym)
        scales[g] = s
        zeros[g] = z
        for j in range(cols.start, cols.stop):
            q, wh, _ = quantize_codes(W64[:, j], s, z, bits)
            codes[:, j] = q
            what[:, j] = wh
    perm = np.arange(n, dtype=np.int64)
    return SweepResult(codes=codes, codes_perm=codes.copy(), scales=scales, zeros=zeros,
                       g_idx=g_index(perm, group_size), perm=perm, what=what)


# ---------------------------------------------------------------------------
# Dense b-bit storage.  [GLOSS] "Quantization targets" and [SKILL] list 2/3/4/8
# bits and the memory reductions that dense storage gives.  Layout (reading):
# per output channel r the codes of input columns 0..in-1 form one
# little-endian bit stream (column k at bits [k*b, (k+1)*b)), cut into 32-bit
# words; word w of channel r is stored at qweight[w, r], so qweight is
# [in*b/32 x out].  in must be a multiple of 32 (3-bit: 32 codes per 3 words).
# ---------------------------------------------------------------------------
def pack(codes, bits: int) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.int64)
    out, n = codes.shape
    if n % 32:
        raise ValueError("in must be a multiple of 32")
    if codes.min(initial=0) < 0 or codes.max(initial=0) >= (1 << bits):
        raise ValueError("code out of range")
    # bit i of code k of row r is stream bit k*bits + i
    bitplanes = (codes[:, :, None] >> np.arange(bits)[None, None, :]) & 1
    stream = bitplanes.reshape(out, n * bits)
    words = stream.reshape(out, n * bits // 32, 32)
    vals = (words << np.arange(32, dtype=np.int64)[None, None, :]).sum(axis=2)
    return vals.astype(np.uint32).view(np.int32).T.copy()


def unpack(qweight, bits: int, n: int) -> np.ndarray:
    q = np.asarray(qweight).astype(np.int32).view(np.uint32).astype(np.int64).T  # [out x words]
    out = q.shape[0]
    bitsarr = (q[:, :, None] >> np.arange(32, dtype=np.int64)[None, None, :]) & 1
    stream = bitsarr.reshape(out, -1)[:, : n * bits].reshape(out, n, bits)
    return (stream << np.arange(bits, dtype=np.int64)[None, None, :]).sum(axis=2)


def dequantize(codes, scales, zeros, g_idx) -> np.ndarray:
    """W^[r, k] = s[g_idx[k], r] * (code[r, k] - z[g_idx[k], r]) in float64."""
    codes = np.asarray(codes, dtype=np.float64)
    g = np.asarray(g_idx, dtype=np.int64)
    s = np.asarray(scales, dtype=np.float64)[g, :].T
    z = np.asarray(zeros, dtype=np.float64)[g, :].T
    return s * (codes - z)


def dequant_matmul(x, qweight, scales, zeros, g_idx, bits: int, x_order=None) -> np.ndarray:
    """Y = X W^T with W the layer's dequantized weights, in float64.

    [GLOSS] paragraph "Inference": the quantized layer is applied by
    dequantizing the weights during the computation and multiplying.  The
    definition written out: Y[t, r] = sum_k X[t, k] * s[g_idx[k], r] *
    (code[r, k] - z[g_idx[k], r]), with code[r, k] the k-th b-bit field of
    row r's little-endian bit stream in qweight (the packed layer as
    gptq_quantize_layer writes it; see ``unpack``).  With x_order (a layer
    from ``group_order``), packed position k multiplies X column
    x_order[k] instead of column k.
    """
    x = np.asarray(x, dtype=np.float64)
    if x_order is not None:
        x = x[:, np.asarray(x_order, dtype=np.int64)]
    n = x.shape[1]
    codes = unpack(qweight, bits, n)
    return x @ dequantize(codes, scales, zeros, g_idx).T


def group_order(qweight, g_idx, bits: int):
    """(qweight_sorted, g_idx_sorted, x_order) of a packed layer.

    With desc_act ([HANDB] Key Parameters) the groups are formed in the
    permuted column order, so the packed layer's g_idx (original order)
    changes group from one input to the next.  Sorting the inputs by group,
    ties kept in input order (a stable sort), gives x_order; the codes are
    re-packed in that order and g_idx_sorted = g_idx[x_order].  The product
    with X[:, x_order] is the same sum over the same terms.
    """
    g = np.asarray(g_idx, dtype=np.int64)
    n = g.shape[0]
    x_order = np.argsort(g, kind="stable")
    codes = unpack(qweight, bits, n)
    return (pack(codes[:, x_order], bits), g[x_order].astype(np.int32),
            x_order.astype(np.int32))


def pack_zeros(zeros, bits: int) -> np.ndarray:
    """Zero-points in storage form: row g of the result is the little-endian
    b-bit stream of zeros[g][0 .. out-1] cut into 32-bit words (zero r at bits
    [r b, (r+1) b)): the codes' dense packing ([GLOSS] "Quantization
    targets") applied along the output channels (a reading: the pages store
    the parameters with the model but do not give their layout)."""
    z = np.asarray(zeros, dtype=np.int64)
    G, out = z.shape
    if (out * bits) % 32:
        raise ValueError("out * bits must be a multiple of 32")
    if z.min(initial=0) < 0 or z.max(initial=0) >= (1 << bits):
        raise ValueError("zero-point out of range")
    stream = ((z[:, :, None] >> np.arange(bits)[None, None, :]) & 1).reshape(G, out * bits)
    words = stream.reshape(G, out * bits // 32, 32)
    vals = (words << np.arange(32, dtype=np.int64)[None, None, :]).sum(axis=2)
    return vals.astype(np.uint32).view(np.int32)


def unpack_zeros(qzeros, bits: int, out: int) -> np.ndarray:
    """Inverse of pack_zeros."""
    q = np.asarray(qzeros).astype(np.int32).view(np.uint32).astype(np.int64)
    G = q.shape[0]
    stream = ((q[:, :, None] >> np.arange(32, dtype=np.int64)[None, None, :]) & 1).reshape(G, -1)
    fields = stream[:, : out * bits].reshape(G, out, bits)
    return (fields << np.arange(bits, dtype=np.int64)[None, None, :]).sum(axis=2)


def silu_mul(g, u) -> np.ndarray:
    """SiLU(g) * u = g / (1 + e^-g) * u elementwise, float64: the gated
    activation that feeds the down projection of a Llama MLP (the pages name
    the Llama layers, not the activation; a reading)."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    return g / (1.0 + np.exp(-g)) * u


@dataclass
class BlockResult:
    H_in: np.ndarray        # 2 X^T X of the block input
    gate: SweepResult
    up: SweepResult
    A: np.ndarray           # the down projection's calibration inputs
    H_down: np.ndarray      # 2 A^T A
    down: SweepResult


def mlp_block(X, Wg, Wu, Wd, bits: int, group_size: int, sym: bool, damp_percent: float,
              desc_act: bool) -> BlockResult:
    """Layer-wise GPTQ over a Llama-style MLP block y = Wd (SiLU(Wg x) * (Wu x)).

    [GLOSS] paragraph "Method" (1): one layer at a time, with calibration
    activations computed through the block (3).  Reading: gate and up share
    the block input, so one Hessian serves both; the down projection's
    inputs are then computed with the gate and up layers already quantized
    (their dequantized weights W^), and its Hessian comes from those.  The
    forward is exact arithmetic in float64: G = X W^g^T, U = X W^u^T,
    A = SiLU(G) * U.
    """
    X64 = np.asarray(X, dtype=np.float64)
    H_in = hessian(X64)
    gate = gptq(Wg, H_in, bits, group_size, sym, damp_percent, desc_act)
    up = gptq(Wu, H_in, bits, group_size, sym, damp_percent, desc_act)
    A = silu_mul(X64 @ gate.what.T, X64 @ up.what.T)
    H_down = hessian(A)
    down = gptq(Wd, H_down, bits, group_size, sym, damp_percent, desc_act)
    return BlockResult(H_in=H_in, gate=gate, up=up, A=A, H_down=H_down, down=down)


def attention(Q, K, V, seq_len: int, heads: int, causal: bool = True) -> np.ndarray:
    """Multi-head softmax attention per sequence, float64.

    [GLOSS] paragraph "Method" (1) and (3): each layer's calibration inputs
    are computed through the model; in a Llama decoder block the output
    projection's input is the attention of the query, key and value
    projections.  The pages do not give the block's arithmetic; the reading
    is plain scaled dot-product attention per head, causal (a decoder
    model), without positional rotation:
        O[t, head] = sum_s P[t, s] V[s, head],
        P[t, :] = softmax_s(Q[t, head] . K[s, head] / sqrt(hd)), s <= t.
    Q, K, V: [tokens x heads * hd], tokens = seqs * seq_len, sequences
    contiguous.  The largest score of a row is subtracted before the
    exponential (the same softmax in exact arithmetic).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    tokens, w = Q.shape
    hd = w // heads
    O = np.zeros((tokens, w))
    for b in range(tokens // seq_len):
        rows = slice(b * seq_len, (b + 1) * seq_len)
        for h in range(heads):
            cols = slice(h * hd, (h + 1) * hd)
            S = Q[rows, cols] @ K[rows, cols].T / math.sqrt(hd)
            if causal:
                S[np.triu_indices(seq_len, 1)] = -np.inf
            S = S - S.max(axis=1, keepdims=True)
            P = np.exp(S)
            P /= P.sum(axis=1, keepdims=True)
            O[rows, cols] = P @ V[rows, cols]
    return O


def residual_rmsnorm(X, A, gamma, eps: float):
    """(Hs, U): the residual stream Hs = X + A and its RMS normalization
    U = Hs / sqrt(mean(Hs^2) + eps) * gamma per row, float64 (the Llama
    block's normalization before the MLP; a reading, the pages do not give
    the block's arithmetic)."""
    Hs = np.asarray(X, dtype=np.float64) + np.asarray(A, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(Hs * Hs, axis=1, keepdims=True) + float(eps))
    return Hs, Hs * r * np.asarray(gamma, dtype=np.float64)[None, :]


@dataclass
class DecoderResult:
    H_x: np.ndarray         # 2 X^T X of the block input (q, k, v)
    q: SweepResult
    k: SweepResult
    v: SweepResult
    O: np.ndarray           # attention output: the output projection's inputs
    H_o: np.ndarray         # 2 O^T O
    o: SweepResult
    U: np.ndarray           # normalized residual stream: the MLP's inputs
    mlp: BlockResult        # gate, up (H = 2 U^T U), down


def decoder_block(X, Wq, Wk, Wv, Wo, gamma, Wg, Wu, Wd, heads: int, seq_len: int, eps: float,
                  bits: int, group_size: int, sym: bool, damp_percent: float,
                  desc_act: bool) -> DecoderResult:
    """Layer-wise GPTQ over a Llama-style decoder block, float64 forward.

    [GLOSS] paragraph "Method" (1): one layer at a time, each from
    calibration activations computed through the block with the layers
    before it already quantized.  Readings: q, k and v share the block
    input, hence one Hessian; the output projection is calibrated on the
    attention of the quantized q, k, v; the MLP on the normalized residual
    stream X + O W^o^T after the quantized output projection (then as in
    ``mlp_block``).
    """
    X64 = np.asarray(X, dtype=np.float64)
    H_x = hessian(X64)
    q = gptq(Wq, H_x, bits, group_size, sym, damp_percent, desc_act)
    k = gptq(Wk, H_x, bits, group_size, sym, damp_percent, desc_act)
    v = gptq(Wv, H_x, bits, group_size, sym, damp_percent, desc_act)
    O = attention(X64 @ q.what.T, X64 @ k.what.T, X64 @ v.what.T, seq_len, heads)
    H_o = hessian(O)
    o = gptq(Wo, H_o, bits, group_size, sym, damp_percent, desc_act)
    _, U = residual_rmsnorm(X64, O @ o.what.T, gamma, eps)
    mlp = mlp_block(U, Wg, Wu, Wd, bits, group_size, sym, damp_percent, desc_act)
    return DecoderResult(H_x=H_x, q=q, k=k, v=v, O=O, H_o=H_o, o=o, U=U, mlp=mlp)


def layer_error(W, What, H) -> float:
    """Calibration error ||X (W - W^)^T||_F^2 = 1/2 sum_r d_r^T H d_r, H = 2 X^T X (undamped)."""
    D = np.asarray(W, dtype=np.float64) - np.asarray(What, dtype=np.float64)
    return 0.5 * float(np.sum((D @ np.asarray(H, dtype=np.float64)) * D))


def storage_bits_per_weight(bits: int, group_size: int, scale_bits: int = 16) -> float:
    """Storage per weight with one scale (scale_bits) and one b-bit zero per group-row."""
    if group_size == -1:
        return float(bits)
    return bits + (scale_bits + bits) / group_size


def n_groups_total(rows: int, cols: int, group_size: int) -> int:
    """Number of (row, group) pairs for a [rows x cols] matrix grouped along cols."""
    return rows * (1 if group_size == -1 else math.ceil(cols / group_size))
