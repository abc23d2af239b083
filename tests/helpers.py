"""Shared test helpers: comparison of the HIP path with the oracle.

The oracle is run on the very same input bytes the GPU receives.  Where a
floating-point value decides an integer (a code, a zero-point), the oracle
decides in float64 and the kernels in float32; a disagreement is accepted
only where the oracle's own pre-rounding value lies within 1e-3 (code units)
of a rounding boundary, and at most 0.1 % of entries may disagree.  After such a
disagreement the oracle continues from the GPU's decision (teacher forcing),
so one boundary case cannot cascade along a row and every later value is
still checked against an exact GPTQ continuation.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as O

CODE_WINDOW = 1e-3       # code units
CODE_FRACTION = 1e-3     # at most 0.1 % of codes may differ
SCALE_RTOL = 1e-3


def np64(t) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy() if t.dtype != torch.int32 \
        else t.detach().to("cpu").numpy()


def gpu_codes(qweight, bits, inp):
    return O.unpack(qweight.cpu().numpy(), bits, inp)


def check_quantize_parity(W_t, U_t, perm_t, bits, gs, sym, qweight, scales, zeros, g_idx,
                          rows=None):
    """Stage check of gptq_quantize_layer against the oracle sweep in replay mode.

    W_t, U_t, perm_t: the exact inputs the GPU got.  rows: optional subset of
    output rows (rows are independent, so a subset is an exact check of those
    rows).  Returns a dict of diagnostics; asserts the tolerances.
    """
    out, inp = W_t.shape
    if rows is None:
        rows = np.arange(out)
    rows = np.asarray(rows)
    W = W_t.detach()[torch.from_numpy(rows)].cpu().to(torch.float64).numpy()
    U = U_t.detach().cpu().to(torch.float64).numpy()
    perm = np.arange(inp) if perm_t is None else perm_t.cpu().numpy().astype(np.int64)
    qsel = qweight.detach()[:, torch.from_numpy(rows).to(qweight.device)]
    codes = gpu_codes(qsel, bits, inp)                       # [rows x in], original order
    sc = scales.cpu().numpy()
    zr = zeros.cpu().numpy().astype(np.int64)
    gi = g_idx.cpu().numpy().astype(np.int64)
    codes_perm = codes[:, perm]
    ref = O.gptq_sweep(W, U, perm, bits, gs, sym,
                       forced_codes=codes_perm, forced_zeros=zr[:, rows])
    assert np.array_equal(gi, O.g_index(perm, gs)), "g_idx differs"
    code_mm = [m for m in ref.mismatches if m[0] == "code"]
    zero_mm = [m for m in ref.mismatches if m[0] == "zero"]
    total = codes_perm.size
    worst = max([m[5] for m in ref.mismatches], default=0.0)
    # boundary distance of the oracle's own pre-rounding value for every mismatch
    far = [m for m in ref.mismatches if m[5] > CODE_WINDOW]
    assert not far, f"{len(far)} decisions differ away from a rounding boundary, e.g. {far[:3]}"
    assert len(code_mm) <= CODE_FRACTION * total, f"{len(code_mm)} of {total} codes differ"
    assert len(zero_mm) <= CODE_FRACTION * zr[:, rows].size
    rel = np.abs(sc[:, rows].astype(np.float64) - ref.scales.astype(np.float64)) / \
        np.maximum(np.abs(ref.scales.astype(np.float64)), 1e-30)
    assert rel.max() <= SCALE_RTOL, f"scale rel err {rel.max()}"
    assert codes.min() >= 0 and codes.max() < 2 ** bits
    return {"code_mismatches": len(code_mm), "zero_mismatches": len(zero_mm),
            "entries": total, "worst_distance": worst, "scale_rel": float(rel.max())}


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def upper_mirror(H: np.ndarray) -> np.ndarray:
    u = np.triu(H)
    return u + np.triu(u, 1).T


def with_ties(W, bits, gs, sym):
    """Boundary-safe W with three rows rewritten (H = I cases):
    row 0 all zero: every group-row is degenerate (range [-1, 1], zero 2^(b-1));
    row 1: every value but the group's extremes moved to an exact half-integer
    multiple of the scale, (c + 1/2) s, so every such code is an exact tie;
    row 2 (asymmetric): the extremes moved to -(z + 1/2) s and
    (maxq - z - 1/2) s, so the zero -lo / s = z + 1/2 is an exact tie (the
    scale stays s) and the other values are clipped into the new range.
    All values stay exact in fp16."""
    W = W.clone().double()
    out, inp = W.shape
    maxq = (1 << bits) - 1
    g = inp if gs == -1 else gs
    r = O.rtn(W[:3].numpy(), bits, gs, sym)      # rows are independent
    W[0] = 0.0
    for c0 in range(0, inp, g):
        grp = W[1, c0:c0 + g]
        s = float(r.scales[c0 // g, 1])
        z = int(r.zeros[c0 // g, 1])
        lo_i, hi_i = int(torch.argmin(grp)), int(torch.argmax(grp))
        rng = np.random.default_rng(c0 + 7)
        for j in range(grp.numel()):
            if j in (lo_i, hi_i):
                continue
            if sym:
                c = int(rng.integers(-(maxq // 2), maxq // 2))        # |c + 1/2| < maxq / 2
            else:
                c = int(rng.integers(-z, maxq - z))                   # c + 1/2 inside [-z, maxq - z]
            W[1, c0 + j] = (c + 0.5) * s
        if not sym and out > 2:
            grp2 = W[2, c0:c0 + g]
            s2 = float(r.scales[c0 // g, 2])
            z2 = int(r.zeros[c0 // g, 2])
            z2 = min(max(z2, 1), maxq - 2)
            lo2, hi2 = -(z2 + 0.5) * s2, (maxq - z2 - 0.5) * s2
            grp2.clamp_(lo2, hi2)
            grp2[int(torch.argmin(grp2))] = lo2
            grp2[int(torch.argmax(grp2))] = hi2
    return W.float()
