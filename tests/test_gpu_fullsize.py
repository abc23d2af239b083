"""Parity at the full layer sizes (Llama-7B q_proj / down_proj, Llama-70B
down_proj shapes, 128 x 2048 calibration tokens), in the launch configuration
bench.py times (32768-token Hessian chunks, one prepare, one quantize call),
on outputs the oracle can compute one by one:

* Hessian: sampled entries H_ij = 2 sum_t x_ti x_tj in fp64 from the same X
  columns; |dH_ij| <= 1e-3 * sqrt(H_ii H_jj) per entry (the natural scale of an
  entry; the relative Frobenius bound 1e-3 is estimated on the sample too).
* Prepare: the full oracle factor where it finishes in seconds (n = 4096,
  11008); at n = 28672 the residual (U^T U H_p - I) on sampled columns and the
  exact perm.  The input H is a torch fp32 product, not the HIP path's.
* Quantize: sampled output rows (rows are independent) against the oracle
  sweep in replay mode, from the oracle's factor (n = 4096) or a synthetic
  dense upper-triangular factor (larger n).
"""
import numpy as np
import pytest
import torch

import oracle as O
import post_weight_quantization_12_amd as P
import workloads
from helpers import check_quantize_parity

pytestmark = pytest.mark.gpu
DEV = "cuda"
CHUNK = 16 * 2048  # tokens per gptq_hessian_accumulate call (as bench.py)


def _banner(msg):
    print(f"[case] {msg}", flush=True)


def _x_full(cfg):
    X = torch.empty((cfg.tokens, cfg.inp), dtype=torch.float16, device=DEV)
    mixing = workloads._mixing(cfg, DEV, 0)
    outl = workloads.outlier_channels(cfg, DEV, 0)
    T = cfg.tokens_per_sample
    for s in range(cfg.samples):
        X[s * T:(s + 1) * T] = workloads.x_sample(cfg, s, DEV, 0, mixing, outl)
    return X


def _sample_features(cfg, k=10, seed=5):
    n = cfg.inp
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 127, 128, 255, 256, 257, n // 2, n - 2, n - 1]
    outl = workloads.outlier_channels(cfg, "cpu", 0).numpy().tolist()[:3]
    rand = rng.choice(n, size=k, replace=False).tolist()
    return sorted(set(int(i) for i in fixed + outl + rand if 0 <= i < n))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cname", ["c1", "c3", "c4a"])
def test_hessian_full_size_sampled(cname):
    cfg = workloads.get(cname)
    _banner(f"full-size hessian {cname} n={cfg.inp} tokens={cfg.tokens}")
    X = _x_full(cfg)
    n = cfg.inp
    H = torch.zeros((n, n), dtype=torch.float32, device=DEV)
    ws = torch.empty((P.hessian_workspace_bytes(n),), dtype=torch.uint8, device=DEV)
    for t0 in range(0, cfg.tokens, CHUNK):
        P.hessian_accumulate(H, X[t0:t0 + CHUNK], workspace=ws)
    torch.cuda.synchronize()
    idx = _sample_features(cfg)
    cols = X[:, idx].to("cpu").numpy().astype(np.float64)       # the same fp16 bytes
    del X
    Hs = H[idx][:, idx].cpu().numpy().astype(np.float64)
    ref = 2.0 * (cols.T @ cols)                                    # fp64 brute sums
    num = den = 0.0
    for a in range(len(idx)):
        for b in range(a, len(idx)):
            d = abs(Hs[a, b] - ref[a, b])
            scale = np.sqrt(ref[a, a] * ref[b, b])
            assert d <= 1e-3 * scale, (idx[a], idx[b], Hs[a, b], ref[a, b])
            num += d * d
            den += ref[a, b] ** 2
    rel = np.sqrt(num / den)
    print(f"  sampled {len(idx)}x{len(idx)} entries, rel fro {rel:.2e}")
    assert rel <= 1e-3
    # the strictly lower triangle is never written
    assert float(H[1, 0].item()) == 0.0 and float(H[n - 1, 0].item()) == 0.0


def _torch_hessian(cfg):
    """H = 2 X^T X by a torch fp32 matmul (independent of the HIP path)."""
    X = _x_full(cfg)
    n = cfg.inp
    H = torch.zeros((n, n), dtype=torch.float32, device=DEV)
    for t0 in range(0, cfg.tokens, CHUNK):
        xc = X[t0:t0 + CHUNK].float()
        H.addmm_(xc.T.contiguous(), xc, alpha=2.0)
    del X
    torch.cuda.synchronize()
    return H


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cname", ["c1", "c3"])
def test_prepare_full_size_against_oracle(cname):
    cfg = workloads.get(cname)
    _banner(f"full-size prepare {cname} n={cfg.inp}")
    H = _torch_hessian(cfg)
    U, perm, info = P.prepare(H, cfg.damp, cfg.desc_act)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    H64 = H.cpu().numpy().astype(np.float64)
    H64 = np.triu(H64) + np.triu(H64, 1).T
    Hd, _ = O.condition(H64, cfg.damp)
    perm_o = O.column_order(H64, cfg.desc_act)
    assert np.array_equal(perm.cpu().numpy(), perm_o)
    Uo = O.hinv_chol(Hd, perm_o)
    Ug = U.cpu().numpy().astype(np.float64)
    err = np.linalg.norm(Ug - Uo) / np.linalg.norm(Uo)
    print(f"  U rel err {err:.2e}")
    assert err <= 2e-3
    assert np.all(np.tril(Ug, -1) == 0)


@pytest.mark.timeout(900)
def test_prepare_full_size_residual_70b():
    cfg = workloads.get("c4a")
    n = cfg.inp
    _banner(f"full-size prepare c4 n={n} (sampled residual)")
    H = _torch_hessian(cfg)
    U, perm, info = P.prepare(H, cfg.damp, True)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    diag = torch.diagonal(H).cpu().numpy().astype(np.float64)
    perm_o = O.column_order(np.diag(diag), True)
    pg = perm.cpu().numpy()
    assert np.array_equal(pg, perm_o)
    # damped, permuted H columns and U, all in fp64 on the host
    mu = float(np.mean(np.where(diag == 0, 1.0, diag)))
    rng = np.random.default_rng(11)
    cols = sorted(set([0, 1, n // 2, n - 2, n - 1] + rng.choice(n, 7, replace=False).tolist()))
    Ug = U.cpu().numpy().astype(np.float64)
    worst = 0.0
    for c in cols:
        src = int(pg[c])
        col = torch.cat([H[:src, src], H[src, src:]]).cpu().numpy().astype(np.float64)  # H[:, src]
        col = col[pg]                                   # H_p[:, c]
        col[c] += cfg.damp * mu
        r = Ug.T @ (Ug @ col)
        r[c] -= 1.0
        worst = max(worst, float(np.linalg.norm(r)))
    print(f"  worst ||(U^T U H_p - I) e_c|| = {worst:.2e}")
    assert worst <= 1e-2


QFULL = [("c1", "oracle"), ("c2", "oracle"), ("c3", "synthetic"), ("c4a", "synthetic"),
         ("c4b", "synthetic")]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cname,factor", QFULL, ids=[q[0] for q in QFULL])
def test_quantize_full_size_sampled_rows(cname, factor):
    cfg = workloads.get(cname)
    out, n = cfg.out, cfg.inp
    _banner(f"full-size quantize {cname} {out}x{n} {cfg.bits}b g{cfg.group_size} "
            f"sym={cfg.sym} factor={factor}")
    if factor == "oracle":
        H = _torch_hessian(cfg)
        H64 = H.cpu().numpy().astype(np.float64)
        del H
        H64 = np.triu(H64) + np.triu(H64, 1).T
        Hd, _ = O.condition(H64, cfg.damp)
        perm = O.column_order(H64, cfg.desc_act)
        U32 = torch.from_numpy(O.hinv_chol(Hd, perm).astype(np.float32))
    else:
        U32 = workloads.synthetic_hinv_chol(n, "cpu", 0)
        perm = np.random.default_rng(3).permutation(n) if cfg.desc_act else np.arange(n)
    W = workloads.weight(cfg, DEV)
    perm_t = torch.from_numpy(perm.astype(np.int32)).to(DEV)
    qw, sc, zr, gi = P.quantize_layer(W, U32.to(DEV), perm_t, cfg.bits, cfg.group_size, cfg.sym,
                                      cfg.block)
    torch.cuda.synchronize()
    rows = sorted(set([0, 1, 31, 32, out // 2, out - 1] +
                      np.random.default_rng(7).choice(out, 6, replace=False).tolist()))
    d = check_quantize_parity(W.cpu(), U32, perm_t, cfg.bits, cfg.group_size, cfg.sym, qw, sc,
                              zr, gi, rows=rows)
    print("  ", d)
