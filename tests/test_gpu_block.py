"""Layer-wise GPTQ over a Llama-style MLP block (gate, up, down) against
the oracle's mlp_block on the same fp16 block input and weights, and the
gated activation kernel against the oracle's silu_mul.

Stage by stage, each stage fed the HIP path's own output of the stage
before: H_in against the oracle's Hessian of the block input (relative
Frobenius 1e-3); gate and up against the oracle sweep in replay mode with
the factor and column order the library used; H_down against the Hessian of
the activations the oracle's fp64 forward gives through the HIP path's
quantized gate and up (1e-3: the HIP forward holds the dequantized weights
and the activations in fp16, about 5e-4 apart); the column order of H_down
exactly; down against the oracle sweep in replay mode with its factor.

End to end, both chains free-running: each layer's calibration error within
2 % of the oracle's (measured with the oracle's Hessian of that layer's
inputs) and below round-to-nearest; code agreement reported.
"""
import numpy as np
import pytest
import torch

import oracle as O
import post_weight_quantization_12_amd as P
import workloads
from helpers import check_quantize_parity, gpu_codes, rel_fro, upper_mirror

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _banner(msg):
    print(f"[case] {msg}", flush=True)


def _silu_tol(a):
    # fp32 evaluation then one rounding to fp16: half an fp16 ulp plus the
    # fp32 error, and half the fp16 subnormal spacing near zero
    return (2.0 ** -11 + 2.0 ** -20) * np.abs(a) + 2.0 ** -25


@pytest.mark.parametrize("rows,cols", [(3, 8), (5, 1000), (64, 2051), (1, 7)])
def test_silu_mul_matches_oracle(rows, cols):
    _banner(f"silu_mul {rows}x{cols}")
    g = torch.Generator().manual_seed(rows * 131 + cols)
    GU = (torch.randn((rows, 2 * cols), generator=g) * 4).to(torch.float16)
    if cols >= 4:   # zero, saturating both ways, a subnormal
        GU[0, :4] = torch.tensor([0.0, 11.0, -11.0, 6e-5], dtype=torch.float16)
    d = GU.to(DEV)
    A = P.silu_mul(d[:, :cols], d[:, cols:])         # halves of one matrix (ld = 2 cols)
    want = O.silu_mul(GU[:, :cols].double().numpy(), GU[:, cols:].double().numpy())
    torch.cuda.synchronize()
    err = np.abs(A.cpu().double().numpy() - want)
    assert np.all(err <= _silu_tol(want)), f"max err {err.max()}"
    # in place over G
    P.silu_mul(d[:, :cols], d[:, cols:], A=d[:, :cols])
    torch.cuda.synchronize()
    assert torch.equal(d[:, :cols].cpu(), A.cpu())


@pytest.mark.parametrize("d,inter,bits,gs,sym,desc", [
    (256, 704, 4, 64, False, True),
    (256, 704, 3, 128, False, False),
    (128, 352, 8, 32, True, True),
])
def test_mlp_block_matches_oracle(d, inter, bits, gs, sym, desc):
    _banner(f"mlp block d={d} inter={inter} {bits}b g{gs} sym={sym} desc={desc}")
    base = workloads.get("c1").shrink(inp=d, n_outliers=4, tokens_per_sample=2048)
    X = workloads.x_tokens(base, 0, 2)                      # 4096 tokens, two chunks below
    Wg, Wu, Wd = workloads.mlp_block_weights(d, inter)
    r = P.block.quantize_mlp_block(X.to(DEV), Wg.to(DEV), Wu.to(DEV), Wd.to(DEV), bits, gs,
                                   sym, 0.01, desc, chunk_tokens=2048, keep_factors=True)
    ref = O.mlp_block(X.numpy(), Wg.float().numpy(), Wu.float().numpy(), Wd.float().numpy(),
                      bits, gs, sym, 0.01, desc)
    h_in = rel_fro(upper_mirror(r.H_in.cpu().double().numpy()), ref.H_in)
    h_dn = rel_fro(upper_mirror(r.H_down.cpu().double().numpy()), ref.H_down)
    # H_down free-running (each side's own gate and up) is reported; the
    # stage check below is the gate
    print(f"  H_in rel {h_in:.2e}  H_down rel {h_dn:.2e} (free-running)")
    assert h_in <= 1e-3
    # ---- stage by stage, each fed the HIP path's previous output ----
    for name, lay, W in (("gate", r.gate, Wg), ("up", r.up, Wu)):
        dd = check_quantize_parity(W, r.U_in.cpu(), r.perm_in, bits, gs, sym, lay.qweight,
                                   lay.scales, lay.zeros, lay.g_idx)
        print(f"  stage {name}: {dd}")
    Xn = X.double().numpy()

    def deq(lay, n):
        return O.dequantize(gpu_codes(lay.qweight, bits, n), lay.scales.cpu().numpy(),
                            lay.zeros.cpu().numpy(), lay.g_idx.cpu().numpy())

    A = O.silu_mul(Xn @ deq(r.gate, d).T, Xn @ deq(r.up, d).T)
    Hg_down = upper_mirror(r.H_down.cpu().double().numpy())
    h_st = rel_fro(Hg_down, O.hessian(A))
    print(f"  stage H_down rel {h_st:.2e}")
    assert h_st <= 1e-3
    assert np.array_equal(r.perm_down.cpu().numpy(), O.column_order(Hg_down, desc))
    dd = check_quantize_parity(Wd, r.U_down.cpu(), r.perm_down, bits, gs, sym, r.down.qweight,
                               r.down.scales, r.down.zeros, r.down.g_idx)
    print(f"  stage down: {dd}")
    for name, lay, W, H, orc in (("gate", r.gate, Wg, ref.H_in, ref.gate),
                                 ("up", r.up, Wu, ref.H_in, ref.up),
                                 ("down", r.down, Wd, ref.H_down, ref.down)):
        n = W.shape[1]
        Wd64 = W.double().numpy()
        codes = gpu_codes(lay.qweight, bits, n)
        Wq = O.dequantize(codes, lay.scales.cpu().numpy(), lay.zeros.cpu().numpy(),
                          lay.g_idx.cpu().numpy())
        e_gpu = O.layer_error(Wd64, Wq, H)
        e_ref = O.layer_error(Wd64, orc.what, H)
        e_rtn = O.layer_error(Wd64, O.rtn(Wd64, bits, gs, sym).what, H)
        agree = float(np.mean(codes == orc.codes))
        print(f"  {name}: E_gpu {e_gpu:.6g}  E_oracle {e_ref:.6g}  E_rtn {e_rtn:.6g}  "
              f"agreement {agree:.5f}")
        assert abs(e_gpu / e_ref - 1.0) <= 0.02
        assert e_gpu < e_rtn
        # free-running code agreement is reported only: a value on a rounding
        # boundary (decided in fp32 here and in fp64 by the oracle) moves the
        # rest of its row; the stage checks above compare code by code
        if not desc:   # with desc_act near-equal diagonal entries may order either way
            assert np.array_equal(lay.g_idx.cpu().numpy(), orc.g_idx)


# ------------------------------------------------------ attention half --
def _attn_tol(Qn, Kn, Vn, seq_len, heads, causal, ref):
    """Per-entry bound: the softmax weights enter the value product as fp16
    (2^-11 relative each) while their sum stays fp32, O is rounded once to
    fp16 (2^-11), fp32 scores and sums add ~2^-16 relative; measured on
    sum_s p_s |v_s| (the oracle's weights on |V|)."""
    absum = O.attention(Qn, Kn, np.abs(Vn), seq_len, heads, causal)
    return (2.0 ** -11 + 2.0 ** -16) * absum + 2.0 ** -11 * np.abs(ref) + 1e-7


ATT = [(2, 256, 2, 128, True), (3, 100, 4, 64, True), (1, 1, 2, 64, True),
       (2, 130, 1, 128, False), (1, 577, 2, 128, True)]


@pytest.mark.parametrize("seqs,seq_len,heads,hd,causal", ATT,
                         ids=[f"{a}x{b}-h{c}-d{d_}-{'causal' if e else 'full'}" for a, b, c, d_, e in ATT])
def test_attention_matches_oracle(seqs, seq_len, heads, hd, causal):
    _banner(f"attention seqs={seqs} len={seq_len} heads={heads} hd={hd} causal={causal}")
    g = torch.Generator().manual_seed(seqs * 1000 + seq_len + hd)
    w = heads * hd
    # Q, K, V as the three parts of one [tokens x 3w] matrix (the driver's layout)
    QKV = (torch.randn((seqs * seq_len, 3 * w), generator=g) * 1.5).to(torch.float16)
    d_ = QKV.to(DEV)
    Og = P.attention_forward(d_[:, :w], d_[:, w:2 * w], d_[:, 2 * w:], seq_len, heads, causal)
    torch.cuda.synchronize()
    Qn, Kn, Vn = (QKV[:, i * w:(i + 1) * w].double().numpy() for i in range(3))
    ref = O.attention(Qn, Kn, Vn, seq_len, heads, causal)
    err = np.abs(Og.cpu().double().numpy() - ref)
    tol = _attn_tol(Qn, Kn, Vn, seq_len, heads, causal, ref)
    print(f"  max |dO| {err.max():.3e}, worst err/tol {float(np.max(err / tol)):.3f}")
    assert np.all(err <= tol)


def test_residual_rmsnorm_matches_oracle():
    _banner("residual rmsnorm")
    g = torch.Generator().manual_seed(5)
    rows, d = 37, 4096 + 40
    X = (torch.randn((rows, d), generator=g) * 2).to(torch.float16)
    A = (torch.randn((rows, d), generator=g) * 0.5).to(torch.float16)
    gm = (1.0 + 0.05 * torch.randn((d,), generator=g)).to(torch.float16)
    X[0] = 0.0
    A[0] = 0.0   # an all-zero row: U = 0 (eps keeps the norm finite)
    Hs, U = P.residual_rmsnorm(X.to(DEV), A.to(DEV), gm.to(DEV), 1e-5)
    torch.cuda.synchronize()
    Hr, Ur = O.residual_rmsnorm(X.double().numpy(), A.double().numpy(), gm.double().numpy(), 1e-5)
    # Hs: one rounding of the exact sum to fp16; U: that rounding, the fp32
    # norm and one more rounding
    assert np.all(np.abs(Hs.cpu().double().numpy() - Hr) <= 2.0 ** -11 * np.abs(Hr) + 2.0 ** -25)
    eu = np.abs(U.cpu().double().numpy() - Ur)
    assert np.all(eu <= (2.0 ** -10 + 2.0 ** -16) * np.abs(Ur) + 2.0 ** -24)
    assert bool((U[0] == 0).all())


DEC = [(256, 512, 2, 128, 4, 64, False, True), (256, 512, 4, 128, 3, 128, False, False),
       (128, 352, 2, 64, 8, 32, True, True)]


@pytest.mark.parametrize("d,inter,heads,seq_len,bits,gs,sym,desc", DEC,
                         ids=[f"d{c[0]}-h{c[2]}-{c[4]}b-g{c[5]}" for c in DEC])
def test_decoder_block_matches_oracle(d, inter, heads, seq_len, bits, gs, sym, desc):
    """A whole decoder block: every stage against the oracle fed the HIP
    path's own previous output (Hessians to 1e-3 relative Frobenius, column
    orders exactly, each layer's codes in replay mode), and each layer's
    calibration error, both chains free-running, within 2 % of the oracle's."""
    _banner(f"decoder block d={d} inter={inter} heads={heads} len={seq_len} {bits}b g{gs} "
            f"sym={sym} desc={desc}")
    seqs, eps = 8, 1e-5
    base = workloads.get("c1").shrink(inp=d, n_outliers=4, tokens_per_sample=seq_len)
    X = workloads.x_tokens(base, 0, seqs)
    Wq, Wk, Wv, Wo, gm, Wg, Wu, Wd = workloads.decoder_block_weights(d, inter)
    dev = [t.to(DEV) for t in (X, Wq, Wk, Wv, Wo, gm, Wg, Wu, Wd)]
    r = P.block.quantize_decoder_block(*dev, heads, seq_len, eps, bits, gs, sym, 0.01, desc,
                                       chunk_seqs=3, keep=True)
    Xn = X.double().numpy()

    def deq(lay, n):
        return O.dequantize(gpu_codes(lay.qweight, bits, n), lay.scales.cpu().numpy(),
                            lay.zeros.cpu().numpy(), lay.g_idx.cpu().numpy())

    def h_stage(Hg, want, name):
        rel = rel_fro(upper_mirror(Hg.cpu().double().numpy()), want)
        print(f"  stage {name} rel {rel:.2e}")
        assert rel <= 1e-3

    # q, k, v from the block input's Hessian
    h_stage(r.H_x, O.hessian(Xn), "H_x")
    for name, lay, W in (("q", r.q, Wq), ("k", r.k, Wk), ("v", r.v, Wv)):
        print(f"  stage {name}: "
              f"{check_quantize_parity(W, r.U_x.cpu(), r.perm_x, bits, gs, sym, *_packed(lay))}")
    # o from the attention of the HIP path's quantized q, k, v
    Oref = O.attention(Xn @ deq(r.q, d).T, Xn @ deq(r.k, d).T, Xn @ deq(r.v, d).T, seq_len,
                       heads)
    Og = r.O.cpu().double().numpy()
    print(f"  stage attention output rel {rel_fro(Og, Oref):.2e}")
    h_stage(r.H_o, O.hessian(Oref), "H_o")
    Hg_o = upper_mirror(r.H_o.cpu().double().numpy())
    assert np.array_equal(r.perm_o.cpu().numpy(), O.column_order(Hg_o, desc))
    print(f"  stage o: {check_quantize_parity(Wo, r.U_o.cpu(), r.perm_o, bits, gs, sym, *_packed(r.o))}")
    # the MLP from the normalized residual stream after the quantized o,
    # fed the HIP path's attention output
    _, Uref = O.residual_rmsnorm(Xn, Og @ deq(r.o, d).T, gm.double().numpy(), eps)
    h_stage(r.mlp.H_in, O.hessian(Uref), "H_mlp")
    Un = r.U.cpu().double().numpy()
    for name, lay, W in (("gate", r.mlp.gate, Wg), ("up", r.mlp.up, Wu)):
        print(f"  stage {name}: "
              f"{check_quantize_parity(W, r.mlp.U_in.cpu(), r.mlp.perm_in, bits, gs, sym, *_packed(lay))}")
    A = O.silu_mul(Un @ deq(r.mlp.gate, d).T, Un @ deq(r.mlp.up, d).T)
    h_stage(r.mlp.H_down, O.hessian(A), "H_down")
    print(f"  stage down: "
          f"{check_quantize_parity(Wd, r.mlp.U_down.cpu(), r.mlp.perm_down, bits, gs, sym, *_packed(r.mlp.down))}")
    # end to end, both chains free-running
    ref = O.decoder_block(Xn, *(t.double().numpy() for t in (Wq, Wk, Wv, Wo, gm, Wg, Wu, Wd)),
                          heads, seq_len, eps, bits, gs, sym, 0.01, desc)
    for name, lay, W, H, orc in (("q", r.q, Wq, ref.H_x, ref.q), ("k", r.k, Wk, ref.H_x, ref.k),
                                 ("v", r.v, Wv, ref.H_x, ref.v), ("o", r.o, Wo, ref.H_o, ref.o),
                                 ("gate", r.mlp.gate, Wg, ref.mlp.H_in, ref.mlp.gate),
                                 ("up", r.mlp.up, Wu, ref.mlp.H_in, ref.mlp.up),
                                 ("down", r.mlp.down, Wd, ref.mlp.H_down, ref.mlp.down)):
        W64 = W.double().numpy()
        e_gpu = O.layer_error(W64, deq(lay, W.shape[1]), H)
        e_ref = O.layer_error(W64, orc.what, H)
        print(f"  {name}: E_gpu {e_gpu:.6g}  E_oracle {e_ref:.6g}  ratio {e_gpu / e_ref:.5f}")
        assert abs(e_gpu / e_ref - 1.0) <= 0.02


def _packed(lay):
    return lay.qweight, lay.scales, lay.zeros, lay.g_idx
