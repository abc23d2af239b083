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
