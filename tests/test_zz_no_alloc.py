"""gptq_dequant_matmul_noalloc (the library's fixed per-device scratch, no
workspace, no allocation) against gptq_dequant_matmul with a workspace.

Both run the same kernels on the same split plan, so the products must agree
bit for bit.  Calls come two in a row, the second smaller, so the second runs
on scratch the first has already written (nothing in it may leak into the
result).  A product whose scratch would not fit is refused on the host.
"""
import pytest
import torch

import post_weight_quantization_12_amd as P
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _banner(msg):
    print(f"[case] {msg}", flush=True)


def _layer(cname, act_order):
    """A random packed layer of the config's shape and bits; with act_order
    its group-sorted copy and x_order (as dequant_group_order makes them)."""
    cfg = workloads.get(cname)
    words, scales, zeros, order = workloads.packed_layer_draws(cfg, DEV)
    g_idx = torch.empty(cfg.inp, dtype=torch.int32, device=DEV)
    g_idx[order] = (torch.arange(cfg.inp, device=DEV) // cfg.group_size).to(torch.int32)
    words, scales, zeros = words.contiguous(), scales.float().contiguous(), zeros.contiguous()
    x_order = None
    if act_order:
        words, g_idx, x_order = P.dequant_group_order(words, g_idx, cfg.bits)
    return cfg, words, scales, zeros, g_idx, x_order


def _x(M, inp, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randn((M, inp), generator=g, device=DEV).to(torch.float16)


def _both(cname, M, ydt, act_order, seed):
    cfg, qw, sc, zr, gi, xo = _layer(cname, act_order)
    X = _x(M, cfg.inp, seed)
    ref = P.dequant_matmul(X, qw, sc, zr, gi, cfg.bits, x_order=xo, out_dtype=ydt)
    Y = torch.full((M, cfg.out), float("nan"), dtype=ydt, device=DEV)
    P.dequant_matmul_noalloc(X, qw, sc, zr, gi, cfg.bits, Y, x_order=xo)
    torch.cuda.synchronize()
    return ref, Y


SEQS = [
    # (config, tokens, Y dtype, act order) twice, the second call smaller
    [("c4a", 8, torch.float32, False), ("c1", 1, torch.float16, False)],
    [("c2", 16, torch.float32, True), ("c3", 3, torch.float16, True)],
]


@pytest.mark.parametrize("seq", SEQS, ids=["decode", "act_order_prefill"])
def test_noalloc_matches_workspace_entry(seq):
    for i, (cname, M, ydt, act) in enumerate(seq):
        cfg = workloads.get(cname)
        need = P.dequant_matmul_workspace_bytes(M, cfg.inp, cfg.out, act)
        _banner(f"noalloc {cname} {cfg.out}x{cfg.inp} {cfg.bits}b M={M} act_order={act} "
                f"scratch={need}")
        assert need <= 16 << 20
        ref, Y = _both(cname, M, ydt, act, seed=100 + i)
        assert torch.equal(Y, ref), f"call {i}: max diff {(Y.float() - ref.float()).abs().max()}"


def test_noalloc_refuses_oversized_scratch():
    _banner("noalloc oversized")
    cfg, qw, sc, zr, gi, xo = _layer("c3", True)
    M = 2048
    assert P.dequant_matmul_workspace_bytes(M, cfg.inp, cfg.out, True) > 16 << 20
    X = _x(M, cfg.inp, 7)
    Y = torch.zeros((M, cfg.out), dtype=torch.float32, device=DEV)
    with pytest.raises(P.GptqError) as e:
        P.dequant_matmul_noalloc(X, qw, sc, zr, gi, cfg.bits, Y, x_order=xo)
    assert e.value.status == 3  # GPTQ_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((Y == 0).all())
