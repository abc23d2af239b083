"""Seeded synthetic inputs for GPTQ layer quantization (shared by tests and bench).

This module only draws random inputs; it holds none of the quantization
method's arithmetic.  Both the oracle side and the GPU side of a test receive
the very same bytes from here.

Every draw comes from its own torch generator seeded from
(seed, config id, stream, index) through numpy's SeedSequence, so any sample
can be produced on its own, on any device, in any order.  Values for one
device are reproducible; the CPU and GPU generators give different streams,
so a test draws once, on one device, and hands the same tensor to both sides.

Streams: 0 = W, 1 = mixing matrix / shared basis, 2 = outlier channel set,
3 = calibration tokens (index = sample), 4 = special test inputs.

The workloads are shaped like the layers the pages quantize (Llama-2-7B
q_proj 4096x4096 and down_proj 4096x11008, Llama-70B down_proj 8192x28672,
calibrated on 128 samples x 2048 tokens); the c4 calibration text and the
model weights are not used: these synthetic draws stand in for them.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np
import torch

__all__ = ["Config", "CONFIGS", "get", "weight", "x_sample", "x_tokens",
           "outlier_channels", "boundary_safe_weight", "synthetic_hinv_chol",
           "generator", "packed_layer_draws", "mlp_block_weights", "decoder_block_weights"]


@dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int
    out: int                # output channels (rows of W)
    inp: int                # input features (columns of W, size of H)
    w_dtype: torch.dtype
    w_std: float
    x_kind: str             # "mix" | "lowrank" | "gated"
    samples: int            # calibration samples
    tokens_per_sample: int
    n_outliers: int
    outlier_scale: float
    bits: int
    group_size: int
    sym: bool
    desc_act: bool
    damp: float
    block: int

    @property
    def tokens(self) -> int:
        return self.samples * self.tokens_per_sample

    def shrink(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = {
    # Tiny single layer: 64x128 fp32 W, X = Z.L (512 tokens, correlated).
    "c0": Config("c0", 0, 64, 128, torch.float32, 0.05, "mix", 1, 512, 0, 1.0,
                 4, 32, False, False, 0.01, 32),
    # Llama-7B q_proj shape, 4-bit asym g128.
    "c1": Config("c1", 1, 4096, 4096, torch.float16, 0.02, "lowrank", 128, 2048, 8, 20.0,
                 4, 128, False, False, 0.01, 128),
    # Same layer and X, 3-bit asym g128, desc_act.
    "c2": Config("c2", 1, 4096, 4096, torch.float16, 0.02, "lowrank", 128, 2048, 8, 20.0,
                 3, 128, False, True, 0.01, 128),
    # Llama-7B down_proj shape (in = 11008), heavy-tailed gated activations.
    "c3": Config("c3", 3, 4096, 11008, torch.float16, 0.015, "gated", 128, 2048, 16, 30.0,
                 4, 128, False, True, 0.01, 128),
    # Llama-70B down_proj shape (in = 28672): 4-bit sym g64 and 8-bit asym g128.
    "c4a": Config("c4a", 4, 8192, 28672, torch.float16, 0.01, "gated", 128, 2048, 32, 30.0,
                  4, 64, True, True, 0.01, 128),
    "c4b": Config("c4b", 4, 8192, 28672, torch.float16, 0.01, "gated", 128, 2048, 32, 30.0,
                  8, 128, False, True, 0.01, 128),
}


def get(name: str) -> Config:
    return CONFIGS[name]


def _seed(*key: int) -> int:
    return int(np.random.SeedSequence([int(k) for k in key]).generate_state(1, dtype=np.uint64)[0]
               & 0x7FFF_FFFF_FFFF_FFFF)


def generator(device, *key: int) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(_seed(*key))
    return g


def _randn(shape, device, *key):
    return torch.randn(shape, generator=generator(device, *key), device=device,
                       dtype=torch.float32)


def weight(cfg: Config, device="cpu", seed: int = 0) -> torch.Tensor:
    """W [out x in] ~ N(0, w_std^2), drawn in fp32, rounded to the config dtype."""
    w = _randn((cfg.out, cfg.inp), device, seed, cfg.cfg_id, 0, 0) * cfg.w_std
    return w.to(cfg.w_dtype)


def outlier_channels(cfg: Config, device="cpu", seed: int = 0) -> torch.Tensor:
    if cfg.n_outliers == 0:
        return torch.zeros(0, dtype=torch.long, device=device)
    g = generator("cpu", seed, cfg.cfg_id, 2, 0)
    return torch.randperm(cfg.inp, generator=g)[: cfg.n_outliers].sort().values.to(device)


def _mixing(cfg: Config, device, seed):
    if cfg.x_kind == "mix":
        # Lower-triangular mixing L: N(0,1) below the diagonal, 1 + |N(0,1)| on it.
        m = _randn((cfg.inp, cfg.inp), device, seed, cfg.cfg_id, 1, 0)
        low = torch.tril(m, -1)
        diag = 1.0 + torch.diagonal(m).abs()
        return low + torch.diag(diag)
    if cfg.x_kind == "lowrank":
        # Shared rank-64 basis A [in x 64] ~ N(0, 1/64): unit-variance shared part.
        return _randn((cfg.inp, 64), device, seed, cfg.cfg_id, 1, 0) / 8.0
    return None


def x_sample(cfg: Config, s: int, device="cpu", seed: int = 0, mixing=None,
             outliers=None, tokens: int | None = None) -> torch.Tensor:
    """Calibration sample s as fp16 [tokens_per_sample x in] (tokens x features)."""
    T = cfg.tokens_per_sample if tokens is None else tokens
    n = cfg.inp
    if cfg.x_kind == "mix":
        L = _mixing(cfg, device, seed) if mixing is None else mixing
        z = _randn((T, n), device, seed, cfg.cfg_id, 3, s)
        x = z @ L  # X = Z . L
    elif cfg.x_kind == "lowrank":
        A = _mixing(cfg, device, seed) if mixing is None else mixing
        gen = generator(device, seed, cfg.cfg_id, 3, s)
        z = torch.randn((T, n), generator=gen, device=device, dtype=torch.float32)
        gl = torch.randn((T, 64), generator=gen, device=device, dtype=torch.float32)
        idx = outlier_channels(cfg, device, seed) if outliers is None else outliers
        z[:, idx] *= cfg.outlier_scale
        x = z + gl @ A.T
    elif cfg.x_kind == "gated":
        gen = generator(device, seed, cfg.cfg_id, 3, s)
        a = torch.randn((T, n), generator=gen, device=device, dtype=torch.float32)
        b = torch.randn((T, n), generator=gen, device=device, dtype=torch.float32)
        x = a.abs_() * b
        idx = outlier_channels(cfg, device, seed) if outliers is None else outliers
        x[:, idx] *= cfg.outlier_scale
    else:
        raise ValueError(cfg.x_kind)
    return x.to(torch.float16)


def x_tokens(cfg: Config, s0: int, s1: int, device="cpu", seed: int = 0,
             tokens: int | None = None) -> torch.Tensor:
    """Samples [s0, s1) stacked: fp16 [(s1-s0)*T x in]."""
    mixing = _mixing(cfg, device, seed)
    outl = outlier_channels(cfg, device, seed)
    return torch.cat([x_sample(cfg, s, device, seed, mixing, outl, tokens)
                      for s in range(s0, s1)], dim=0)


def boundary_safe_weight(out: int, inp: int, bits: int, group_size: int, sym: bool,
                         device="cpu", seed: int = 0) -> torch.Tensor:
    """fp32 W whose every group-row has an exactly representable quantization grid.

    Per (row, group): a power-of-two scale s = 2^k (k in [-9, -5]).  Asymmetric:
    a zero z in [1, maxq-1], the values -z*s and (maxq-z)*s placed in the group
    so its range is exactly [-z*s, (maxq-z)*s], and the other entries
    s*(c + u) with integer c in [-z, maxq-z] and u a multiple of 2^-(10-bits)
    with |u| <= 0.4.  Symmetric: -(maxq/2)*s placed in the group, the others
    with |w| < (maxq/2)*s on the same grid.  All values are exact in fp16.
    """
    maxq = (1 << bits) - 1
    gs = inp if group_size == -1 else group_size
    g = generator("cpu", seed, 99, 4, bits * 1000 + gs)
    n_groups = -(-inp // gs)
    W = torch.zeros((out, inp), dtype=torch.float64)
    step = 2.0 ** -(10 - bits)
    umax = int(0.4 / step)
    for gi in range(n_groups):
        c0, c1 = gi * gs, min((gi + 1) * gs, inp)
        width = c1 - c0
        k = torch.randint(-9, -4, (out, 1), generator=g).to(torch.float64)
        s = torch.pow(2.0, k)
        u = torch.randint(-umax, umax + 1, (out, width), generator=g).to(torch.float64) * step
        if not sym:
            z = torch.randint(1, maxq, (out, 1), generator=g).to(torch.float64)
            c = torch.randint(0, maxq + 1, (out, width), generator=g).to(torch.float64) - z
            u = torch.where((c == -z) & (u < 0), -u, u)           # stay inside [lo, hi]
            u = torch.where((c == maxq - z) & (u > 0), -u, u)
            vals = s * (c + u)
            pos = torch.randperm(width, generator=g)[:2]
            vals[:, pos[0]] = (-z * s)[:, 0]
            vals[:, pos[1]] = ((maxq - z) * s)[:, 0]
        else:
            half = maxq / 2.0
            lim = int(np.floor(half - 0.5))
            c = torch.randint(-lim, lim + 1, (out, width), generator=g).to(torch.float64)
            vals = s * (c + u)
            pos = torch.randperm(width, generator=g)[:1]
            vals[:, pos[0]] = (-half * s)[:, 0]
        W[:, c0:c1] = vals
    return W.to(torch.float32).to(device)


def synthetic_hinv_chol(n: int, device="cpu", seed: int = 0, row_norm: float = 0.3) -> torch.Tensor:
    """A dense upper-triangular fp32 matrix with a positive diagonal.

    Any such matrix is the upper Cholesky factor of the inverse of some
    positive definite matrix, so it is a valid factor input for the sweep.
    Off-diagonal entries of row j, divided by the diagonal, have norm about
    ``row_norm`` (the size a real calibration Hessian gives).
    """
    gen = generator(device, seed, 98, 4, n)
    m = torch.randn((n, n), generator=gen, device=device, dtype=torch.float32)
    d = 0.5 + torch.rand((n,), generator=gen, device=device, dtype=torch.float32)
    rem = torch.arange(n - 1, -1, -1, device=device, dtype=torch.float32).clamp_min(1.0)
    sig = row_norm / torch.sqrt(rem)
    U = torch.triu(m, 1) * (sig * d)[:, None]
    U += torch.diag(d)
    return U.contiguous()


def packed_layer_draws(cfg: Config, device="cpu", seed: int = 0):
    """Random contents for a packed layer of cfg's shape and bit width.

    Returns (words, scales, zeros, order): words int32 [inp * bits / 32 x out]
    uniformly random (every b-bit field is a uniform code), scales fp32
    [G x out] uniform in [1e-3, 5e-2], zeros int32 [G x out] uniform in
    [0, 2^bits), G = number of groups of cfg.group_size along inp, and order a
    random permutation of the inp columns when cfg.desc_act (else the
    identity), the column order a desc_act layer's groups follow.
    """
    gs = cfg.inp if cfg.group_size == -1 else cfg.group_size
    G = -(-cfg.inp // gs)
    g = generator(device, seed, cfg.cfg_id, 5, cfg.bits * 1000 + gs)
    words = torch.randint(-2 ** 31, 2 ** 31 - 1, (cfg.inp * cfg.bits // 32, cfg.out),
                          generator=g, device=device, dtype=torch.int64).to(torch.int32)
    scales = 1e-3 + 4.9e-2 * torch.rand((G, cfg.out), generator=g, device=device)
    zeros = torch.randint(0, 2 ** cfg.bits, (G, cfg.out), generator=g, device=device,
                          dtype=torch.int32)
    if cfg.desc_act:
        order = torch.randperm(cfg.inp, generator=g, device=device)
    else:
        order = torch.arange(cfg.inp, device=device)
    return words, scales, zeros, order


def mlp_block_weights(d: int, inter: int, device="cpu", seed: int = 0):
    """(Wg, Wu [inter x d], Wd [d x inter]) fp16 for a Llama-style MLP block:
    N(0, 0.02^2) for the gate and up projections (as the q_proj-shaped
    layer), N(0, 0.015^2) for the down projection (as the down_proj-shaped
    layer); drawn in fp32, rounded to fp16."""
    wg = _randn((inter, d), device, seed, 20, 0, d) * 0.02
    wu = _randn((inter, d), device, seed, 21, 0, d) * 0.02
    wd = _randn((d, inter), device, seed, 22, 0, d) * 0.015
    return wg.to(torch.float16), wu.to(torch.float16), wd.to(torch.float16)


def decoder_block_weights(d: int, inter: int, device="cpu", seed: int = 0):
    """(Wq, Wk, Wv, Wo [d x d], gamma [d], Wg, Wu [inter x d], Wd [d x inter])
    fp16 for a Llama-style decoder block: the projections ~ N(0, 0.02^2)
    (N(0, 0.015^2) for the down projection, as the down_proj-shaped layer),
    the norm weight 1 + N(0, 0.05^2); drawn in fp32, rounded to fp16."""
    wq, wk, wv, wo = (_randn((d, d), device, seed, 23 + i, 0, d) * 0.02 for i in range(4))
    gamma = 1.0 + 0.05 * _randn((d,), device, seed, 27, 0, d)
    wg, wu, wd = mlp_block_weights(d, inter, device, seed)
    return tuple(t.to(torch.float16) for t in (wq, wk, wv, wo, gamma)) + (wg, wu, wd)
