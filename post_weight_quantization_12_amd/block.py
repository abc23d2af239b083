"""Layer-wise GPTQ over a Llama-style MLP block: y = Wd (SiLU(Wg x) * (Wu x)).

The glossary entry "gptq" (paragraph "Method") quantizes one layer at a
time from calibration activations.  Here the gate and up projections share
the block input, so one Hessian serves both; the down projection's
calibration inputs are then computed through the block with the gate and up
layers already quantized (dequantize-on-the-fly products), and its Hessian
comes from them.  Every step runs in the HIP library; this module only
sequences the calls and holds the buffers.
"""
from __future__ import annotations

from dataclasses import dataclass

from . import _lib as L


@dataclass
class PackedLayer:
    qweight: object   # int32 [in * bits / 32 x out]
    scales: object    # fp32 [n_groups x out]
    zeros: object     # int32 [n_groups x out]
    g_idx: object     # int32 [in]


@dataclass
class BlockResult:
    gate: PackedLayer
    up: PackedLayer
    down: PackedLayer
    H_in: object      # fp32 [d x d], upper triangle
    H_down: object    # fp32 [inter x inter], upper triangle


def quantize_mlp_block(X, Wg, Wu, Wd, bits: int, group_size: int, sym: bool, damp: float,
                       desc_act: bool, block: int = 128, chunk_tokens: int = 32768,
                       stream=None, mark=None) -> BlockResult:
    """X fp16 [tokens x d] (the block input), Wg / Wu [inter x d], Wd
    [d x inter] (fp16 or fp32).  The calibration tokens go through the block
    in chunks of chunk_tokens (the activations of one chunk live at a time).
    mark: optional callable, called with a phase name at each phase boundary
    (e.g. to record timing events on the stream).  stream: the stream of the
    library calls; the buffers this function allocates, clears and joins
    with torch are ordered on torch's current stream, so pass that stream
    (None: the current stream's handle is taken)."""
    torch = L._torch()
    mark = mark or (lambda name: None)
    if stream is None:
        stream = torch.cuda.current_stream(X.device)
    dev = X.device
    ntok, d = X.shape
    inter = Wg.shape[0]
    if tuple(Wu.shape) != (inter, d) or tuple(Wd.shape) != (d, inter):
        raise ValueError("Wg, Wu must be [inter x d] and Wd [d x inter]")
    chunks = [X[i:i + chunk_tokens] for i in range(0, ntok, chunk_tokens)]

    # gate and up: the block input's Hessian (X is resident: one call)
    H_in = torch.zeros((d, d), dtype=torch.float32, device=dev)
    ws = torch.empty((L.hessian_workspace_bytes(d),), dtype=torch.uint8, device=dev)
    mark("start")
    L.hessian_accumulate(H_in, X, stream, ws)
    mark("hessian_in")
    U_in, perm_in, info_in = L.prepare(H_in, damp, desc_act, stream=stream)
    mark("prepare_in")
    gate = PackedLayer(*L.quantize_layer(Wg, U_in, perm_in, bits, group_size, sym, block,
                                         stream=stream))
    up = PackedLayer(*L.quantize_layer(Wu, U_in, perm_in, bits, group_size, sym, block,
                                       stream=stream))
    del U_in
    mark("quantize_gate_up")

    # the down projection's inputs, through the quantized gate and up layers
    gu = [gate, up]
    order = None
    if desc_act:
        # both layers share perm_in, hence g_idx: one group order serves both
        ordered = []
        for lay in gu:
            qs, gs, order = L.dequant_group_order(lay.qweight, lay.g_idx, bits, stream=stream)
            ordered.append(PackedLayer(qs, lay.scales, lay.zeros, gs))
        gu = ordered
    # gate and up as one layer of 2 inter outputs (same inputs and groups)
    qw2 = torch.cat([gu[0].qweight, gu[1].qweight], dim=1).contiguous()
    sc2 = torch.cat([gu[0].scales, gu[1].scales], dim=1).contiguous()
    zr2 = torch.cat([gu[0].zeros, gu[1].zeros], dim=1).contiguous()
    g2 = gu[0].g_idx
    mark("group_order")
    H_down = torch.zeros((inter, inter), dtype=torch.float32, device=dev)
    ws_d = torch.empty((L.hessian_workspace_bytes(inter),), dtype=torch.uint8, device=dev)
    GU = torch.empty((min(chunk_tokens, ntok), 2 * inter), dtype=torch.float16, device=dev)
    A = torch.empty((min(chunk_tokens, ntok), inter), dtype=torch.float16, device=dev)
    wsm = None
    for c in chunks:
        m = c.shape[0]
        need = L.dequant_matmul_workspace_bytes(m, d, 2 * inter, order is not None)
        if need and (wsm is None or wsm.numel() < need):
            wsm = torch.empty((need,), dtype=torch.uint8, device=dev)
        L.dequant_matmul(c, qw2, sc2, zr2, g2, bits, x_order=order, Y=GU[:m],
                         workspace=wsm if need else None, stream=stream)
        L.silu_mul(GU[:m, :inter], GU[:m, inter:], A=A[:m], stream=stream)
        L.hessian_accumulate(H_down, A[:m], stream, ws_d)
    mark("forward_hessian_down")
    del GU, A, qw2, sc2, zr2
    U_d, perm_d, info_d = L.prepare(H_down, damp, desc_act, stream=stream)
    mark("prepare_down")
    down = PackedLayer(*L.quantize_layer(Wd, U_d, perm_d, bits, group_size, sym, block,
                                         stream=stream))
    mark("quantize_down")
    torch.cuda.synchronize(dev)
    if int(info_in.item()) != 0 or int(info_d.item()) != 0:
        raise RuntimeError("gptq_prepare: a block Hessian is not positive definite after "
                           f"damping (info {int(info_in.item())}, {int(info_d.item())})")
    return BlockResult(gate=gate, up=up, down=down, H_in=H_in, H_down=H_down)
