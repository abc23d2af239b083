"""Layer-wise GPTQ over Llama-style blocks.

The glossary entry "gptq" (paragraph "Method") quantizes one layer at a
time from calibration activations computed through the model with the
layers before it already quantized.

quantize_mlp_block: y = Wd (SiLU(Wg x) * (Wu x)).  The gate and up
projections share the block input, so one Hessian serves both; the down
projection's calibration inputs are then computed through the block with
the gate and up layers already quantized (dequantize-on-the-fly products),
and its Hessian comes from them.

quantize_decoder_block: a whole decoder block.  q, k and v share the block
input's Hessian; the output projection is calibrated on the attention of
the quantized q, k, v; the MLP on the normalized residual stream
X + O W^o^T after the quantized output projection.

Every step runs in the HIP library; this module only sequences the calls
and holds the buffers.
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
    # the factors and column orders the layers were quantized with
    # (keep_factors=True only; None otherwise)
    U_in: object = None
    perm_in: object = None
    U_down: object = None
    perm_down: object = None


def quantize_mlp_block(X, Wg, Wu, Wd, bits: int, group_size: int, sym: bool, damp: float,
                       desc_act: bool, block: int = 128, chunk_tokens: int = 32768,
                       stream=None, mark=None, keep_factors: bool = False) -> BlockResult:
    """X fp16 [tokens x d] (the block input), Wg / Wu [inter x d], Wd
    [d x inter] (fp16 or fp32).  The calibration tokens go through the block
    in chunks of chunk_tokens (the activations of one chunk live at a time).
    mark: optional callable, called with a phase name at each phase boundary
    (e.g. to record timing events on the stream).  stream: the stream of the
    library calls; the buffers this function allocates, clears and joins
    with torch are ordered on torch's current stream, so pass that stream
    (None: the current stream's handle is taken).  keep_factors: also return
    the factors and column orders of the two Hessians (for stage checks)."""
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
    if not keep_factors:
        U_in = None
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
    kept = (U_in, perm_in, U_d, perm_d) if keep_factors else (None,) * 4
    return BlockResult(gate=gate, up=up, down=down, H_in=H_in, H_down=H_down, U_in=kept[0],
                       perm_in=kept[1], U_down=kept[2], perm_down=kept[3])


@dataclass
class DecoderBlockResult:
    q: PackedLayer
    k: PackedLayer
    v: PackedLayer
    o: PackedLayer
    mlp: BlockResult  # gate, up, down; its H_in is the MLP input's Hessian
    H_x: object       # fp32 [d x d], upper triangle: the block input's Hessian
    H_o: object       # fp32 [d x d], upper triangle: the attention output's Hessian
    # kept with keep=True only (None otherwise): the stage inputs
    O: object = None       # fp16 [tokens x d], attention output (o_proj's inputs)
    U: object = None       # fp16 [tokens x d], normalized residual stream (the MLP's inputs)
    U_x: object = None
    perm_x: object = None
    U_o: object = None
    perm_o: object = None


def _joined(layers, bits, desc_act, stream):
    """Layers sharing one input and one column order as one packed layer
    (outputs side by side); with desc_act, in group order (one order serves
    all: they share g_idx).  Returns (qweight, scales, zeros, g_idx, x_order)."""
    torch = L._torch()
    order = None
    if desc_act:
        ordered = []
        for lay in layers:
            qs, gs, order = L.dequant_group_order(lay.qweight, lay.g_idx, bits, stream=stream)
            ordered.append(PackedLayer(qs, lay.scales, lay.zeros, gs))
        layers = ordered
    return (torch.cat([l.qweight for l in layers], dim=1).contiguous(),
            torch.cat([l.scales for l in layers], dim=1).contiguous(),
            torch.cat([l.zeros for l in layers], dim=1).contiguous(),
            layers[0].g_idx, order)


def quantize_decoder_block(X, Wq, Wk, Wv, Wo, gamma, Wg, Wu, Wd, heads: int, seq_len: int,
                           eps: float, bits: int, group_size: int, sym: bool, damp: float,
                           desc_act: bool, block: int = 128, chunk_seqs: int = 16,
                           stream=None, mark=None, keep: bool = False) -> DecoderBlockResult:
    """X fp16 [seqs * seq_len x d] (the block input, sequences contiguous);
    Wq, Wk, Wv, Wo [d x d], gamma fp16 [d], Wg, Wu [inter x d], Wd [d x inter].
    The calibration sequences go through the attention chunk_seqs at a
    time; the attention output and the MLP input stay resident (2 x tokens
    x d fp16).  mark / stream as in quantize_mlp_block; keep: also return
    the stage inputs (attention output, MLP input, factors and orders)."""
    torch = L._torch()
    mark = mark or (lambda name: None)
    if stream is None:
        stream = torch.cuda.current_stream(X.device)
    dev = X.device
    ntok, d = X.shape
    if ntok % seq_len:
        raise ValueError("the tokens must be whole sequences of seq_len")
    for name, W in (("Wq", Wq), ("Wk", Wk), ("Wv", Wv), ("Wo", Wo)):
        if tuple(W.shape) != (d, d):
            raise ValueError(f"{name} must be [d x d]")
    chunk = chunk_seqs * seq_len

    # q, k, v: the block input's Hessian
    H_x = torch.zeros((d, d), dtype=torch.float32, device=dev)
    ws = torch.empty((L.hessian_workspace_bytes(d),), dtype=torch.uint8, device=dev)
    mark("start")
    L.hessian_accumulate(H_x, X, stream, ws)
    mark("hessian_x")
    U_x, perm_x, info_x = L.prepare(H_x, damp, desc_act, stream=stream)
    mark("prepare_x")
    qkv = [PackedLayer(*L.quantize_layer(W, U_x, perm_x, bits, group_size, sym, block,
                                         stream=stream)) for W in (Wq, Wk, Wv)]
    mark("quantize_qkv")

    # the output projection's inputs: attention of the quantized q, k, v
    qw3, sc3, zr3, g3, order = _joined(qkv, bits, desc_act, stream)
    O = torch.empty((ntok, d), dtype=torch.float16, device=dev)
    QKV = torch.empty((min(chunk, ntok), 3 * d), dtype=torch.float16, device=dev)
    wsm = None
    for c0 in range(0, ntok, chunk):
        m = min(chunk, ntok - c0)
        need = L.dequant_matmul_workspace_bytes(m, d, 3 * d, order is not None)
        if need and (wsm is None or wsm.numel() < need):
            wsm = torch.empty((need,), dtype=torch.uint8, device=dev)
        L.dequant_matmul(X[c0:c0 + m], qw3, sc3, zr3, g3, bits, x_order=order, Y=QKV[:m],
                         workspace=wsm if need else None, stream=stream)
        L.attention_forward(QKV[:m, :d], QKV[:m, d:2 * d], QKV[:m, 2 * d:], seq_len, heads,
                            True, O=O[c0:c0 + m], stream=stream)
    del QKV, qw3, sc3, zr3
    mark("forward_attention")
    H_o = torch.zeros((d, d), dtype=torch.float32, device=dev)
    L.hessian_accumulate(H_o, O, stream, ws)
    mark("hessian_o")
    U_o, perm_o, info_o = L.prepare(H_o, damp, desc_act, stream=stream)
    mark("prepare_o")
    o = PackedLayer(*L.quantize_layer(Wo, U_o, perm_o, bits, group_size, sym, block,
                                      stream=stream))
    mark("quantize_o")

    # the MLP's inputs: the normalized residual stream after the quantized o
    qwo, sco, zro, go, order_o = _joined([o], bits, desc_act, stream)
    U = torch.empty((ntok, d), dtype=torch.float16, device=dev)
    AO = torch.empty((min(chunk, ntok), d), dtype=torch.float16, device=dev)
    Hs = torch.empty_like(AO)
    for c0 in range(0, ntok, chunk):
        m = min(chunk, ntok - c0)
        need = L.dequant_matmul_workspace_bytes(m, d, d, order_o is not None)
        if need and (wsm is None or wsm.numel() < need):
            wsm = torch.empty((need,), dtype=torch.uint8, device=dev)
        L.dequant_matmul(O[c0:c0 + m], qwo, sco, zro, go, bits, x_order=order_o, Y=AO[:m],
                         workspace=wsm if need else None, stream=stream)
        L.residual_rmsnorm(X[c0:c0 + m], AO[:m], gamma, eps, Hs=Hs[:m], U=U[c0:c0 + m],
                           stream=stream)
    del AO, Hs, wsm
    mark("forward_norm")
    mlp = quantize_mlp_block(U, Wg, Wu, Wd, bits, group_size, sym, damp, desc_act, block,
                             chunk, stream, mark, keep_factors=keep)
    torch.cuda.synchronize(dev)
    if int(info_x.item()) != 0 or int(info_o.item()) != 0:
        raise RuntimeError("gptq_prepare: a block Hessian is not positive definite after "
                           f"damping (info {int(info_x.item())}, {int(info_o.item())})")
    kept = (O, U, U_x, perm_x, U_o, perm_o) if keep else (None,) * 6
    return DecoderBlockResult(q=qkv[0], k=qkv[1], v=qkv[2], o=o, mlp=mlp, H_x=H_x, H_o=H_o,
                              O=kept[0], U=kept[1], U_x=kept[2], perm_x=kept[3], U_o=kept[4],
                              perm_o=kept[5])
