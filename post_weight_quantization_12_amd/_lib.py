"""ctypes binding of libgptq_mi355x.so (argument marshalling only).

Every step of the quantization runs in the HIP library; this module checks
tensor devices / dtypes / shapes, passes raw device pointers plus the current
HIP stream, and turns status codes into exceptions.  torch provides device
memory and streams, nothing else.  There is no fallback: if the library is
missing, loading fails with an error that says how to build it.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgptq_mi355x.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "gptq.h")

GPTQ_OK, GPTQ_ERR_INVALID_ARG, GPTQ_ERR_UNSUPPORTED, GPTQ_ERR_WORKSPACE, GPTQ_ERR_HIP = range(5)
GPTQ_F16, GPTQ_BF16, GPTQ_F32 = 0, 1, 2
MAX_PREPARE_N = 32768


class GptqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None


def header_functions() -> list[str]:
    """Names of the functions declared in include/gptq.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(gptq_[a-z_0-9]+)\s*\(", text, flags=re.M)


def load():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m post_weight_quantization_12_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, c_int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.gptq_hessian_workspace_bytes.argtypes = [i64]
    lib.gptq_hessian_workspace_bytes.restype = ctypes.c_size_t
    lib.gptq_hessian_accumulate.argtypes = [vp, i64, vp, c_int, i64, i64, vp, ctypes.c_size_t, vp]
    lib.gptq_hessian_accumulate.restype = c_int
    lib.gptq_prepare_workspace_bytes.argtypes = [i64]
    lib.gptq_prepare_workspace_bytes.restype = ctypes.c_size_t
    lib.gptq_prepare.argtypes = [vp, i64, ctypes.c_float, c_int, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.gptq_prepare.restype = c_int
    lib.gptq_quantize_workspace_bytes.argtypes = [i64, i64, c_int, c_int, c_int]
    lib.gptq_quantize_workspace_bytes.restype = ctypes.c_size_t
    lib.gptq_quantize_layer.argtypes = [vp, c_int, i64, i64, vp, vp, c_int, c_int, c_int, c_int,
                                        vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.gptq_quantize_layer.restype = c_int
    lib.gptq_dequant_matmul_workspace_bytes.argtypes = [i64, i64, i64, c_int]
    lib.gptq_dequant_matmul_workspace_bytes.restype = ctypes.c_size_t
    lib.gptq_dequant_matmul.argtypes = [vp, c_int, i64, i64, i64, vp, vp, vp, vp, vp, i64, i64,
                                        c_int, vp, c_int, i64, vp, ctypes.c_size_t, vp]
    lib.gptq_dequant_matmul.restype = c_int
    lib.gptq_dequant_matmul_noalloc.argtypes = [vp, c_int, i64, i64, i64, vp, vp, vp, vp, vp, i64,
                                                i64, c_int, vp, c_int, i64, vp]
    lib.gptq_dequant_matmul_noalloc.restype = c_int
    lib.gptq_dequant_group_order_workspace_bytes.argtypes = [i64]
    lib.gptq_dequant_group_order_workspace_bytes.restype = ctypes.c_size_t
    lib.gptq_dequant_group_order.argtypes = [vp, vp, i64, i64, c_int, vp, vp, vp, vp,
                                             ctypes.c_size_t, vp]
    lib.gptq_dequant_group_order.restype = c_int
    lib.gptq_silu_mul.argtypes = [vp, i64, vp, i64, i64, i64, vp, i64, vp]
    lib.gptq_silu_mul.restype = c_int
    lib.gptq_attention_forward.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, i64, i64, c_int,
                                           c_int, c_int, vp]
    lib.gptq_attention_forward.restype = c_int
    lib.gptq_residual_rmsnorm.argtypes = [vp, i64, vp, i64, vp, i64, i64, ctypes.c_float, vp,
                                          i64, vp, i64, vp]
    lib.gptq_residual_rmsnorm.restype = c_int
    lib.gptq_export_params.argtypes = [vp, vp, i64, i64, c_int, vp, vp, vp]
    lib.gptq_export_params.restype = c_int
    lib.gptq_unpack_zeros.argtypes = [vp, i64, i64, c_int, vp, vp]
    lib.gptq_unpack_zeros.restype = c_int
    lib.gptq_status_string.argtypes = [c_int]
    lib.gptq_status_string.restype = ctypes.c_char_p
    lib.gptq_last_error_message.argtypes = []
    lib.gptq_last_error_message.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != GPTQ_OK:
        lib = load()
        msg = lib.gptq_status_string(status).decode()
        detail = lib.gptq_last_error_message().decode()
        raise GptqError(status, f"{msg}: {detail}" if detail else msg)


def _torch():
    import torch
    return torch


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on(stream):
    """Context for the buffers a wrapper allocates (outputs, workspaces).

    They are allocated on the stream the call is queued on: torch's caching
    allocator then hands their memory to other work only in that stream's
    order, so a call on a side stream cannot have its workspace reused by
    work on the current stream while its kernels still run."""
    if stream is None:
        return contextlib.nullcontext()
    return _torch().cuda.stream(stream)


def _dtype_code(dt) -> int:
    torch = _torch()
    if dt == torch.float16:
        return GPTQ_F16
    if dt == torch.bfloat16:
        return GPTQ_BF16
    if dt == torch.float32:
        return GPTQ_F32
    raise TypeError(f"unsupported dtype {dt}")


def _need_cuda(name, t):
    if t is None or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


# ---------------------------------------------------------------- calls --
def hessian_workspace_bytes(n: int) -> int:
    return int(load().gptq_hessian_workspace_bytes(n))


def hessian_accumulate(H, X, stream=None, workspace=None):
    """H (fp32 [n x n], upper triangle) += 2 X^T X for X [ntok x n] fp16/bf16.

    ``workspace``: None, or a GPU byte tensor of at least
    hessian_workspace_bytes(n) (lets small layers split tiles along the
    tokens)."""
    lib = load()
    _need_cuda("H", H)
    _need_cuda("X", X)
    n = H.shape[0]
    if H.dtype != _torch().float32 or H.dim() != 2 or H.shape[1] != n or not H.is_contiguous():
        raise ValueError("H must be a contiguous fp32 [n x n] tensor")
    if X.dim() != 2 or X.shape[1] != n or X.stride(1) != 1:
        raise ValueError("X must be [ntok x n] with unit column stride")
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (_ptr(workspace), workspace.numel())
    _check(lib.gptq_hessian_accumulate(_ptr(H), n, _ptr(X), _dtype_code(X.dtype), X.shape[0],
                                       X.stride(0) if X.shape[0] > 1 else n, ws_ptr, ws_bytes,
                                       _stream(stream)))
    return H


def prepare_workspace_bytes(n: int) -> int:
    return int(load().gptq_prepare_workspace_bytes(n))


def prepare(H, damp_percent: float, desc_act: bool, Hinv_chol=None, perm=None, info=None,
            workspace=None, stream=None):
    """Returns (Hinv_chol fp32 [n x n], perm int32 [n], info int32 [1]) on H's device."""
    torch = _torch()
    lib = load()
    _need_cuda("H", H)
    n = H.shape[0]
    if H.dtype != torch.float32 or H.dim() != 2 or H.shape[1] != n or not H.is_contiguous():
        raise ValueError("H must be a contiguous fp32 [n x n] tensor")
    dev = H.device
    with _on(stream):
        if Hinv_chol is None:
            Hinv_chol = torch.empty((n, n), dtype=torch.float32, device=dev)
        if perm is None:
            perm = torch.empty((n,), dtype=torch.int32, device=dev)
        if info is None:
            info = torch.empty((1,), dtype=torch.int32, device=dev)
        need = prepare_workspace_bytes(n)
        if workspace is None:
            workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    _check(lib.gptq_prepare(_ptr(H), n, float(damp_percent), int(bool(desc_act)), _ptr(Hinv_chol),
                            _ptr(perm), _ptr(info), _ptr(workspace), workspace.numel(),
                            _stream(stream)))
    return Hinv_chol, perm, info


def quantize_workspace_bytes(out: int, inp: int, bits: int, group_size: int, block: int) -> int:
    return int(load().gptq_quantize_workspace_bytes(out, inp, bits, group_size, block))


def n_groups(inp: int, group_size: int) -> int:
    return 1 if group_size == -1 else -(-inp // group_size)


def quantize_layer(W, Hinv_chol, perm, bits: int, group_size: int, sym: bool, block: int,
                   qweight=None, scales=None, zeros=None, g_idx=None, workspace=None,
                   stream=None):
    """Returns (qweight int32 [in*bits/32 x out], scales fp32 [g x out],
    zeros int32 [g x out], g_idx int32 [in])."""
    torch = _torch()
    lib = load()
    _need_cuda("W", W)
    _need_cuda("Hinv_chol", Hinv_chol)
    if W.dim() != 2 or not W.is_contiguous():
        raise ValueError("W must be a contiguous [out x in] tensor")
    out, inp = W.shape
    if Hinv_chol.dtype != torch.float32 or tuple(Hinv_chol.shape) != (inp, inp) \
            or not Hinv_chol.is_contiguous():
        raise ValueError("Hinv_chol must be a contiguous fp32 [in x in] tensor")
    if perm is not None and (perm.dtype != torch.int32 or perm.numel() != inp or not perm.is_cuda):
        raise ValueError("perm must be a GPU int32 [in] tensor")
    dev = W.device
    g = n_groups(inp, group_size)
    with _on(stream):
        if qweight is None:
            qweight = torch.empty((max(inp * bits // 32, 1), out), dtype=torch.int32, device=dev)
        if scales is None:
            scales = torch.empty((g, out), dtype=torch.float32, device=dev)
        if zeros is None:
            zeros = torch.empty((g, out), dtype=torch.int32, device=dev)
        if g_idx is None:
            g_idx = torch.empty((inp,), dtype=torch.int32, device=dev)
        need = quantize_workspace_bytes(out, inp, bits, group_size, block)
        if workspace is None:
            workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    _check(lib.gptq_quantize_layer(_ptr(W), _dtype_code(W.dtype), out, inp, _ptr(Hinv_chol),
                                   _ptr(perm), int(bits), int(group_size), int(bool(sym)),
                                   int(block), _ptr(qweight), _ptr(scales), _ptr(zeros),
                                   _ptr(g_idx), _ptr(workspace), workspace.numel(),
                                   _stream(stream)))
    return qweight, scales, zeros, g_idx


def dequant_matmul_workspace_bytes(M: int, inp: int, out: int, has_order: bool = False) -> int:
    return int(load().gptq_dequant_matmul_workspace_bytes(M, inp, out, int(bool(has_order))))


def dequant_matmul(X, qweight, scales, zeros, g_idx, bits: int, x_order=None, out_dtype=None,
                   Y=None, workspace=None, stream=None):
    """Y = X W^T with W dequantized on the fly from the packed layer
    (qweight int32 [in*bits/32 x out], scales fp32 / zeros int32
    [n_groups x out], g_idx int32 [in]) for fp16 X [M x in].  x_order
    (int32 [in], optional): packed position p multiplies X column
    x_order[p] (the layer from dequant_group_order).  Y is fp32 (default) or
    fp16 [M x out]."""
    torch = _torch()
    lib = load()
    for name, t in (("X", X), ("qweight", qweight), ("scales", scales), ("zeros", zeros),
                    ("g_idx", g_idx)):
        _need_cuda(name, t)
    if X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be [M x in] with unit column stride")
    M, inp = X.shape
    if qweight.dtype != torch.int32 or qweight.dim() != 2 or not qweight.is_contiguous():
        raise ValueError("qweight must be a contiguous int32 [in*bits/32 x out] tensor")
    if qweight.shape[0] * 32 != inp * bits:
        raise ValueError("qweight rows must be in * bits / 32")
    out = qweight.shape[1]
    G = scales.shape[0]
    if scales.dtype != torch.float32 or tuple(scales.shape) != (G, out) or not scales.is_contiguous():
        raise ValueError("scales must be a contiguous fp32 [n_groups x out] tensor")
    if zeros.dtype != torch.int32 or tuple(zeros.shape) != (G, out) or not zeros.is_contiguous():
        raise ValueError("zeros must be a contiguous int32 [n_groups x out] tensor")
    if g_idx.dtype != torch.int32 or tuple(g_idx.shape) != (inp,):
        raise ValueError("g_idx must be an int32 [in] tensor")
    if x_order is not None:
        _need_cuda("x_order", x_order)
        if x_order.dtype != torch.int32 or tuple(x_order.shape) != (inp,):
            raise ValueError("x_order must be an int32 [in] tensor")
    if out_dtype is None:
        out_dtype = torch.float32 if Y is None else Y.dtype
    with _on(stream):
        if Y is None:
            Y = torch.empty((M, out), dtype=out_dtype, device=X.device)
        if workspace is None:
            need = dequant_matmul_workspace_bytes(M, inp, out, x_order is not None)
            workspace = torch.empty((need,), dtype=torch.uint8, device=X.device) if need else None
    if Y.dim() != 2 or tuple(Y.shape) != (M, out) or Y.stride(1) != 1:
        raise ValueError("Y must be [M x out] with unit column stride")
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (_ptr(workspace), workspace.numel())
    _check(lib.gptq_dequant_matmul(_ptr(X), _dtype_code(X.dtype), M, inp,
                                   X.stride(0) if M > 1 else inp, _ptr(qweight), _ptr(scales),
                                   _ptr(zeros), _ptr(g_idx),
                                   None if x_order is None else _ptr(x_order), G, out, bits,
                                   _ptr(Y), _dtype_code(Y.dtype), Y.stride(0) if M > 1 else out,
                                   ws_ptr, ws_bytes, _stream(stream)))
    return Y


def dequant_matmul_noalloc(X, qweight, scales, zeros, g_idx, bits: int, Y, x_order=None,
                           stream=None):
    """dequant_matmul through gptq_dequant_matmul_noalloc: no workspace (the
    library's fixed per-device scratch) and no allocation here either, so Y
    (fp32 or fp16 [M x out]) must be given."""
    torch = _torch()
    lib = load()
    for name, t in (("X", X), ("qweight", qweight), ("scales", scales), ("zeros", zeros),
                    ("g_idx", g_idx), ("Y", Y)):
        _need_cuda(name, t)
    if X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be [M x in] with unit column stride")
    M, inp = X.shape
    if qweight.dtype != torch.int32 or qweight.dim() != 2 or not qweight.is_contiguous():
        raise ValueError("qweight must be a contiguous int32 [in*bits/32 x out] tensor")
    if qweight.shape[0] * 32 != inp * bits:
        raise ValueError("qweight rows must be in * bits / 32")
    out = qweight.shape[1]
    G = scales.shape[0]
    if scales.dtype != torch.float32 or tuple(scales.shape) != (G, out) or not scales.is_contiguous():
        raise ValueError("scales must be a contiguous fp32 [n_groups x out] tensor")
    if zeros.dtype != torch.int32 or tuple(zeros.shape) != (G, out) or not zeros.is_contiguous():
        raise ValueError("zeros must be a contiguous int32 [n_groups x out] tensor")
    if g_idx.dtype != torch.int32 or tuple(g_idx.shape) != (inp,):
        raise ValueError("g_idx must be an int32 [in] tensor")
    if x_order is not None:
        _need_cuda("x_order", x_order)
        if x_order.dtype != torch.int32 or tuple(x_order.shape) != (inp,):
            raise ValueError("x_order must be an int32 [in] tensor")
    if Y.dim() != 2 or tuple(Y.shape) != (M, out) or Y.stride(1) != 1:
        raise ValueError("Y must be [M x out] with unit column stride")
    _check(lib.gptq_dequant_matmul_noalloc(_ptr(X), _dtype_code(X.dtype), M, inp,
                                           X.stride(0) if M > 1 else inp, _ptr(qweight),
                                           _ptr(scales), _ptr(zeros), _ptr(g_idx),
                                           None if x_order is None else _ptr(x_order), G, out,
                                           bits, _ptr(Y), _dtype_code(Y.dtype),
                                           Y.stride(0) if M > 1 else out, _stream(stream)))
    return Y


def dequant_group_order_workspace_bytes(inp: int) -> int:
    return int(load().gptq_dequant_group_order_workspace_bytes(inp))


def dequant_group_order(qweight, g_idx, bits: int, stream=None):
    """(qweight_sorted, g_idx_sorted, x_order): the packed layer's input
    positions sorted by group (stable) and its codes re-packed in that order,
    for dequant_matmul(X, qweight_sorted, scales, zeros, g_idx_sorted, bits,
    x_order=x_order)."""
    torch = _torch()
    lib = load()
    _need_cuda("qweight", qweight)
    _need_cuda("g_idx", g_idx)
    if qweight.dtype != torch.int32 or qweight.dim() != 2 or not qweight.is_contiguous():
        raise ValueError("qweight must be a contiguous int32 [in*bits/32 x out] tensor")
    inp = g_idx.shape[0]
    if g_idx.dtype != torch.int32 or g_idx.dim() != 1 or not g_idx.is_contiguous():
        raise ValueError("g_idx must be a contiguous int32 [in] tensor")
    if qweight.shape[0] * 32 != inp * bits:
        raise ValueError("qweight rows must be in * bits / 32")
    out = qweight.shape[1]
    with _on(stream):
        qs = torch.empty_like(qweight)
        gs = torch.empty_like(g_idx)
        order = torch.empty_like(g_idx)
        ws = torch.empty((dequant_group_order_workspace_bytes(inp),), dtype=torch.uint8,
                         device=qweight.device)
    _check(lib.gptq_dequant_group_order(_ptr(qweight), _ptr(g_idx), inp, out, int(bits),
                                        _ptr(qs), _ptr(gs), _ptr(order), _ptr(ws), ws.numel(),
                                        _stream(stream)))
    return qs, gs, order


def silu_mul(G, U, A=None, stream=None):
    """A = SiLU(G) * U for fp16 [rows x cols] G, U (unit column stride; they
    may be views of one matrix).  A: fp16 out, allocated when None."""
    torch = _torch()
    lib = load()
    _need_cuda("G", G)
    _need_cuda("U", U)
    for name, t in (("G", G), ("U", U)):
        if t.dtype != torch.float16 or t.dim() != 2 or t.stride(1) != 1:
            raise ValueError(f"{name} must be fp16 [rows x cols] with unit column stride")
    if tuple(G.shape) != tuple(U.shape):
        raise ValueError("G and U must have the same shape")
    rows, cols = G.shape
    if A is None:
        with _on(stream):
            A = torch.empty((rows, cols), dtype=torch.float16, device=G.device)
    if A.dtype != torch.float16 or tuple(A.shape) != (rows, cols) or A.stride(1) != 1:
        raise ValueError("A must be fp16 [rows x cols] with unit column stride")
    ld = lambda t: t.stride(0) if rows > 1 else cols
    _check(lib.gptq_silu_mul(_ptr(G), ld(G), _ptr(U), ld(U), rows, cols, _ptr(A), ld(A),
                             _stream(stream)))
    return A


def attention_forward(Q, K, V, seq_len: int, heads: int, causal: bool = True, O=None,
                      stream=None):
    """O = softmax(Q K^T / sqrt(hd)) V per sequence and head for fp16
    Q, K, V [tokens x heads * hd] (unit column stride; views of one matrix
    are fine); tokens = seqs * seq_len, hd = 64 or 128.  O: fp16 out,
    allocated when None."""
    torch = _torch()
    lib = load()
    for name, t in (("Q", Q), ("K", K), ("V", V)):
        _need_cuda(name, t)
        if t.dtype != torch.float16 or t.dim() != 2 or t.stride(1) != 1:
            raise ValueError(f"{name} must be fp16 [tokens x heads*hd] with unit column stride")
    if not (Q.shape == K.shape == V.shape):
        raise ValueError("Q, K and V must have the same shape")
    tokens, w = Q.shape
    if seq_len < 1 or tokens % seq_len:
        raise ValueError("tokens must be a multiple of seq_len")
    if heads < 1 or w % heads:
        raise ValueError("the width must be heads * head_dim")
    if O is None:
        with _on(stream):
            O = torch.empty((tokens, w), dtype=torch.float16, device=Q.device)
    if O.dtype != torch.float16 or tuple(O.shape) != (tokens, w) or O.stride(1) != 1:
        raise ValueError("O must be fp16 [tokens x heads*hd] with unit column stride")
    ld = lambda t: t.stride(0) if tokens > 1 else w
    _check(lib.gptq_attention_forward(_ptr(Q), ld(Q), _ptr(K), ld(K), _ptr(V), ld(V), _ptr(O),
                                      ld(O), tokens // seq_len, seq_len, heads, w // heads,
                                      int(bool(causal)), _stream(stream)))
    return O


def residual_rmsnorm(X, A, gamma, eps: float, Hs=None, U=None, stream=None):
    """(Hs, U): Hs = X + A, U = Hs / sqrt(mean(Hs^2) + eps) * gamma, rows of
    fp16 [rows x d] (unit column stride), gamma fp16 [d]."""
    torch = _torch()
    lib = load()
    for name, t in (("X", X), ("A", A), ("gamma", gamma)):
        _need_cuda(name, t)
    for name, t in (("X", X), ("A", A)):
        if t.dtype != torch.float16 or t.dim() != 2 or t.stride(1) != 1:
            raise ValueError(f"{name} must be fp16 [rows x d] with unit column stride")
    if X.shape != A.shape:
        raise ValueError("X and A must have the same shape")
    rows, d = X.shape
    if gamma.dtype != torch.float16 or tuple(gamma.shape) != (d,) or not gamma.is_contiguous():
        raise ValueError("gamma must be a contiguous fp16 [d] tensor")
    with _on(stream):
        if Hs is None:
            Hs = torch.empty((rows, d), dtype=torch.float16, device=X.device)
        if U is None:
            U = torch.empty((rows, d), dtype=torch.float16, device=X.device)
    for name, t in (("Hs", Hs), ("U", U)):
        if t.dtype != torch.float16 or tuple(t.shape) != (rows, d) or t.stride(1) != 1:
            raise ValueError(f"{name} must be fp16 [rows x d] with unit column stride")
    ld = lambda t: t.stride(0) if rows > 1 else d
    _check(lib.gptq_residual_rmsnorm(_ptr(X), ld(X), _ptr(A), ld(A), _ptr(gamma), rows, d,
                                     float(eps), _ptr(Hs), ld(Hs), _ptr(U), ld(U),
                                     _stream(stream)))
    return Hs, U


def export_params(scales, zeros, bits: int, stream=None):
    """(scales fp16 [G x out], qzeros int32 [G x out*bits/32]) for saving."""
    torch = _torch()
    lib = load()
    _need_cuda("scales", scales)
    _need_cuda("zeros", zeros)
    if scales.dtype != torch.float32 or scales.dim() != 2 or not scales.is_contiguous():
        raise ValueError("scales must be a contiguous fp32 [n_groups x out] tensor")
    if zeros.dtype != torch.int32 or tuple(zeros.shape) != tuple(scales.shape) \
            or not zeros.is_contiguous():
        raise ValueError("zeros must be a contiguous int32 tensor shaped like scales")
    G, out = scales.shape
    with _on(stream):
        s16 = torch.empty((G, out), dtype=torch.float16, device=scales.device)
        qz = torch.empty((G, out * bits // 32), dtype=torch.int32, device=scales.device)
    _check(lib.gptq_export_params(_ptr(scales), _ptr(zeros), G, out, int(bits), _ptr(s16),
                                  _ptr(qz), _stream(stream)))
    return s16, qz


def unpack_zeros(qzeros, out: int, bits: int, stream=None):
    """zeros int32 [G x out] from qzeros int32 [G x out*bits/32]."""
    torch = _torch()
    lib = load()
    _need_cuda("qzeros", qzeros)
    if qzeros.dtype != torch.int32 or qzeros.dim() != 2 or not qzeros.is_contiguous():
        raise ValueError("qzeros must be a contiguous int32 [n_groups x out*bits/32] tensor")
    G = qzeros.shape[0]
    if qzeros.shape[1] * 32 != out * bits:
        raise ValueError("qzeros columns must be out * bits / 32")
    with _on(stream):
        z = torch.empty((G, out), dtype=torch.int32, device=qzeros.device)
    _check(lib.gptq_unpack_zeros(_ptr(qzeros), G, out, int(bits), _ptr(z), _stream(stream)))
    return z
