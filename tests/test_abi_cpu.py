"""The C-ABI library loads, exports every function include/gptq.h declares,
and rejects invalid arguments on the host before any HIP call (no GPU needed)."""
import ctypes

import pytest

import post_weight_quantization_12_amd as P
from post_weight_quantization_12_amd import _lib as L

FAKE = ctypes.c_void_p(4096)  # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    return P.load()


def test_exports_every_header_function(lib):
    names = P.header_functions()
    assert set(names) == {"gptq_hessian_workspace_bytes", "gptq_hessian_accumulate",
                          "gptq_prepare_workspace_bytes",
                          "gptq_prepare", "gptq_quantize_workspace_bytes",
                          "gptq_quantize_layer", "gptq_dequant_matmul_workspace_bytes",
                          "gptq_dequant_matmul", "gptq_dequant_matmul_noalloc",
                          "gptq_dequant_group_order_workspace_bytes",
                          "gptq_dequant_group_order", "gptq_silu_mul", "gptq_attention_forward",
                          "gptq_residual_rmsnorm", "gptq_export_params",
                          "gptq_unpack_zeros", "gptq_status_string",
                          "gptq_last_error_message"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in range(5):
        assert lib.gptq_status_string(s)
    assert b"unknown" in lib.gptq_status_string(99)


def test_hessian_argument_errors(lib):
    f = lib.gptq_hessian_accumulate
    assert f(None, 8, FAKE, 0, 4, 8, None, 0, None) == L.GPTQ_ERR_INVALID_ARG
    assert b"H" in lib.gptq_last_error_message()
    assert f(FAKE, 8, None, 0, 4, 8, None, 0, None) == L.GPTQ_ERR_INVALID_ARG
    assert f(FAKE, 0, FAKE, 0, 4, 8, None, 0, None) == L.GPTQ_ERR_INVALID_ARG
    assert f(FAKE, 8, FAKE, 0, -1, 8, None, 0, None) == L.GPTQ_ERR_INVALID_ARG
    assert f(FAKE, 8, FAKE, 0, 4, 7, None, 0, None) == L.GPTQ_ERR_INVALID_ARG
    assert b"ldx" in lib.gptq_last_error_message()
    assert f(FAKE, 8, FAKE, 2, 4, 8, None, 0, None) == L.GPTQ_ERR_UNSUPPORTED
    # a workspace, when given, must be at least the queried size
    ws = lib.gptq_hessian_workspace_bytes(8)
    assert ws > 0 and lib.gptq_hessian_workspace_bytes(0) == 0
    # whole 256 x 256 tiles fill the GPU at n = 11008 (990 tiles): no workspace
    assert lib.gptq_hessian_workspace_bytes(11008) == 0
    # n = 4096 (136 tiles): the token-split partials, one 256 KiB tile per item
    assert lib.gptq_hessian_workspace_bytes(4096) >= 1024 * 256 * 1024
    assert f(FAKE, 8, FAKE, 0, 4, 8, FAKE, ws - 1, None) == L.GPTQ_ERR_WORKSPACE
    # ntok == 0 is a no-op that never touches the device
    assert f(FAKE, 8, FAKE, 0, 0, 8, None, 0, None) == L.GPTQ_OK
    assert lib.gptq_last_error_message() == b""


def test_prepare_argument_errors(lib):
    f = lib.gptq_prepare
    ws = lib.gptq_prepare_workspace_bytes(64)
    assert ws > 64 * 64 * 4
    assert lib.gptq_prepare_workspace_bytes(0) == 0
    assert lib.gptq_prepare_workspace_bytes(L.MAX_PREPARE_N + 1) == 0
    assert f(None, 64, 0.01, 0, FAKE, FAKE, FAKE, FAKE, ws, None) == L.GPTQ_ERR_INVALID_ARG
    assert f(FAKE, 64, 0.01, 0, FAKE, None, FAKE, FAKE, ws, None) == L.GPTQ_ERR_INVALID_ARG
    assert f(FAKE, 64, -0.1, 0, ctypes.c_void_p(8192), FAKE, FAKE, FAKE, ws, None) == \
        L.GPTQ_ERR_INVALID_ARG
    assert f(FAKE, 64, float("nan"), 0, ctypes.c_void_p(8192), FAKE, FAKE, FAKE, ws, None) == \
        L.GPTQ_ERR_INVALID_ARG
    assert f(FAKE, L.MAX_PREPARE_N + 1, 0.01, 0, ctypes.c_void_p(8192), FAKE, FAKE, FAKE, ws,
             None) == L.GPTQ_ERR_UNSUPPORTED
    assert f(FAKE, 64, 0.01, 0, FAKE, ctypes.c_void_p(8192), FAKE, FAKE, ws, None) == \
        L.GPTQ_ERR_INVALID_ARG  # H aliases Hinv_chol
    assert f(FAKE, 64, 0.01, 0, ctypes.c_void_p(8192), FAKE, FAKE, FAKE, ws - 1, None) == \
        L.GPTQ_ERR_WORKSPACE


def _q(lib, out=16, inp=256, bits=4, gs=128, sym=0, block=128, ws=None, W=FAKE, dtype=0):
    if ws is None:
        ws = lib.gptq_quantize_workspace_bytes(out, inp, bits, gs, block) or 1
    return lib.gptq_quantize_layer(W, dtype, out, inp, FAKE, None, bits, gs, sym, block,
                                   FAKE, FAKE, FAKE, FAKE, FAKE, ws, None)


def test_quantize_argument_errors(lib):
    assert lib.gptq_quantize_workspace_bytes(16, 256, 4, 128, 128) >= 16 * 256 * 4 + 256 * 256 * 4
    assert _q(lib, W=None) == L.GPTQ_ERR_INVALID_ARG
    assert _q(lib, dtype=7) == L.GPTQ_ERR_INVALID_ARG
    assert _q(lib, out=0) == L.GPTQ_ERR_INVALID_ARG
    assert _q(lib, inp=250) == L.GPTQ_ERR_INVALID_ARG
    assert b"multiple of 32" in lib.gptq_last_error_message()
    assert _q(lib, bits=5) == L.GPTQ_ERR_UNSUPPORTED
    assert _q(lib, bits=1) == L.GPTQ_ERR_UNSUPPORTED
    assert _q(lib, block=96) == L.GPTQ_ERR_UNSUPPORTED
    assert _q(lib, gs=96) == L.GPTQ_ERR_INVALID_ARG     # does not divide block
    assert _q(lib, gs=2) == L.GPTQ_ERR_INVALID_ARG      # not a multiple of 4
    assert _q(lib, gs=256) == L.GPTQ_ERR_INVALID_ARG    # larger than block
    assert _q(lib, gs=0) == L.GPTQ_ERR_INVALID_ARG
    assert _q(lib, sym=2) == L.GPTQ_ERR_INVALID_ARG
    assert _q(lib, ws=10) == L.GPTQ_ERR_WORKSPACE
    assert lib.gptq_quantize_workspace_bytes(16, 256, 5, 128, 128) == 0


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        P.hessian_accumulate(torch.zeros(4, 4), torch.zeros(2, 4, dtype=torch.float16))
    with pytest.raises(ValueError):
        P.prepare(torch.eye(4), 0.01, False)


def test_dequant_matmul_argument_errors(lib):
    f = lib.gptq_dequant_matmul
    A16 = ctypes.c_void_p(4096)   # 16-byte aligned, never dereferenced
    ok = dict(X=A16, xd=L.GPTQ_F16, M=2, inp=64, ldx=64, q=FAKE, s=FAKE, z=FAKE, g=FAKE,
              xo=None, G=2, out=8, bits=4, Y=FAKE, yd=L.GPTQ_F32, ldy=8)

    def call(**kw):
        a = dict(ok, **kw)
        ws = lib.gptq_dequant_matmul_workspace_bytes(a["M"], a["inp"], a["out"],
                                                     int(a["xo"] is not None))
        return f(a["X"], a["xd"], a["M"], a["inp"], a["ldx"], a["q"], a["s"], a["z"], a["g"],
                 a["xo"], a["G"], a["out"], a["bits"], a["Y"], a["yd"], a["ldy"],
                 kw.get("ws", FAKE if ws else None), kw.get("wsb", ws), None)

    assert call(X=None) == L.GPTQ_ERR_INVALID_ARG
    assert call(q=None) == L.GPTQ_ERR_INVALID_ARG
    assert call(Y=None) == L.GPTQ_ERR_INVALID_ARG
    assert call(M=-1) == L.GPTQ_ERR_INVALID_ARG
    assert call(inp=48, ldx=48) == L.GPTQ_ERR_INVALID_ARG
    assert b"multiple of 32" in lib.gptq_last_error_message()
    assert call(out=0) == L.GPTQ_ERR_INVALID_ARG
    assert call(G=0) == L.GPTQ_ERR_INVALID_ARG
    assert call(ldx=32) == L.GPTQ_ERR_INVALID_ARG
    assert call(ldy=4) == L.GPTQ_ERR_INVALID_ARG
    assert call(xd=L.GPTQ_BF16) == L.GPTQ_ERR_UNSUPPORTED
    assert call(yd=L.GPTQ_BF16) == L.GPTQ_ERR_INVALID_ARG
    assert call(bits=5) == L.GPTQ_ERR_UNSUPPORTED
    assert call(ldx=68) == L.GPTQ_ERR_UNSUPPORTED
    assert call(X=ctypes.c_void_p(4098)) == L.GPTQ_ERR_UNSUPPORTED
    # the small-M path splits the input range: a workspace is required
    need = lib.gptq_dequant_matmul_workspace_bytes(1, 4096, 4096, 0)
    # 8192 tokens: 32 x 16 tiles of 256 x 256 fill the GPU, no split; only the
    # chunk group table (4096 / 32 ints) remains
    assert need > 0 and lib.gptq_dequant_matmul_workspace_bytes(8192, 4096, 4096, 0) == 512
    # out not a multiple of 4: only the 128-row tiles may run, no table
    assert lib.gptq_dequant_matmul_workspace_bytes(8192, 4096, 4098, 0) == 0
    # 64 tokens: 32 output tiles, the input range split for the rest of the GPU
    assert lib.gptq_dequant_matmul_workspace_bytes(64, 4096, 4096, 0) >= 2 * 64 * 4096 * 4
    assert lib.gptq_dequant_matmul_workspace_bytes(0, 4096, 4096, 0) == 0
    # with an x_order the matrix-core path gathers X (M x in fp16) first
    assert lib.gptq_dequant_matmul_workspace_bytes(64, 4096, 4096, 1) >= 64 * 4096 * 2
    assert call(M=64, xo=FAKE, ws=None, wsb=0) == L.GPTQ_ERR_INVALID_ARG
    assert call(M=64, xo=FAKE, ws=FAKE, wsb=64 * 64 * 2 - 1) == L.GPTQ_ERR_WORKSPACE
    assert call(M=1, inp=4096, ldx=4096, out=4096, ldy=4096, ws=None, wsb=0) == \
        L.GPTQ_ERR_INVALID_ARG
    assert call(M=1, inp=4096, ldx=4096, out=4096, ldy=4096, ws=FAKE, wsb=need - 1) == \
        L.GPTQ_ERR_WORKSPACE
    # M == 0 is a no-op that never touches the device
    assert call(M=0) == L.GPTQ_OK


def test_dequant_group_order_argument_errors(lib):
    f = lib.gptq_dequant_group_order
    Q2 = ctypes.c_void_p(8192)
    ws = lib.gptq_dequant_group_order_workspace_bytes(64)
    assert ws >= 2 * 64 * 4 and lib.gptq_dequant_group_order_workspace_bytes(0) == 0

    def call(q=FAKE, g=FAKE, inp=64, out=8, bits=4, qs=Q2, gs=FAKE, xo=FAKE, w=FAKE, wsb=ws):
        return f(q, g, inp, out, bits, qs, gs, xo, w, wsb, None)

    assert call(q=None) == L.GPTQ_ERR_INVALID_ARG
    assert call(g=None) == L.GPTQ_ERR_INVALID_ARG
    assert call(qs=None) == L.GPTQ_ERR_INVALID_ARG
    assert call(xo=None) == L.GPTQ_ERR_INVALID_ARG
    assert call(qs=FAKE) == L.GPTQ_ERR_INVALID_ARG
    assert b"alias" in lib.gptq_last_error_message()
    assert call(inp=48) == L.GPTQ_ERR_INVALID_ARG
    assert call(out=0) == L.GPTQ_ERR_INVALID_ARG
    assert call(bits=5) == L.GPTQ_ERR_UNSUPPORTED
    assert call(w=None) == L.GPTQ_ERR_INVALID_ARG
    assert call(wsb=ws - 1) == L.GPTQ_ERR_WORKSPACE


def test_silu_mul_argument_errors(lib):
    f = lib.gptq_silu_mul
    assert f(None, 8, FAKE, 8, 2, 8, FAKE, 8, None) == L.GPTQ_ERR_INVALID_ARG
    assert f(FAKE, 8, FAKE, 8, -1, 8, FAKE, 8, None) == L.GPTQ_ERR_INVALID_ARG
    assert f(FAKE, 4, FAKE, 8, 2, 8, FAKE, 8, None) == L.GPTQ_ERR_INVALID_ARG
    assert b"leading" in lib.gptq_last_error_message()
    assert f(FAKE, 8, FAKE, 8, 0, 8, FAKE, 8, None) == L.GPTQ_OK   # no-op, no device access


def test_export_argument_errors(lib):
    f = lib.gptq_export_params
    assert f(None, FAKE, 2, 8, 4, FAKE, FAKE, None) == L.GPTQ_ERR_INVALID_ARG
    assert f(FAKE, FAKE, 0, 8, 4, FAKE, FAKE, None) == L.GPTQ_ERR_INVALID_ARG
    assert f(FAKE, FAKE, 2, 8, 5, FAKE, FAKE, None) == L.GPTQ_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, 2, 6, 4, FAKE, FAKE, None) == L.GPTQ_ERR_UNSUPPORTED  # 24 bits a row
    g = lib.gptq_unpack_zeros
    assert g(None, 2, 8, 4, FAKE, None) == L.GPTQ_ERR_INVALID_ARG
    assert g(FAKE, 2, 10, 3, FAKE, None) == L.GPTQ_ERR_UNSUPPORTED            # 30 bits a row


def test_dequant_matmul_noalloc_host_checks(lib):
    """The fixed-scratch variant checks its arguments like gptq_dequant_matmul
    and refuses, before any HIP call, a product whose scratch would exceed
    the fixed size."""
    f = lib.gptq_dequant_matmul_noalloc
    A16 = ctypes.c_void_p(4096)

    def call(M=2, inp=64, out=8, X=A16, xo=None, bits=4):
        return f(X, L.GPTQ_F16, M, inp, inp, FAKE, FAKE, FAKE, FAKE, xo, 2, out, bits, FAKE,
                 L.GPTQ_F32, out, None)

    assert call(X=None) == L.GPTQ_ERR_INVALID_ARG
    assert call(bits=5) == L.GPTQ_ERR_UNSUPPORTED
    assert call(M=0) == L.GPTQ_OK
    # 2048 act-order tokens of the 11008-input layer: the gathered X alone is
    # 2048 * 11008 * 2 bytes, beyond the fixed 16 MiB
    assert lib.gptq_dequant_matmul_workspace_bytes(2048, 11008, 4096, 1) > 16 << 20
    assert call(M=2048, inp=11008, out=4096, xo=FAKE) == L.GPTQ_ERR_WORKSPACE
    assert b"16777216" in lib.gptq_last_error_message()
    # every decode product (M <= 8) fits, up to the 70B down_proj shape
    for M in (1, 2, 4, 8):
        for inp, out in ((4096, 4096), (11008, 4096), (28672, 8192), (8192, 28672)):
            assert lib.gptq_dequant_matmul_workspace_bytes(M, inp, out, 1) <= 16 << 20
