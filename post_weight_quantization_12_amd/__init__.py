"""GPTQ layer-wise weight quantization on AMD Instinct MI355X (gfx950).

The work runs in hand-written HIP kernels behind a C ABI (include/gptq.h,
libgptq_mi355x.so); this package is the thin Python binding.
"""
from ._lib import (  # noqa: F401
    GptqError,
    GPTQ_BF16,
    GPTQ_F16,
    GPTQ_F32,
    attention_forward,
    dequant_group_order,
    dequant_group_order_workspace_bytes,
    dequant_matmul,
    dequant_matmul_noalloc,
    dequant_matmul_workspace_bytes,
    export_params,
    hessian_accumulate,
    hessian_workspace_bytes,
    header_functions,
    load,
    n_groups,
    prepare,
    prepare_workspace_bytes,
    quantize_layer,
    quantize_workspace_bytes,
    residual_rmsnorm,
    silu_mul,
    unpack_zeros,
)
from . import block  # noqa: F401,E402
from . import checkpoint  # noqa: F401,E402
