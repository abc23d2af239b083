"""Local checkpoint of quantized layers: a safetensors file and a
quantize_config.json in one directory.

The pages save quantized models with save_quantized as safetensors plus a
quantize_config.json holding the quantization parameters ("AutoGPTQ"
catalogue page, Safetensors Support; "GPTQ > Using AutoGPTQ in Practice",
the BaseQuantizeConfig fields bits, group_size, desc_act, damp_percent).
Stored per layer <name>: <name>.qweight int32 [in*b/32 x out] (as
gptq_quantize_layer packs it), <name>.qzeros int32 [G x out*b/32] and
<name>.scales fp16 [G x out] (gptq_export_params), <name>.g_idx int32 [in].
The conversions run in the HIP library; this module moves the tensors to
and from the file.  No upload: the pages' Hub integration is out of scope.
"""
from __future__ import annotations

import json
import os

from . import _lib as L

CONFIG_NAME = "quantize_config.json"
WEIGHTS_NAME = "model.safetensors"


def save_quantized(directory: str, layers: dict, bits: int, group_size: int, desc_act: bool,
                   damp_percent: float, sym: bool, stream=None) -> None:
    """layers: name -> (qweight, scales fp32, zeros int32, g_idx), device tensors."""
    import safetensors.torch
    torch = L._torch()
    os.makedirs(directory, exist_ok=True)
    tensors = {}
    for name, (qweight, scales, zeros, g_idx) in layers.items():
        s16, qz = L.export_params(scales, zeros, bits, stream=stream)
        for key, t in (("qweight", qweight), ("qzeros", qz), ("scales", s16), ("g_idx", g_idx)):
            tensors[f"{name}.{key}"] = t
    torch.cuda.synchronize()
    safetensors.torch.save_file({k: v.detach().cpu().contiguous() for k, v in tensors.items()},
                                os.path.join(directory, WEIGHTS_NAME))
    with open(os.path.join(directory, CONFIG_NAME), "w") as f:
        json.dump({"bits": int(bits), "group_size": int(group_size), "desc_act": bool(desc_act),
                   "damp_percent": float(damp_percent), "sym": bool(sym)}, f, indent=2)


def load_quantized(directory: str, device="cuda", stream=None):
    """(config dict, name -> (qweight, scales fp32, zeros int32, g_idx)) on device.
    The stored fp16 scales come back as fp32 (exactly)."""
    import safetensors.torch
    torch = L._torch()
    cfg = json.load(open(os.path.join(directory, CONFIG_NAME)))
    raw = safetensors.torch.load_file(os.path.join(directory, WEIGHTS_NAME), device="cpu")
    names = sorted({k.rsplit(".", 1)[0] for k in raw})
    layers = {}
    for name in names:
        qweight = raw[f"{name}.qweight"].to(device)
        s16 = raw[f"{name}.scales"].to(device)
        out = s16.shape[1]
        zeros = L.unpack_zeros(raw[f"{name}.qzeros"].to(device).contiguous(), out, cfg["bits"],
                               stream=stream)
        layers[name] = (qweight, s16.to(torch.float32), zeros, raw[f"{name}.g_idx"].to(device))
    return cfg, layers
