"""Throughput of GPTQ layer quantization on one MI355X.

One step = the whole per-layer path on one batch of synthetic calibration
data already resident in HBM:
    H = 0; H += 2 X_c^T X_c for every chunk (gptq_hessian_accumulate)
    gptq_prepare (damp, desc_act order, U = chol(H_p^-1) upper)
    gptq_quantize_layer (sweep + lazy GEMMs + pack)
value = weights quantized per second = out * in / step time.

Default workload: the Llama-7B q_proj-shaped layer (W 4096 x 4096 fp16,
128 samples x 2048 tokens of fp16 calibration activations, 4-bit asymmetric,
group 128, damp 0.01, block 128).  --config c3 selects the 4096 x 11008
down_proj layer, c4a / c4b the 8192 x 28672 70B down_proj layer.

Prints ONE JSON line (rank 0; this build is single-GPU).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP16_TFLOPS = 2500.0      # MI355X dense fp16 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "GPTQ weights quantized/sec per layer (4-bit g128) + Hessian TFLOP/s, 1 GPU"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_sha(name: str) -> str:
    p = os.path.join(ROOT, "post_weight_quantization_12_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def load_traffic(kernel_file: str, workload: str, launch_units: float):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    --pmc summary, or None when there is none or the kernel source changed."""
    path = os.path.join(ROOT, "profiles", f"syrk_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except ValueError:
        return None
    if d.get("source_sha") != kernel_source_sha(kernel_file):
        return None
    return float(d["hbm_bytes_per_launch"])


def syrk_kernel_name(n: int) -> str:
    """Kernels one gptq_hessian_accumulate launch runs (with a workspace): the
    stream-K schedule adds a fix-up kernel when 256 x 256 tiles would leave
    more than a quarter of the compute units idle."""
    import torch
    nt = (n + 255) // 256
    tiles = nt * (nt + 1) // 2
    cus = torch.cuda.get_device_properties(0).multi_processor_count // 8 * 8
    if 4 * tiles < 3 * min(cus, 512):
        return "syrk_dma_kernel + syrk_streamk_fixup (gptq_hessian_accumulate, stream-K)"
    return "syrk_dma_kernel (gptq_hessian_accumulate)"


def cpu_baseline(cfg, steps_tokens: int):
    """The oracle, untuned, on a bounded sample of the same workload:
    Hessian over one 2048-token sample, the full prepare at the layer's n,
    and the sweep of 32 output rows; scaled to the whole layer."""
    import numpy as np
    import torch

    import oracle as O
    import workloads

    torch.set_num_threads(max(1, len(os.sched_getaffinity(0))))
    X = workloads.x_sample(cfg, 0, "cpu").numpy()
    W = workloads.weight(cfg, "cpu").double().numpy()
    rows = 32
    t0 = time.perf_counter()
    H = O.hessian(X)
    t_h = time.perf_counter() - t0
    t0 = time.perf_counter()
    Hd, _ = O.condition(H, cfg.damp)
    perm = O.column_order(H, cfg.desc_act)
    U = O.hinv_chol(Hd, perm)
    t_p = time.perf_counter() - t0
    t0 = time.perf_counter()
    res = O.gptq_sweep(W[:rows], U, perm, cfg.bits, cfg.group_size, cfg.sym)
    O.pack(res.codes, cfg.bits)
    t_s = time.perf_counter() - t0
    t_full = t_h * (steps_tokens / X.shape[0]) + t_p + t_s * (cfg.out / rows)
    weights = cfg.out * cfg.inp
    return {
        "value": weights / t_full,
        "unit": "weights/s",
        "cores": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": (f"Hessian over 1 of {cfg.samples} samples ({X.shape[0]} tokens, "
                   f"{t_h:.2f} s, scaled x{steps_tokens // X.shape[0]}); full prepare at "
                   f"n={cfg.inp} ({t_p:.2f} s); sweep+pack of {rows} of {cfg.out} rows "
                   f"({t_s:.2f} s, scaled x{cfg.out // rows}); fp64 NumPy"),
        "sample_seconds": round(t_h + t_p + t_s, 2),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="c1", choices=["c1", "c2", "c3", "c4a", "c4b"])
    ap.add_argument("--chunk-samples", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain 1 GiB device-to-device copy (a reference kernel "
                         "of known traffic for calibrating rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this GPTQ build runs on one GPU only (no sharding, no collectives); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import post_weight_quantization_12_amd as P
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = workloads.get(args.config)
    n, out = cfg.inp, cfg.out
    log(f"[bench] config {cfg.name}: W {out}x{n}, X {cfg.samples}x{cfg.tokens_per_sample}x{n} fp16, "
        f"{cfg.bits}-bit g{cfg.group_size} sym={cfg.sym} desc_act={cfg.desc_act}")

    # ---- synthetic inputs, generated on the GPU and kept resident -------------
    t0 = time.perf_counter()
    mixing = workloads._mixing(cfg, dev, 0)
    outl = workloads.outlier_channels(cfg, dev, 0)
    X = torch.empty((cfg.tokens, n), dtype=torch.float16, device=dev)
    T = cfg.tokens_per_sample
    for s in range(cfg.samples):
        X[s * T:(s + 1) * T] = workloads.x_sample(cfg, s, dev, 0, mixing, outl)
    W = workloads.weight(cfg, dev)
    del mixing
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f} s "
        f"(X {X.numel() * 2 / 2**30:.2f} GiB)")

    H = torch.empty((n, n), dtype=torch.float32, device=dev)
    U = torch.empty((n, n), dtype=torch.float32, device=dev)
    perm = torch.empty((n,), dtype=torch.int32, device=dev)
    info = torch.empty((1,), dtype=torch.int32, device=dev)
    wsh = torch.empty((P.hessian_workspace_bytes(n),), dtype=torch.uint8, device=dev)
    wsp = torch.empty((P.prepare_workspace_bytes(n),), dtype=torch.uint8, device=dev)
    g = P.n_groups(n, cfg.group_size)
    qweight = torch.empty((n * cfg.bits // 32, out), dtype=torch.int32, device=dev)
    scales = torch.empty((g, out), dtype=torch.float32, device=dev)
    zeros = torch.empty((g, out), dtype=torch.int32, device=dev)
    g_idx = torch.empty((n,), dtype=torch.int32, device=dev)
    wsq = torch.empty((P.quantize_workspace_bytes(out, n, cfg.bits, cfg.group_size, cfg.block),),
                      dtype=torch.uint8, device=dev)
    chunk = args.chunk_samples * T
    chunks = [X[i:i + chunk] for i in range(0, cfg.tokens, chunk)]
    stream = torch.cuda.current_stream()

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    def step(record):
        e0 = ev()
        H.zero_()
        syrk_ev = []
        for c in chunks:
            a = ev()
            P.hessian_accumulate(H, c, stream, wsh)
            syrk_ev.append((a, ev()))
        e1 = ev()
        P.prepare(H, cfg.damp, cfg.desc_act, U, perm, info, wsp, stream)
        e2 = ev()
        P.quantize_layer(W, U, perm, cfg.bits, cfg.group_size, cfg.sym, cfg.block,
                         qweight, scales, zeros, g_idx, wsq, stream)
        e3 = ev()
        if record is not None:
            record.append((e0, e1, e2, e3, syrk_ev))

    if args.copy_probe:
        src = torch.empty((1 << 30) // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()

    recs = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(recs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert int(info.item()) == 0, "factorization failed"

    ms_step = wall * 1e3 / args.steps
    hess_ms = [r[0].elapsed_time(r[1]) for r in recs]
    prep_ms = [r[1].elapsed_time(r[2]) for r in recs]
    quant_ms = [r[2].elapsed_time(r[3]) for r in recs]
    launch_ms = [a.elapsed_time(b) for r in recs for (a, b) in r[4]]
    mean = lambda v: sum(v) / len(v)
    syrk_flops_total = float(cfg.tokens) * n * (n + 1)
    hess_tflops = syrk_flops_total / (mean(hess_ms) * 1e-3) / 1e12
    syrk_launch_flops = float(chunk) * n * (n + 1)
    syrk_launch_ms = mean(launch_ms)
    achieved = syrk_launch_flops / (syrk_launch_ms * 1e-3) / 1e12
    weights = out * n
    layer_ms = mean(prep_ms) + mean(quant_ms)

    result = {
        "metric": METRIC,
        "value": weights / (ms_step * 1e-3),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 in, f32 accumulate",
        "data": "synthetic (seeded; stands in for c4 calibration text and Llama weights)",
        "config": {
            "workload": (f"{cfg.name}: GPTQ one layer W {out}x{n} fp16, calibration "
                         f"{cfg.samples}x{cfg.tokens_per_sample} tokens fp16, {cfg.bits}-bit "
                         f"{'sym' if cfg.sym else 'asym'} g{cfg.group_size}, desc_act="
                         f"{cfg.desc_act}, damp {cfg.damp}, block {cfg.block}"),
            "out": out, "in": n, "tokens": cfg.tokens, "bits": cfg.bits,
            "group_size": cfg.group_size, "desc_act": cfg.desc_act, "block": cfg.block,
            "chunk_tokens": chunk,
        },
        "hessian_tflops": hess_tflops,
        "stage_ms": {"hessian": mean(hess_ms), "prepare": mean(prep_ms),
                     "quantize": mean(quant_ms)},
        "layer_weights_per_s": weights / (layer_ms * 1e-3),
        "roofline": {
            "kernel": syrk_kernel_name(n),
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_FP16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_FP16_TFLOPS,
            "launch_ms": syrk_launch_ms,
            "flops_per_launch": syrk_launch_flops,
            "traffic": load_traffic("syrk.hip", cfg.name, chunk),
        },
    }
    del X, chunks
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(cfg, cfg.tokens)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
