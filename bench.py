"""Throughput of GPTQ layer quantization on one MI355X.

One step = the whole per-layer path on one batch of synthetic calibration
data already resident in HBM:
    H = 0; H += 2 X^T X over all calibration tokens (one
    gptq_hessian_accumulate call by default; --chunk-samples streams chunks)
    gptq_prepare (damp, desc_act order, U = chol(H_p^-1) upper)
    gptq_quantize_layer (sweep + lazy GEMMs + pack)
value = weights quantized per second = out * in / step time.

Default workload: the Llama-7B down_proj-shaped layer (W 4096 x 11008 fp16,
128 samples x 2048 tokens of heavy-tailed fp16 calibration activations,
4-bit asymmetric, group 128, desc_act, damp 0.01, block 128), the 4-bit g128
layer the throughput is reported on.  --config c1 / c2 select the 4096 x 4096
q_proj-shaped layer (4-bit, 3-bit desc_act), c4a / c4b the 8192 x 28672 70B
down_proj layer.

Prints ONE JSON line (rank 0; this build is single-GPU).

--dequant-tokens M times gptq_dequant_matmul instead (X of M fp16 tokens times
the config's packed layer, random codes) and prints one JSON line for it.

--summarize DIR (no GPU): turns the rocprofv3 output of the profiling
commands (DIR/trace, DIR/FETCH_SIZE, DIR/WRITE_SIZE, see PROFILE_COMMANDS)
into profiles/layer_<config>_kernel_stats.md and
profiles/syrk_<config>_traffic.json.
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
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 (vector and matrix)
METRIC = "GPTQ weights quantized/sec per layer (4-bit g128) + Hessian TFLOP/s, 1 GPU"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_sha(name: str) -> str:
    p = os.path.join(ROOT, "post_weight_quantization_12_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def load_traffic(kernel_file: str, workload: str, call_tokens: int):
    """HBM bytes per gptq_hessian_accumulate call from the committed rocprofv3
    --pmc summary, or None when there is none, it was taken with another call
    size, or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", f"syrk_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except ValueError:
        return None
    if d.get("source_sha") != kernel_source_sha(kernel_file):
        return None
    if d.get("call_tokens") != call_tokens:
        return None
    return float(d["hbm_bytes_per_call"])


def syrk_schedule(n: int, ntok: int, cus: int):
    """(kernels, launches) of one gptq_hessian_accumulate call with a
    workspace, following the library's choice (syrk.hip, launch_syrk): whole
    256 x 256 tiles (one launch per 32768 tokens) when they fill the
    workgroup rounds to 90 %, else the token-split schedule for calls of at
    least 256 stages of 32 tokens per token block, else stream-K."""
    nwg = min(max(cus // 8 * 8, 8), 512)
    nt = (n + 255) // 256
    tiles = nt * (nt + 1) // 2
    nk = (ntok + 31) // 32
    rounds = (tiles + nwg - 1) // nwg
    if 10 * tiles < 9 * rounds * nwg:
        blocks = 1
        while blocks < 8 and tiles * blocks // 8 < 4 * (nwg // 8):
            blocks *= 2
        if nk // blocks >= 256:
            return (f"syrk_dma_kernel + syrk_ksplit_fixup (token split, {blocks} blocks)", 1)
        if 4 * tiles < 3 * nwg:
            return ("syrk_dma_kernel + syrk_streamk_fixup (stream-K)", 1)
    launches = (ntok + 32767) // 32768
    return (f"syrk_dma_kernel (whole tiles, {launches} launches of <= 32768 tokens)", launches)


PROFILE_COMMANDS = {
    "trace": ("rocprofv3 --kernel-trace --stats -T -d {d}/trace -o t --output-format csv -- "
              "python -u bench.py --config {c} --steps 2 --warmup 1 --no-cpu-baseline"),
    "FETCH_SIZE": ("rocprofv3 --pmc FETCH_SIZE -T -d {d}/FETCH_SIZE -o p --output-format csv -- "
                   "python -u bench.py --config {c} --steps 1 --warmup 1 --no-cpu-baseline "
                   "--copy-probe"),
    "WRITE_SIZE": ("rocprofv3 --pmc WRITE_SIZE -T -d {d}/WRITE_SIZE -o p --output-format csv -- "
                   "python -u bench.py --config {c} --steps 1 --warmup 1 --no-cpu-baseline "
                   "--copy-probe"),
}


DEQUANT_PROFILE_COMMANDS = {
    "trace": ("rocprofv3 --kernel-trace --stats -T -d {d}/trace -o t --output-format csv -- "
              "python -u bench.py --config {c} --dequant-tokens {m} --steps 2 --warmup 1 "
              "--no-cpu-baseline"),
    "FETCH_SIZE": ("rocprofv3 --pmc FETCH_SIZE -T -d {d}/FETCH_SIZE -o p --output-format csv -- "
                   "python -u bench.py --config {c} --dequant-tokens {m} --steps 1 --warmup 1 "
                   "--no-cpu-baseline --copy-probe"),
    "WRITE_SIZE": ("rocprofv3 --pmc WRITE_SIZE -T -d {d}/WRITE_SIZE -o p --output-format csv -- "
                   "python -u bench.py --config {c} --dequant-tokens {m} --steps 1 --warmup 1 "
                   "--no-cpu-baseline --copy-probe"),
}
DQ_KERNELS = ("dq_small_kernel", "dq_reduce_kernel", "dq_mfma_kernel", "dq_tile_kernel",
              "dq_chunk_group_kernel", "dq_gather_x_kernel", "dq_gather_x_cols_kernel")


def _dq_kernel(name: str) -> bool:
    return any(k in name for k in DQ_KERNELS)


def load_dequant_traffic(cfg_name: str, M: int):
    """HBM bytes per gptq_dequant_matmul call from the committed rocprofv3
    summary, or None when there is none or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", f"dequant_{cfg_name}_m{M}_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except ValueError:
        return None
    if d.get("source_sha") != kernel_source_sha("dequant_matmul.hip"):
        return None
    return float(d["hbm_bytes_per_call"])


def summarize_dequant(cfg_name: str, M: int, d: str):
    """profiles/dequant_<config>_m<M>_kernel_stats.md and _traffic.json from
    the DEQUANT_PROFILE_COMMANDS output in d."""
    import csv
    import workloads
    cfg = workloads.get(cfg_name)
    tag = f"dequant_{cfg_name}_m{M}"
    shape = (f"X {M} x {cfg.inp} fp16, packed W {cfg.out}x{cfg.inp} {cfg.bits}-bit "
             f"g{cfg.group_size}" + (", group-ordered (desc_act layer)" if cfg.desc_act else ""))
    trace = list(csv.DictReader(open(os.path.join(d, "trace", "t_kernel_trace.csv"))))
    stats = {}
    for r in trace:
        name = r["Kernel_Name"]
        if not _dq_kernel(name):
            continue
        name = next(k for k in DQ_KERNELS if k in name)
        stats.setdefault(name, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    lines = [f"# rocprofv3 kernel statistics: gptq_dequant_matmul, {cfg_name} ({shape})", "",
             "Command (run from the repository root on one MI355X):", "",
             "    " + DEQUANT_PROFILE_COMMANDS["trace"].format(d=d, c=cfg_name, m=M), "",
             "All calls of the run (50 warm-up and 2 x 50 timed calls, back to back).", "",
             "| kernel | calls | avg us | min us | max us |", "|---|---:|---:|---:|---:|"]
    for name, ds in sorted(stats.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| {name} | {len(ds)} | {sum(ds) / len(ds) / 1e3:.2f} | "
                     f"{min(ds) / 1e3:.2f} | {max(ds) / 1e3:.2f} |")
    with open(os.path.join(ROOT, "profiles", f"{tag}_kernel_stats.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    GiB = 1 << 30
    per = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        rows = list(csv.DictReader(open(os.path.join(d, ctr, "p_counter_collection.csv"))))
        # per call: the main kernel's dispatches count the calls
        calls = sum(1 for r in rows if ("dq_small_kernel" in r["Kernel_Name"]
                                        or "dq_mfma_kernel" in r["Kernel_Name"]
                                        or "dq_tile_kernel" in r["Kernel_Name"]))
        tot = sum(float(r["Counter_Value"]) for r in rows if _dq_kernel(r["Kernel_Name"]))
        copy = max(float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"])
        per[ctr] = (tot / calls, copy)
    ff = (GiB / 1024) / per["FETCH_SIZE"][1]
    wf = (GiB / 1024) / per["WRITE_SIZE"][1]
    hbm = per["FETCH_SIZE"][0] * 1024 * ff + per["WRITE_SIZE"][0] * 1024 * wf
    gs = cfg.inp if cfg.group_size == -1 else cfg.group_size
    G = -(-cfg.inp // gs)
    alg = (cfg.inp * cfg.bits // 8 * cfg.out + 8 * G * cfg.out + 4 * cfg.inp + 2 * M * cfg.inp
           + 2 * M * cfg.out + (4 * cfg.inp if cfg.desc_act else 0))
    out = {
        "source": "post_weight_quantization_12_amd/csrc/dequant_matmul.hip",
        "source_sha": kernel_source_sha("dequant_matmul.hip"),
        "workload": f"{cfg_name}: {shape}",
        "commands": [DEQUANT_PROFILE_COMMANDS[c].format(d=d, c=cfg_name, m=M)
                     for c in ("FETCH_SIZE", "WRITE_SIZE")],
        "counted": "all dequant kernels of the run, divided by the number of calls",
        "fetch_kib_per_call": round(per["FETCH_SIZE"][0], 1),
        "write_kib_per_call": round(per["WRITE_SIZE"][0], 1),
        "copy_probe": {"kernel": "__amd_rocclr_copyBuffer (torch device copy of 1 GiB)",
                       "fetch_kib": round(per["FETCH_SIZE"][1], 1),
                       "write_kib": round(per["WRITE_SIZE"][1], 1)},
        "fetch_factor": round(ff, 4), "write_factor": round(wf, 4),
        "hbm_bytes_per_call": int(hbm),
        "algorithmic_bytes_per_call": alg,
        "traffic_over_algorithmic": round(hbm / alg, 2),
    }
    with open(os.path.join(ROOT, "profiles", f"{tag}_traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def _kernel_base_name(name: str) -> str:
    """The kernel's identifier: mangled names of this library's templated or
    anonymous-namespace kernels (_ZN4gptq12_GLOBAL__N_1<len><name>...) are cut
    to <name>."""
    import re
    m = re.match(r"_ZN4gptq12_GLOBAL__N_1(\d+)", name)
    if m:
        n = int(m.group(1))
        return name[m.end():m.end() + n]
    return name.split("(")[0].replace("void ", "")[:60]


BLOCK_PROFILE_COMMAND = ("rocprofv3 --kernel-trace --stats -T -d {d}/trace -o t --output-format csv "
                         "-- python -u bench.py --{mode} --steps 1 --warmup 1 --no-cpu-baseline")
BLOCK_TITLES = {
    "block": ("block_mlp_kernel_stats.md", 3,
              "bench.py --block (Llama-7B MLP block, d 4096, inter 11008, 4-bit g128 asym, "
              "desc_act on, 128 x 2048 calibration tokens)"),
    "decoder": ("decoder_block_kernel_stats.md", 7,
                "bench.py --decoder (Llama-7B decoder block: q, k, v, o 4096 x 4096 with 32 "
                "heads of 128, gate, up, down 4096 / 11008, 4-bit g128 asym, desc_act on, 128 "
                "sequences of 2048 tokens)"),
}


def summarize_block(d: str, mode: str = "block"):
    """profiles/<block|decoder>_..._kernel_stats.md from the
    BLOCK_PROFILE_COMMAND trace in d: per-kernel statistics of the timed
    step (the second of two)."""
    import csv
    fname, layers, title = BLOCK_TITLES[mode]
    trace = list(csv.DictReader(open(os.path.join(d, "trace", "t_kernel_trace.csv"))))
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    # each step packs every layer once: the warm-up step ends with its last pack
    packs = [int(r["End_Timestamp"]) for r in trace if r["Kernel_Name"].startswith("pack_kernel")]
    first = packs[layers - 1] if len(packs) >= 2 * layers else 0
    k = sum(1 for r in trace if int(r["Start_Timestamp"]) < first)
    stats = {}
    span = [None, None]
    for r in trace:
        t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        if t0 < first:
            continue
        name = _kernel_base_name(r["Kernel_Name"])
        stats.setdefault(name, []).append(t1 - t0)
        span = [t0 if span[0] is None else min(span[0], t0), t1 if span[1] is None else max(span[1], t1)]
    lines = ["# rocprofv3 kernel statistics: " + title, "",
             "Command (run from the repository root on one MI355X):", "",
             "    " + BLOCK_PROFILE_COMMAND.format(d=d, mode=mode), "",
             f"The timed step only ({(span[1] - span[0]) / 1e6:.1f} ms from its first kernel "
             f"to its last under the profiler; {k} earlier launches belong to the warm-up).", "",
             "| kernel | calls | total ms | avg us |", "|---|---:|---:|---:|"]
    for name, ds in sorted(stats.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| {name} | {len(ds)} | {sum(ds) / 1e6:.3f} | {sum(ds) / len(ds) / 1e3:.2f} |")
    with open(os.path.join(ROOT, "profiles", fname), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


MFMA_COUNTERS = "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_BUSY_CYCLES GRBM_GUI_ACTIVE"
MFMA_PROFILE_COMMAND = ("rocprofv3 --pmc " + MFMA_COUNTERS + " -T -d {d}/MFMA -o p "
                        "--output-format csv -- python -u bench.py --config {c} --steps 1 "
                        "--warmup 1 --no-cpu-baseline")


def summarize_mfma(cfg_name: str, d: str):
    """profiles/layer_<config>_mfma_counters.md from the MFMA_PROFILE_COMMAND
    run in d/MFMA: per kernel family of the timed step (the run's second),
    the matrix cores' busy fraction, the fp16 MFMA work issued and the shader
    clock.  The counters come summed over the 8 XCDs (GRBM_GUI_ACTIVE: 8 x the
    active cycles) and the 1024 SIMDs (SQ_VALU_MFMA_BUSY_CYCLES)."""
    import csv
    rows = list(csv.DictReader(open(os.path.join(d, "MFMA", "p_counter_collection.csv"))))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    syrk_ids = sorted({int(r["Dispatch_Id"]) for r in rows
                       if r["Kernel_Name"].startswith("syrk_dma_kernel")})
    first = syrk_ids[len(syrk_ids) // 2] if syrk_ids else 0
    fam = {}
    phase = "prepare"
    for r in rows:
        did = int(r["Dispatch_Id"])
        if did < first:
            continue
        k = _kernel_base_name(r["Kernel_Name"])
        if k.startswith("gather_w_kernel"):
            phase = "quantize"
        if k.startswith("syrk_"):
            phase = "prepare"
        name = k + (" (" + phase + ")" if k == "gemm_f32_dma" else "")
        f = fam.setdefault(name, {"dur": {}, "busy": 0.0, "mops": 0.0, "gui": 0.0})
        f["dur"][did] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        v = float(r["Counter_Value"])
        key = {"SQ_VALU_MFMA_BUSY_CYCLES": "busy", "SQ_INSTS_VALU_MFMA_MOPS_F16": "mops",
               "GRBM_GUI_ACTIVE": "gui"}.get(r["Counter_Name"])
        if key:
            f[key] += v
    xcd, simds = 8, 1024
    lines = [f"# rocprofv3 matrix-core counters: bench.py --config {cfg_name}", "",
             "Command (run from the repository root on one MI355X):", "",
             "    " + MFMA_PROFILE_COMMAND.format(d=d, c=cfg_name), "",
             "Per kernel family, the dispatches of the run's timed step; time = the sum of the "
             "dispatches' durations under the counters (kernels of the factorization overlap on "
             "three streams).  Active cycles = GRBM_GUI_ACTIVE / 8 XCDs; MFMA util = "
             "SQ_VALU_MFMA_BUSY_CYCLES / (active cycles x 1024 SIMDs); fp16 MFMA work issued = "
             "SQ_INSTS_VALU_MFMA_MOPS_F16 x 512 (gemm_eh_dma issues two fp16 products per "
             "algorithmic one over 512 or more error columns in layers up to 16384 wide, three "
             "otherwise; gemm_f32_dma with split operands three); clock = "
             "active cycles / time, given for the SYRK only: it runs long and alone on the GPU, "
             "while for short or overlapping dispatches the counting window is wider than the "
             "kernel.", "",
             "| kernel | dispatches | ms | MFMA util | fp16 MFMA TFLOP issued | issued TFLOP/s | "
             "clock GHz |", "|---|---:|---:|---:|---:|---:|---:|"]
    for name, f in sorted(fam.items(), key=lambda kv: -kv[1]["busy"]):
        if f["busy"] <= 0 and f["mops"] <= 0:
            continue
        t = sum(f["dur"].values()) * 1e-9
        act = f["gui"] / xcd
        util = f["busy"] / max(act * simds, 1.0)
        fl = f["mops"] * 512
        clock = f"{act / t / 1e9:.2f}" if name.startswith("syrk_") else ""
        lines.append(f"| {name} | {len(f['dur'])} | {t * 1e3:.3f} | {util:.3f} | {fl / 1e12:.3f} | "
                     f"{fl / t / 1e12:.0f} | {clock} |")
    with open(os.path.join(ROOT, "profiles", f"layer_{cfg_name}_mfma_counters.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize(cfg_name: str, d: str):
    """Write the profiles/ summaries from rocprofv3 CSV output in d (the
    PROFILE_COMMANDS run with the default call size).  FETCH_SIZE and
    WRITE_SIZE are scaled by what they read for the 1 GiB device copy that
    --copy-probe runs (a kernel of known traffic)."""
    import csv
    import workloads
    cfg = workloads.get(cfg_name)
    n = cfg.inp
    shape = (f"W {cfg.out}x{n}, {cfg.bits}-bit g{cfg.group_size}, desc_act "
             f"{'on' if cfg.desc_act else 'off'}")
    # Per-kernel statistics over the two timed steps only: the warm-up step
    # also pays one-time costs (its first SYRK call ran 3.5x longer under
    # the profiler), which the timed steps never see.
    trace = list(csv.DictReader(open(os.path.join(d, "trace", "t_kernel_trace.csv"))))
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    syrk_starts = [int(r["Start_Timestamp"]) for r in trace
                   if r["Kernel_Name"].startswith("syrk_dma_kernel")]
    per_step = len(syrk_starts) // 3
    t_timed = syrk_starts[per_step]
    stats = {}
    for r in trace:
        if int(r["Start_Timestamp"]) < t_timed:
            continue
        name = _kernel_base_name(r["Kernel_Name"])
        dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        stats.setdefault(name, []).append(dur)
    lines = [f"# rocprofv3 kernel statistics: bench.py --config {cfg_name} ({shape})", "",
             "Command (run from the repository root on one MI355X):", "",
             "    " + PROFILE_COMMANDS["trace"].format(d=d, c=cfg_name), "",
             "Statistics over the 2 timed steps (from the kernel trace; the warm-up step is",
             "left out), one gptq_hessian_accumulate call over all "
             f"{cfg.tokens} calibration tokens per step.", "",
             "| kernel | calls | total ms | avg us | min us | max us |",
             "|---|---:|---:|---:|---:|---:|"]
    for name, ds in sorted(stats.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| {name} | {len(ds)} | {sum(ds) / 1e6:.3f} | {sum(ds) / len(ds) / 1e3:.2f} | "
                     f"{min(ds) / 1e3:.2f} | {max(ds) / 1e3:.2f} |")
    timed = [r for r in trace if int(r["Start_Timestamp"]) >= t_timed]
    lines += ["", "## Per-stage roofline (timed steps, mean per step)", ""] + stage_roofline(
        cfg, timed)
    lines += ["", "## HBM traffic per stage (rocprofv3 FETCH_SIZE + WRITE_SIZE)", ""] + \
        stage_traffic(cfg, d, timed)
    with open(os.path.join(ROOT, "profiles", f"layer_{cfg_name}_kernel_stats.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    GiB = 1 << 30
    per = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        rows = list(csv.DictReader(open(os.path.join(d, ctr, "p_counter_collection.csv"))))
        # the timed call: its SYRK dispatches follow the warm-up call's
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        ids = [int(r["Dispatch_Id"]) for r in rows if r["Kernel_Name"].startswith("syrk_dma_kernel")]
        first = ids[len(ids) // 2]
        syrk = collections_sum([r for r in rows if int(r["Dispatch_Id"]) >= first],
                               lambda k: k.startswith("syrk_"))
        copy = max(float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"])
        per[ctr] = (syrk, copy)
    ff = (GiB / 1024) / per["FETCH_SIZE"][1]
    wf = (GiB / 1024) / per["WRITE_SIZE"][1]
    fetch_b = per["FETCH_SIZE"][0][0] * 1024 * ff
    write_b = per["WRITE_SIZE"][0][0] * 1024 * wf
    alg = cfg.tokens * n * 2 + 2 * (n * (n + 1) // 2) * 4
    out = {
        "kernels": per["FETCH_SIZE"][0][1],
        "source": "post_weight_quantization_12_amd/csrc/syrk.hip",
        "source_sha": kernel_source_sha("syrk.hip"),
        "workload": f"{cfg_name}: {shape}; X {cfg.samples}x{cfg.tokens_per_sample} tokens fp16",
        "call_tokens": cfg.tokens,
        "commands": [PROFILE_COMMANDS[c].format(d=d, c=cfg_name)
                     for c in ("FETCH_SIZE", "WRITE_SIZE")],
        "counted": "the SYRK dispatches of the timed call (the second; the first is warm-up)",
        "fetch_kib_per_call": round(per["FETCH_SIZE"][0][0], 1),
        "write_kib_per_call": round(per["WRITE_SIZE"][0][0], 1),
        "copy_probe": {"kernel": "__amd_rocclr_copyBuffer (torch device copy of 1 GiB)",
                       "bytes_read": GiB, "bytes_written": GiB,
                       "fetch_kib": round(per["FETCH_SIZE"][1], 1),
                       "write_kib": round(per["WRITE_SIZE"][1], 1)},
        "fetch_factor": round(ff, 4), "write_factor": round(wf, 4),
        "hbm_bytes_per_call": int(fetch_b + write_b),
        "algorithmic_bytes_per_call": alg,
        "traffic_over_algorithmic": round((fetch_b + write_b) / alg, 2),
    }
    with open(os.path.join(ROOT, "profiles", f"syrk_{cfg_name}_traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


# Stages of the layer path and their kernels (base names as rocprofv3 -T
# prints them; templated kernels keep a mangled name, matched by substring).
STAGES = [
    ("a1 Hessian SYRK", ("syrk_",)),
    ("a2 damp / order / gather", ("diag_stats_kernel", "rank_count_kernel", "rank_scatter_kernel",
                                  "symmetrize_kernel", "scale_kernel", "gather_kernel",
                                  "fill_f32_kernel", "gather_w_kernel")),
    ("a3 factor (Cholesky + inverse, U')", ("cholinv_leaf_kernel", "reverse_inplace_kernel",
                                             "gemm_f32_dma@prepare")),
    ("a4 block sweep", ("sweep16_kernel", "sweep16_pair_kernel", "sweep_kernel")),
    ("a5 lazy trailing update", ("gemm_eh_dma", "uprime_split_kernel", "gemm_f32_dma@quantize")),
    ("a6 pack", ("pack_kernel", "perm_tables_kernel")),
]


def sweep_pairs(cfg):
    """Pairs of adjacent full 128-column blocks the quantize recursion sweeps
    in one kernel (both halves of a two-block range; the recursion splits on
    pair boundaries), for this layer."""
    B, n = cfg.block, cfg.inp
    gs = cfg.group_size if cfg.group_size > 0 else 0
    if B != 128 or gs not in (0, 16, 32, 64, 128) or n <= B:
        return 0

    def rec(a, b):
        if b - a <= B:
            return 0
        if b - a == 2 * B:
            return 1
        nblk = (b - a + B - 1) // B
        m = a + B * ((nblk + 1) // 2)
        mp = a + 2 * B * (((nblk + 1) // 2 + 1) // 2)  # split on pair boundaries
        if mp < b:
            m = mp
        return rec(a, m) + rec(m, b)
    return rec(0, n)


def stage_roofline(cfg, rows):
    """Markdown lines: per stage, the summed kernel time per step, the
    algorithmic work and its fraction of the stage's bound.  gemm_f32_dma
    belongs to a3 before the step's first gather_w_kernel (prepare) and to a5
    after it (quantize).  The factorization runs on three streams, so its
    wall time (first start to last end per step) is given too."""
    n, out, b, gs = cfg.inp, cfg.out, cfg.bits, cfg.group_size
    gs = n if gs == -1 else gs
    rows = sorted(rows, key=lambda r: int(r["Start_Timestamp"]))
    steps = sum(1 for r in rows if r["Kernel_Name"].startswith("syrk_dma_kernel")) or 1
    if cfg.tokens > 32768 and steps > 2:  # whole tiles: one launch per 32768 tokens
        steps = max(1, steps // ((cfg.tokens + 32767) // 32768))
    tot = {name: 0 for name, _ in STAGES}
    a3_wall = 0
    phase = "prepare"
    a3_span = None
    for r in rows:
        k = r["Kernel_Name"]
        t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        if k.startswith("syrk_dma_kernel"):
            phase = "prepare"
            if a3_span:
                a3_wall += a3_span[1] - a3_span[0]
                a3_span = None
        if "gather_w_kernel" in k:
            phase = "quantize"
        key = "gemm_f32_dma@" + phase if k.startswith("gemm_f32_dma") else k
        for name, ks in STAGES:
            if any(x in key for x in ks):
                tot[name] += t1 - t0
                if name.startswith("a3"):
                    a3_span = [t0, t1] if a3_span is None else [min(a3_span[0], t0),
                                                               max(a3_span[1], t1)]
                break
    if a3_span:
        a3_wall += a3_span[1] - a3_span[0]
    # the update of each pair of adjacent 128-column blocks (2 out B^2 flop)
    # runs inside the pair's sweep kernel (a4); a5 counts the GEMMs' share
    a5_flop = float(out) * n * (n - cfg.block) - sweep_pairs(cfg) * 2.0 * out * cfg.block ** 2
    work = {
        "a1 Hessian SYRK": (float(cfg.tokens) * n * (n + 1), "flop", "fp16 MFMA", PEAK_FP16_TFLOPS * 1e12),
        "a2 damp / order / gather": (8.0 * n * n + 6.0 * out * n, "B", "HBM", PEAK_HBM_GBS * 1e9),
        "a3 factor (Cholesky + inverse, U')": (2.0 * n ** 3 / 3, "flop", "fp32 (split-fp16 MFMA)",
                                               PEAK_FP32_TFLOPS * 1e12),
        "a4 block sweep": (7.0 * out * n + 8.0 * out * n / gs, "B", "HBM (latency-bound)",
                           PEAK_HBM_GBS * 1e9),
        "a5 lazy trailing update": (a5_flop, "flop", "fp16 MFMA", PEAK_FP16_TFLOPS * 1e12),
        "a6 pack": (out * n * (1 + b / 8.0), "B", "HBM", PEAK_HBM_GBS * 1e9),
    }
    lines = ["| stage | kernel ms | algorithmic work | achieved | bound | frac | MFMA pipe |",
             "|---|---:|---:|---:|---|---:|---:|"]
    for name, _ in STAGES:
        t = tot[name] / steps * 1e-9
        w, unit, bound, peak = work[name]
        if t <= 0:
            continue
        ach = w / t
        shown = f"{ach / 1e12:.1f} TFLOP/s" if unit == "flop" else f"{ach / 1e9:.0f} GB/s"
        wshown = f"{w:.3g} {unit}"
        # the trailing GEMMs over >= 512 error columns (nearly all the work)
        # multiply the errors as two fp16 parts by U' in fp16 (two fp16 MFMA
        # products per algorithmic one), above 16384 columns by U' and its
        # fp16 remainder (three)
        prods = 3 if n > 16384 else 2
        pipe = f"{prods * ach / (PEAK_FP16_TFLOPS * 1e12):.3f}" if name.startswith("a5") else ""
        lines.append(f"| {name} | {t * 1e3:.3f} | {wshown} | {shown} | {bound} | "
                     f"{ach / peak:.3f} | {pipe} |")
    lines.append("")
    lines.append(f"a3 wall time per step (first start to last end; its kernels run on three "
                 f"streams): {a3_wall / steps / 1e6:.3f} ms, "
                 f"{2.0 * n ** 3 / 3 / (a3_wall / steps * 1e-9) / 1e12:.1f} TFLOP/s.")
    lines.append("Peaks: fp16 MFMA 2.5 PFLOP/s, fp32 157.3 TFLOP/s, HBM 8 TB/s. Work per "
                 "stage: a1 N n(n+1), a2 8 n^2 + 6 out in bytes, a3 2 n^3 / 3, a4 "
                 "7 out in + 8 out in / gs bytes, a5 out in (in - B) less 2 out B^2 per pair of "
                 "adjacent blocks swept by one kernel (" + str(sweep_pairs(cfg)) + " pairs; their "
                 "update runs in a4), a6 out in (1 + b/8) bytes. "
                 "MFMA pipe: fp16 MFMA work actually issued (" +
                 ("three" if n > 16384 else "two") + " products per algorithmic one in the "
                 "trailing GEMMs) over the fp16 peak.")
    return lines


def _stage_of(kernel_base: str, phase: str):
    key = "gemm_f32_dma@" + phase if kernel_base.startswith("gemm_f32_dma") else kernel_base
    for name, ks in STAGES:
        if any(x in key for x in ks):
            return name
    return None


def stage_traffic(cfg, d, timed_trace):
    """Markdown lines: per stage, the HBM bytes the counters saw in the timed
    step (the second step of the FETCH_SIZE / WRITE_SIZE runs; each counter
    scaled by what it reads for a 1 GiB copy) and those bytes over the
    stage's kernel time per step from the trace."""
    import csv
    GiB = 1 << 30
    tot = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        rows = list(csv.DictReader(open(os.path.join(d, ctr, "p_counter_collection.csv"))))
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        ids = [int(r["Dispatch_Id"]) for r in rows if r["Kernel_Name"].startswith("syrk_dma_kernel")]
        first = ids[len(ids) // 2] if ids else 0
        copy = max(float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"])
        factor = (GiB / 1024) / copy
        phase = "prepare"
        for r in rows:
            if int(r["Dispatch_Id"]) < first:
                continue
            k = _kernel_base_name(r["Kernel_Name"])
            if k.startswith("gather_w_kernel"):
                phase = "quantize"
            if k.startswith("syrk_"):
                phase = "prepare"
            st = _stage_of(k, phase)
            if st:
                tot.setdefault(st, [0.0, 0.0])[0 if ctr == "FETCH_SIZE" else 1] += \
                    float(r["Counter_Value"]) * 1024 * factor
    # kernel time per stage and step (as in the roofline table)
    steps = sum(1 for r in timed_trace if r["Kernel_Name"].startswith("syrk_dma_kernel")) or 1
    if cfg.tokens > 32768 and steps > 2:
        steps = max(1, steps // ((cfg.tokens + 32767) // 32768))
    tt = {}
    phase = "prepare"
    for r in sorted(timed_trace, key=lambda r: int(r["Start_Timestamp"])):
        k = _kernel_base_name(r["Kernel_Name"])
        if k.startswith("gather_w_kernel"):
            phase = "quantize"
        if k.startswith("syrk_"):
            phase = "prepare"
        st = _stage_of(k, phase)
        if st:
            tt[st] = tt.get(st, 0) + int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    lines = ["| stage | fetched MB | written MB | kernel ms | measured HBM GB/s | frac of 8 TB/s |",
             "|---|---:|---:|---:|---:|---:|"]
    for name, _ in STAGES:
        if name not in tot or name not in tt:
            continue
        f, w = tot[name]
        t = tt[name] / steps * 1e-9
        lines.append(f"| {name} | {f / 1e6:.1f} | {w / 1e6:.1f} | {t * 1e3:.3f} | "
                     f"{(f + w) / t / 1e9:.0f} | {(f + w) / t / 1e9 / PEAK_HBM_GBS:.3f} |")
    lines.append("")
    lines.append("FETCH_SIZE counts L2 misses sent to the memory side (some are served by the "
                 "Infinity Cache), so these are upper bounds on DRAM bytes.")
    return lines


def collections_sum(rows, pick):
    """(sum of Counter_Value over the dispatches whose kernel name matches,
    {kernel: dispatches})."""
    total, names = 0.0, {}
    for r in rows:
        k = r["Kernel_Name"].strip()  # base names (rocprofv3 -T)
        if pick(k):
            total += float(r["Counter_Value"])
            names[k] = names.get(k, 0) + 1
    return total, names


def host_description() -> dict:
    """The host the CPU baseline runs on: CPU model, the cores this process
    may use, and the BLAS library NumPy calls with its thread count."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas, threads = None, None
    try:
        import numpy  # noqa: F401  (loads the BLAS library)
        from threadpoolctl import threadpool_info
        for lib in threadpool_info():
            if lib.get("user_api") == "blas":
                blas = f"{lib.get('internal_api')} {lib.get('version')}"
                threads = lib.get("num_threads")
                break
    except Exception:
        pass
    return {"cpu_model": model, "allowed_cores": len(os.sched_getaffinity(0)),
            "os_cpu_count": os.cpu_count(), "blas": blas, "blas_threads": threads}


def cpu_baseline(cfg, steps_tokens: int):
    """The oracle, untuned, on a bounded sample of the same workload:
    Hessian over one 2048-token sample, the full prepare at the layer's n,
    and the sweep of 32 output rows; scaled to the whole layer."""
    import numpy as np
    import torch

    import oracle as O
    import workloads

    torch.set_num_threads(max(1, len(os.sched_getaffinity(0))))
    host = host_description()
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
        "cores": host["blas_threads"] or len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "host": host,
        "sample": (f"Hessian over 1 of {cfg.samples} samples ({X.shape[0]} tokens, "
                   f"{t_h:.2f} s, scaled x{steps_tokens // X.shape[0]}); full prepare at "
                   f"n={cfg.inp} ({t_p:.2f} s); sweep+pack of {rows} of {cfg.out} rows "
                   f"({t_s:.2f} s, scaled x{cfg.out // rows}); fp64 NumPy"),
        "sample_seconds": round(t_h + t_p + t_s, 2),
    }


def layer_roofline(cfg, hess_ms: float, prep_ms: float, quant_ms: float) -> dict:
    """Whole-layer roofline: the sum of the stages' ideal times at their
    bounds (a1 N n(n+1) flop and a5 out in (in - B) flop at the fp16 MFMA
    peak, a3 2 n^3 / 3 flop at the fp32 peak, a2 8 n^2 + 6 out in, a4
    7 out in + 8 out in / gs and a6 out in (1 + b/8) bytes at the HBM peak)
    over the measured time, with and without the Hessian."""
    n, out, b = cfg.inp, cfg.out, cfg.bits
    gs = n if cfg.group_size == -1 else cfg.group_size
    f16, f32, hbm = PEAK_FP16_TFLOPS * 1e12, PEAK_FP32_TFLOPS * 1e12, PEAK_HBM_GBS * 1e9
    ideal = {
        "a1": float(cfg.tokens) * n * (n + 1) / f16,
        "a2": (8.0 * n * n + 6.0 * out * n) / hbm,
        "a3": 2.0 * n ** 3 / 3 / f32,
        "a4": (7.0 * out * n + 8.0 * out * n / gs) / hbm,
        "a5": float(out) * n * (n - cfg.block) / f16,
        "a6": out * n * (1 + b / 8.0) / hbm,
    }
    t_layer = sum(v for k, v in ideal.items() if k != "a1")
    t_all = t_layer + ideal["a1"]
    return {
        "ideal_ms": {k: v * 1e3 for k, v in ideal.items()},
        "layer_ideal_ms": t_layer * 1e3,
        "layer_ms": prep_ms + quant_ms,
        "layer_frac": t_layer * 1e3 / (prep_ms + quant_ms),
        "step_ideal_ms": t_all * 1e3,
        "step_ms": hess_ms + prep_ms + quant_ms,
        "step_frac": t_all * 1e3 / (hess_ms + prep_ms + quant_ms),
    }


def dequant_cpu_baseline(cfg, M, words, scales, zeros, g_idx, x):
    """The oracle's dequant_matmul, untuned, on a column sample of the layer
    (the first `cols` output columns, all M tokens), scaled to all columns."""
    import numpy as np
    import torch

    import oracle as O

    torch.set_num_threads(max(1, len(os.sched_getaffinity(0))))
    cols = min(cfg.out, max(64, (1 << 24) // cfg.inp))
    wn = words[:, :cols].cpu().numpy()
    sn = scales[:, :cols].cpu().numpy()
    zn = zeros[:, :cols].cpu().numpy()
    gn = g_idx.cpu().numpy()
    xn = x.cpu().numpy()
    t0 = time.perf_counter()
    O.dequant_matmul(xn, wn, sn, zn, gn, cfg.bits)
    t = (time.perf_counter() - t0) * cfg.out / cols
    return {
        "value": 2.0 * M * cfg.inp * cfg.out / t / 1e12,
        "unit": "TFLOP/s",
        "cores": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": (f"{cols} of {cfg.out} output columns, all {M} tokens "
                   f"({t * cols / cfg.out:.2f} s, scaled x{cfg.out / cols:.0f}); fp64 NumPy"),
    }


def dequant_main(args):
    """--dequant-tokens M: gptq_dequant_matmul Y = X W^T (X fp16 [M x in], the
    packed layer of the config's shape and bit width, Y fp16) timed on its own.
    Roofline: HBM for M <= 8 (algorithmic bytes = packed words + scales +
    zeros + g_idx + X + Y), fp16 MFMA above (2 M in out flop)."""
    import torch

    import post_weight_quantization_12_amd as P
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = workloads.get(args.config)
    M, n, out = args.dequant_tokens, cfg.inp, cfg.out
    gs = n if cfg.group_size == -1 else cfg.group_size
    words, scales, zeros, order = workloads.packed_layer_draws(cfg, dev, 0)
    g_idx = torch.empty((n,), dtype=torch.int32, device=dev)
    g_idx[order] = (torch.arange(n, device=dev) // gs).to(torch.int32)  # group of a column
    gx = workloads.generator(dev, 0, cfg.cfg_id, 6, M)
    X = torch.randn((M, n), generator=gx, device=dev).to(torch.float16)
    Y = torch.empty((M, out), dtype=torch.float16, device=dev)
    wsb = P.dequant_matmul_workspace_bytes(M, n, out)
    ws = torch.empty((max(wsb, 1),), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    log(f"[bench] dequant_matmul {cfg.name}: X {M}x{n} fp16, packed W {out}x{n} "
        f"{cfg.bits}-bit g{cfg.group_size} desc_act={cfg.desc_act}, Y fp16")

    x_order = None
    order_ms = None
    if cfg.desc_act and not args.dequant_as_packed:
        # act-order layer: re-ordered by group once, as at load time
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        words, g_idx, x_order = P.dequant_group_order(words, g_idx, cfg.bits, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        order_ms = a.elapsed_time(b)
        wsb = P.dequant_matmul_workspace_bytes(M, n, out, True)
        ws = torch.empty((max(wsb, 1),), dtype=torch.uint8, device=dev)

    def call():
        P.dequant_matmul(X, words, scales, zeros, g_idx, cfg.bits, x_order=x_order, Y=Y,
                         workspace=ws if wsb else None, stream=stream)

    if args.copy_probe:
        src = torch.empty((1 << 30) // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    reps = 50
    for _ in range(args.warmup * reps):
        call()
    torch.cuda.synchronize()
    evs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            call()
        b.record(stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = sum(a.elapsed_time(b) for a, b in evs) / (args.steps * reps)

    # the same product with dense fp16 weights (hipBLASLt through torch), for context
    Wd = torch.randn((out, n), device=dev).to(torch.float16)
    for _ in range(reps):
        torch.matmul(X, Wd.t())
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        torch.matmul(X, Wd.t())
    b.record(stream)
    torch.cuda.synchronize()
    dense_ms = a.elapsed_time(b) / reps
    del Wd

    flops = 2.0 * M * n * out
    G = scales.shape[0]
    alg_bytes = float(n * cfg.bits // 8 * out + 8 * G * out + 4 * n + 2 * M * n + 2 * M * out
                      + (4 * n if x_order is not None else 0))
    small = M <= 8   # the library's few-token kernel
    if small:
        achieved, peak, unit, bound = alg_bytes / (call_ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s", "hbm"
        kernel = ("dq_small_kernel" + (" + dq_reduce_kernel" if wsb else ""))
    else:
        achieved, peak, unit, bound = flops / (call_ms * 1e-3) / 1e12, PEAK_FP16_TFLOPS, "TFLOP/s", "mfma"
        # from 256 tokens (out % 4 == 0, aligned weights): the 256 x 256 tiles
        tiles = ("dq_chunk_group_kernel + dq_tile_kernel" if M >= 256 and out % 4 == 0
                 else "dq_mfma_kernel")
        kernel = (("dq_gather_x_kernel + " if x_order is not None else "") + tiles
                  + (" + dq_reduce_kernel (split input range)" if M < 256 or out % 4 else
                     " [+ dq_reduce_kernel when the input range is split]"))
    result = {
        "metric": "dequantize-on-the-fly matmul Y = X W^T from the packed layer, TFLOP/s",
        "value": flops / (call_ms * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "calls_per_step": reps,
        "us_per_call": call_ms * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 X, fp32 dequant + accumulate" if small else "f16 X and dequantized W, f32 accumulate",
        "data": "synthetic (seeded random codes, scales, zeros and column order)",
        "config": {
            "workload": (f"{cfg.name} packed layer: W {out}x{n} {cfg.bits}-bit g{cfg.group_size} "
                         f"desc_act={cfg.desc_act}, X {M} tokens fp16, Y fp16"),
            "tokens": M, "out": out, "in": n, "bits": cfg.bits, "group_size": cfg.group_size,
            "desc_act": cfg.desc_act,
            "layer": ("group-ordered (gptq_dequant_group_order, once)" if x_order is not None
                      else "as packed"),
        },
        "group_order_ms_once": order_ms,
        "dense_fp16_us_per_call": dense_ms * 1e3,
        "speedup_vs_dense_fp16": dense_ms / call_ms,
        "roofline": {
            "kernel": f"{kernel} = one gptq_dequant_matmul call",
            "kernel_launches_per_call": kernel.count("+") + 1,
            "bound": bound,
            "achieved": achieved,
            "peak": peak,
            "unit": unit,
            "frac": achieved / peak,
            "call_ms": call_ms,
            "bytes_per_call": alg_bytes,
            "flops_per_call": flops,
            "traffic": load_dequant_traffic(cfg.name, M),
        },
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = dequant_cpu_baseline(cfg, M, words, scales, zeros, g_idx, X)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def block_cpu_baseline(d, inter, bits, gs, sym, desc, X, Wg, Wu, Wd, samples):
    """The oracle on a bounded sample of the block: Hessians and the forward
    of one 2048-token sample (scaled to all samples), both factorizations in
    full, the sweeps of 32 rows of each layer (scaled to all rows); fp64."""
    import numpy as np
    import torch

    import oracle as O

    torch.set_num_threads(max(1, len(os.sched_getaffinity(0))))
    x = X[:2048].cpu().double().numpy()
    wg, wu, wd = (w.cpu().double().numpy() for w in (Wg, Wu, Wd))
    rows = 32
    t = {}
    t0 = time.perf_counter()
    H = O.hessian(x)
    t["hessian_in"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    Hd_, _ = O.condition(H, 0.01)
    perm = O.column_order(H, desc)
    U = O.hinv_chol(Hd_, perm)
    t["prepare_in"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.gptq_sweep(wg[:rows], U, perm, bits, gs, sym)
    t["sweep_gate"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    A = O.silu_mul(x @ wg.T, x @ wu.T)
    H2 = O.hessian(A)
    t["forward_hessian_down"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    Hd2, _ = O.condition(H2, 0.01)
    perm2 = O.column_order(H2, desc)
    U2 = O.hinv_chol(Hd2, perm2)
    t["prepare_down"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.gptq_sweep(wd[:rows], U2, perm2, bits, gs, sym)
    t["sweep_down"] = time.perf_counter() - t0
    full = ((t["hessian_in"] + t["forward_hessian_down"]) * samples + t["prepare_in"]
            + t["prepare_down"] + t["sweep_gate"] * 2 * inter / rows + t["sweep_down"] * d / rows)
    return {
        "value": 3.0 * d * inter / full,
        "unit": "weights/s",
        "cores": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": (f"one 2048-token sample for the Hessians and the forward (scaled x{samples}), "
                   f"both factorizations in full, 32-row sweeps (scaled to {inter}, {inter} and "
                   f"{d} rows); fp64 NumPy; "
                   + ", ".join(f"{k} {v:.2f} s" for k, v in t.items())),
        "sample_seconds": round(sum(t.values()), 2),
    }


def block_main(args):
    """--block: layer-wise GPTQ of a Llama-7B-shaped MLP block (gate, up
    4096 -> 11008, down 11008 -> 4096), calibration through the quantized
    gate and up layers; one step = the whole block."""
    import torch

    import post_weight_quantization_12_amd as P
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d, inter = 4096, 11008
    bits, gs, sym, desc, damp = 4, 128, False, True, 0.01
    base = workloads.get("c1")
    t0 = time.perf_counter()
    mixing = workloads._mixing(base, dev, 0)
    outl = workloads.outlier_channels(base, dev, 0)
    T = base.tokens_per_sample
    X = torch.empty((base.tokens, d), dtype=torch.float16, device=dev)
    for s in range(base.samples):
        X[s * T:(s + 1) * T] = workloads.x_sample(base, s, dev, 0, mixing, outl)
    Wg, Wu, Wd = workloads.mlp_block_weights(d, inter, dev)
    torch.cuda.synchronize()
    log(f"[bench] block inputs ready in {time.perf_counter() - t0:.1f} s")
    stream = torch.cuda.current_stream()
    recs = []

    def step(record):
        ev = {}

        def mark(name):
            if record:
                e = torch.cuda.Event(enable_timing=True)
                e.record(stream)
                ev[name] = e
        P.block.quantize_mlp_block(X, Wg, Wu, Wd, bits, gs, sym, damp, desc, stream=stream,
                                   mark=mark)
        if record:
            recs.append(ev)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    names = list(recs[0].keys())
    phases = {}
    for a, b in zip(names[:-1], names[1:]):
        phases[b] = sum(r[a].elapsed_time(r[b]) for r in recs) / len(recs)
    ms = wall * 1e3 / args.steps
    weights = 3 * d * inter
    fwd_flops = 2.0 * base.tokens * d * 2 * inter
    fwd_ms = phases["forward_hessian_down"]
    result = {
        "metric": "GPTQ Llama-7B MLP block (gate, up, down) weights quantized/sec, 1 GPU",
        "value": weights / (ms * 1e-3),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 in, f32 accumulate",
        "data": "synthetic (seeded; stands in for c4 calibration text and Llama weights)",
        "config": {
            "workload": (f"MLP block d={d} inter={inter}: calibration {base.samples}x{T} tokens "
                         f"fp16, {bits}-bit g{gs} asym desc_act={desc} damp {damp}; down_proj "
                         "calibrated through the quantized gate and up layers"),
            "tokens": base.tokens, "d": d, "inter": inter, "bits": bits, "group_size": gs,
            "desc_act": desc, "chunk_tokens": 32768,
        },
        "phase_ms": phases,
        "roofline": {
            "kernel": ("forward phase: dq_gather_x_kernel + dq_tile_kernel (gate and up as one "
                       "[4096 -> 22016] layer), silu_mul_kernel, syrk_dma_kernel per 32768-token "
                       "chunk"),
            "bound": "mfma",
            "achieved": (fwd_flops + float(base.tokens) * inter * (inter + 1)) / (fwd_ms * 1e-3)
            / 1e12,
            "peak": PEAK_FP16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": (fwd_flops + float(base.tokens) * inter * (inter + 1)) / (fwd_ms * 1e-3)
            / 1e12 / PEAK_FP16_TFLOPS,
            "phase_ms": fwd_ms,
            "flops": fwd_flops + float(base.tokens) * inter * (inter + 1),
            "traffic": None,
        },
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = block_cpu_baseline(d, inter, bits, gs, sym, desc, X, Wg, Wu, Wd,
                                                    base.samples)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def decoder_cpu_baseline(d, inter, heads, seq_len, bits, gs, sym, desc, X, Ws, samples):
    """The oracle on a bounded sample of the decoder block: the Hessians and
    the forward of one sequence (scaled to all sequences), the four
    factorizations in full, 32-row sweeps of each layer (scaled to all
    rows); fp64 NumPy."""
    import torch

    import oracle as O

    torch.set_num_threads(max(1, len(os.sched_getaffinity(0))))
    x = X[:seq_len].cpu().double().numpy()
    wq, wk, wv, wo, gm, wg, wu, wd = (w.cpu().double().numpy() for w in Ws)
    rows = 32
    t = {"hessians_forward": 0.0, "prepare": 0.0, "sweeps": 0.0}

    def timed(key, f, *a):
        t0 = time.perf_counter()
        r = f(*a)
        t[key] += time.perf_counter() - t0
        return r

    def factor(H):
        Hd_, _ = O.condition(H, 0.01)
        perm = O.column_order(H, desc)
        return O.hinv_chol(Hd_, perm), perm

    Hx = timed("hessians_forward", O.hessian, x)
    Ux, px = timed("prepare", factor, Hx)
    for w in (wq, wk, wv):
        timed("sweeps", O.gptq_sweep, w[:rows], Ux, px, bits, gs, sym)
    att = timed("hessians_forward", lambda: O.attention(x @ wq.T, x @ wk.T, x @ wv.T, seq_len,
                                                         heads))
    Ho = timed("hessians_forward", O.hessian, att)
    Uo, po = timed("prepare", factor, Ho)
    timed("sweeps", O.gptq_sweep, wo[:rows], Uo, po, bits, gs, sym)
    _, u = timed("hessians_forward", O.residual_rmsnorm, x, att @ wo.T, gm, 1e-5)
    Hm = timed("hessians_forward", O.hessian, u)
    Um, pm = timed("prepare", factor, Hm)
    for w in (wg, wu):
        timed("sweeps", O.gptq_sweep, w[:rows], Um, pm, bits, gs, sym)
    a = timed("hessians_forward", lambda: O.silu_mul(u @ wg.T, u @ wu.T))
    Hd2 = timed("hessians_forward", O.hessian, a)
    Ud, pd = timed("prepare", factor, Hd2)
    t_sd = time.perf_counter()
    O.gptq_sweep(wd[:rows], Ud, pd, bits, gs, sym)
    t_sd = time.perf_counter() - t_sd
    t["sweeps"] += t_sd
    # rows: q, k, v, o, down have d rows, gate and up inter rows (32 each swept)
    t_sweep_full = (t["sweeps"] - t_sd) / 6 * (4 * d + 2 * inter) / rows + t_sd * d / rows
    full = t["hessians_forward"] * samples + t["prepare"] + t_sweep_full
    return {
        "value": (4.0 * d * d + 3.0 * d * inter) / full,
        "unit": "weights/s",
        "cores": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "host": host_description(),
        "sample": (f"one {seq_len}-token sequence for the Hessians and the forward (scaled "
                   f"x{samples}), the four factorizations in full, 32-row sweeps of each layer "
                   "(scaled to all rows); fp64 NumPy; "
                   + ", ".join(f"{k} {v:.2f} s" for k, v in t.items())),
        "sample_seconds": round(sum(t.values()), 2),
    }


def decoder_main(args):
    """--decoder: layer-wise GPTQ of a Llama-7B-shaped decoder block (q, k, v,
    o 4096 x 4096, 32 heads of 128; gate, up 4096 -> 11008, down 11008 ->
    4096), 128 calibration sequences of 2048 tokens; one step = the block."""
    import torch

    import post_weight_quantization_12_amd as P
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d, inter, heads, eps = 4096, 11008, 32, 1e-5
    bits, gs, sym, desc, damp = 4, 128, False, True, 0.01
    base = workloads.get("c1")
    L = base.tokens_per_sample
    t0 = time.perf_counter()
    mixing = workloads._mixing(base, dev, 0)
    outl = workloads.outlier_channels(base, dev, 0)
    X = torch.empty((base.tokens, d), dtype=torch.float16, device=dev)
    for s in range(base.samples):
        X[s * L:(s + 1) * L] = workloads.x_sample(base, s, dev, 0, mixing, outl)
    Ws = workloads.decoder_block_weights(d, inter, dev)
    torch.cuda.synchronize()
    log(f"[bench] decoder inputs ready in {time.perf_counter() - t0:.1f} s")
    stream = torch.cuda.current_stream()
    recs = []

    def step(record):
        ev = {}

        def mark(name):
            if record:
                e = torch.cuda.Event(enable_timing=True)
                e.record(stream)
                ev[f"{len(ev):02d}_{name}"] = e
        P.block.quantize_decoder_block(X, *Ws, heads, L, eps, bits, gs, sym, damp, desc,
                                       stream=stream, mark=mark)
        if record:
            recs.append(ev)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    names = sorted(recs[0].keys())
    phases = {}
    for a, b in zip(names[:-1], names[1:]):
        phases[b[3:] if b[3:] not in phases else b] = \
            sum(r[a].elapsed_time(r[b]) for r in recs) / len(recs)
    ms = wall * 1e3 / args.steps
    weights = 4 * d * d + 3 * d * inter
    att_flops = 2.0 * base.samples * heads * L * L * (d // heads)   # causal: half of 4 L^2 hd
    result = {
        "metric": "GPTQ Llama-7B decoder block (q, k, v, o, gate, up, down) weights quantized/sec, 1 GPU",
        "value": weights / (ms * 1e-3),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 in, f32 accumulate",
        "data": "synthetic (seeded; stands in for c4 calibration text and Llama weights)",
        "config": {
            "workload": (f"decoder block d={d} heads={heads} inter={inter}: calibration "
                         f"{base.samples} sequences x {L} tokens fp16, {bits}-bit g{gs} asym "
                         f"desc_act={desc} damp {damp}; each layer calibrated through the "
                         "quantized layers before it"),
            "tokens": base.tokens, "d": d, "heads": heads, "inter": inter, "bits": bits,
            "group_size": gs, "desc_act": desc,
        },
        "phase_ms": phases,
        "attention_flops_algorithmic": att_flops,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = decoder_cpu_baseline(d, inter, heads, L, bits, gs, sym, desc, X,
                                                      Ws, base.samples)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def export_main(args):
    """--export: gptq_export_params on the config's layer (fp16 scales,
    packed zeros; HBM roofline) and a save / load of the layer through the
    local checkpoint writer (host and file time, for context)."""
    import tempfile

    import torch

    import post_weight_quantization_12_amd as P
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = workloads.get(args.config)
    words, scales, zeros, order = workloads.packed_layer_draws(cfg, dev, 0)
    gs = cfg.inp if cfg.group_size == -1 else cfg.group_size
    g_idx = torch.empty((cfg.inp,), dtype=torch.int32, device=dev)
    g_idx[order] = (torch.arange(cfg.inp, device=dev) // gs).to(torch.int32)
    G, out = scales.shape
    reps = 50
    for _ in range(5):
        P.export_params(scales, zeros, cfg.bits)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        P.export_params(scales, zeros, cfg.bits)
    b.record()
    torch.cuda.synchronize()
    call_ms = a.elapsed_time(b) / reps
    alg = G * out * (4 + 4 + 2) + G * out * cfg.bits // 8
    with tempfile.TemporaryDirectory() as d:
        t0 = time.perf_counter()
        P.checkpoint.save_quantized(d, {"layer": (words, scales, zeros, g_idx)}, cfg.bits,
                                    cfg.group_size, cfg.desc_act, cfg.damp, cfg.sym)
        t_save = time.perf_counter() - t0
        size = sum(os.path.getsize(os.path.join(d, f)) for f in os.listdir(d))
        t0 = time.perf_counter()
        P.checkpoint.load_quantized(d)
        torch.cuda.synchronize()
        t_load = time.perf_counter() - t0
    achieved = alg / (call_ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "gptq_export_params (fp16 scales + packed zeros) GB/s",
        "value": achieved, "unit": "GB/s", "n_gpus": 1, "steps": reps, "warmup": 5,
        "ms_per_step": call_ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32 -> f16, int32 -> b-bit", "data": "synthetic",
        "config": {"workload": f"{cfg.name} layer parameters: {G} groups x {out} channels, "
                               f"{cfg.bits}-bit", "groups": G, "out": out, "bits": cfg.bits},
        "roofline": {"kernel": "export_kernel", "bound": "hbm", "achieved": achieved,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "bytes_per_call": alg, "traffic": None},
        "checkpoint": {"bytes": size, "save_s": t_save, "load_s": t_load,
                       "save_GBps": size / t_save / 1e9, "load_GBps": size / t_load / 1e9},
        "cpu_baseline": None,
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="c3", choices=["c1", "c2", "c3", "c4a", "c4b"])
    ap.add_argument("--chunk-samples", type=int, default=None,
                    help="calibration samples per gptq_hessian_accumulate call "
                         "(default: all of them in one call)")
    ap.add_argument("--summarize", metavar="DIR", default=None,
                    help="write the profiles/ summaries from rocprofv3 output in DIR and exit")
    ap.add_argument("--mfma-counters", action="store_true",
                    help="with --summarize: write the matrix-core counter summary instead")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dequant-tokens", type=int, default=None, metavar="M",
                    help="time gptq_dequant_matmul with M tokens on the config's packed layer "
                         "instead of the quantization step")
    ap.add_argument("--export", action="store_true",
                    help="time gptq_export_params and a checkpoint save / load of the layer")
    ap.add_argument("--block", action="store_true",
                    help="time layer-wise GPTQ of a Llama-7B-shaped MLP block instead")
    ap.add_argument("--decoder", action="store_true",
                    help="time layer-wise GPTQ of a whole Llama-7B-shaped decoder block instead")
    ap.add_argument("--dequant-as-packed", action="store_true",
                    help="with --dequant-tokens on an act-order config: use the layer as packed "
                         "instead of its group order")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain 1 GiB device-to-device copy (a reference kernel "
                         "of known traffic for calibrating rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()

    if args.summarize:
        if args.dequant_tokens is not None:
            summarize_dequant(args.config, args.dequant_tokens, args.summarize)
        elif args.block:
            summarize_block(args.summarize, "block")
        elif args.decoder:
            summarize_block(args.summarize, "decoder")
        elif args.mfma_counters:
            summarize_mfma(args.config, args.summarize)
        else:
            summarize(args.config, args.summarize)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this GPTQ build runs on one GPU only (no sharding, no collectives); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.dequant_tokens is not None:
        dequant_main(args)
        return
    if args.block:
        block_main(args)
        return
    if args.decoder:
        decoder_main(args)
        return
    if args.export:
        export_main(args)
        return

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
    chunk = (args.chunk_samples or cfg.samples) * T
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
    kernels, launches = syrk_schedule(n, chunk, torch.cuda.get_device_properties(0).multi_processor_count)
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
        "layer_roofline": layer_roofline(cfg, mean(hess_ms), mean(prep_ms), mean(quant_ms)),
        "roofline": {
            "kernel": f"{kernels} = one gptq_hessian_accumulate call",
            "kernel_launches_per_call": launches,
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_FP16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_FP16_TFLOPS,
            "call_ms": syrk_launch_ms,
            "flops_per_call": syrk_launch_flops,
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
