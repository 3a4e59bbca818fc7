"""Throughput of the ftx BERT encoder forward on one MI355X.

Default workload: BERT-base, 12 layers, 12 heads x 64, fp16 (fp32 accumulation), sequence
length 32, batch 512, no padding; weights N(0, 0.02), input N(0, 1), seeded, synthetic.
A step is one full forward (all 12 layers) of the batch, inputs already in device memory.

Prints ONE JSON line: sequences/s (value), ms per step, TFLOP/s and its fraction of the
dense fp16 MFMA peak, the roofline of the dominant kernel measured with HIP events on the
forward's stream, and the fp64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sequences/sec + TFLOPS (% MFMA peak), 12-layer BERT-base fp16, seq 32/128"
WORKLOAD_DEFAULT = "bert_base_fp16_s32"
PEAK_MFMA_TFLOPS = {"fp16": 2516.6, "bf16": 2516.6, "fp32": 157.3}
PEAK_HBM_GBS = 8000.0
# MI355X: 256 CUs of 4 SIMDs at a 2.4 GHz peak engine clock (AMD's published figures); the
# MFMA-busy fraction divides SQ_VALU_MFMA_BUSY_CYCLES (summed over every SIMD) by
# SIMDs x clock x kernel time
SIMDS = 1024
CLOCK_HZ = 2.4e9
# bytes read before each timed launch of the HBM measurement: four times the 256 MB
# last-level cache (MALL), so every input of the timed kernel comes from HBM (read, not
# written: written lines would leave the caches dirty, and their write-back would land in the
# timed kernel)
FLUSH_BYTES = 1 << 30
DTYPE_TAG = {"fp16": "f16", "bf16": "bf16", "fp32": "f32"}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=None, help=f"default {WORKLOAD_DEFAULT}")
    p.add_argument("--batch", type=int, default=None)
    p.add_argument("--unfused", action="store_true", help="standalone bias+split and bias+GELU kernels")
    p.add_argument("--no-fold-layernorm", action="store_true",
                   help="the first LayerNorm of each layer as its own kernel (not folded into "
                        "the FFN-in projection)")
    p.add_argument("--no-prefetch-weights", action="store_true",
                   help="never read W2 into the last-level cache ahead of the second FFN projection")
    p.add_argument("--graph", action="store_true", help="replay the forward as one HIP graph")
    p.add_argument("--fused-attention", type=int, default=1, choices=(0, 1, 2),
                   help="projection + attention in one kernel: 0 never, 1 from 256 tokens and "
                        "64 tiles of 256 rows or a split-K Q/K/V projection (default), 2 "
                        "whenever the shape fits")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU-oracle sample time")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-kernel-times", action="store_true")
    p.add_argument("--copy-calib-mb", type=int, default=0,
                   help="before the forwards, run a plain device copy kernel (torch.neg, fp16) over "
                        "this many MiB three times, so a counter run also sees a kernel of known traffic")
    p.add_argument("--summarize-rocprof", nargs="+", metavar="DIR",
                   help="TRACE_DIR FETCH_DIR WRITE_DIR [MFMA_DIR]: write profiles/<--summary-name>.md "
                        "and _traffic.json from rocprofv3 output of this benchmark, then exit (no GPU "
                        "needed)")
    p.add_argument("--no-hbm", action="store_true",
                   help="skip the HBM measurement of the element-wise kernels with the MALL flushed")
    p.add_argument("--hbm-reps", type=int, default=20)
    p.add_argument("--hbm-only", action="store_true",
                   help="only the element-wise HBM measurement (one JSON line), e.g. under a kernel trace")
    p.add_argument("--summarize-hbm", metavar="TRACE_DIR", default=None,
                   help="write profiles/<--summary-name>.md from a rocprofv3 --kernel-trace run of "
                        "--hbm-only, then exit (no GPU needed)")
    p.add_argument("--summarize-trace", metavar="TRACE_DIR", default=None,
                   help="write profiles/<--summary-name>.md from a rocprofv3 kernel-trace run of "
                        "this benchmark (kernel stats only), then exit (no GPU needed)")
    p.add_argument("--calibrate-gemm", action="store_true",
                   help="time the workload's four projection shapes with the ftx GEMM (plain, and "
                        "FFN-in with its bias + GELU epilogue) and with the vendor library GEMM "
                        "(torch.matmul, same weight layout) for comparison; one JSON line")
    p.add_argument("--summarize-calibration", metavar="JSON_FILE", default=None,
                   help="write profiles/<--summary-name>.md from the saved output of --calibrate-gemm, "
                        "then exit (no GPU needed)")
    p.add_argument("--summary-name", default=None)
    p.add_argument("--summary-commands", nargs="*", default=[])
    return p.parse_args()


def launches_per_layer(counts, step) -> int:
    """Launches of `step` per layer, from launch counts per step class (the Q/K/V step runs once
    per layer; the FFN block may run in row chunks, each chunk a launch per step)."""
    ref = next((counts[k] for k in ("qkv_attention", "qkv_gemm") if counts.get(k)), 0)
    if not ref or step not in ("ffn1_gemm", "ffn2_gemm", "ln2", "bias_gelu"):
        return 1
    return max(1, round(counts.get(step, 0) / ref))


def fold_stats_bytes(shape) -> int:
    """Bytes of the per-tile row statistics of the folded LayerNorm: one (mean, M2) float pair
    per row and attention-output tile column (the planner's tile width at 256 CUs)."""
    from transformer_encoder_bert_amd import ftx
    tn = ftx.ftx_plan_linear(shape.dtype, shape.tokens, shape.hidden, shape.hidden, 256)[1]
    return shape.tokens * -(-shape.hidden // tn) * 8


def step_work(shape, step: str, folded: bool = False):
    """Algorithmic work of ONE launch of a step class: (flops, bytes).
    Bytes are the minimum HBM traffic (each operand read once, result written once), with
    the fp32 tensors of the bf16 mode (the attention-output and FFN-out results, the fp32 copy
    of Y1) at 4 bytes.  folded: the first LayerNorm folded into FFN-in (the attention-output
    projection also reads the residual and writes Z1 and its row statistics, the second
    LayerNorm reads them back)."""
    T, S, H, F, B = shape.tokens, shape.seq_len, shape.hidden, shape.ffn, shape.batch
    e = 4 if shape.dtype == "fp32" else 2
    f32res = shape.dtype == "bf16"
    ea = 4 if f32res else e  # the attention-output and FFN-out results
    if step == "qkv_gemm":
        return 2.0 * T * 3 * H * H, (T * H + 3 * H * H + 3 * T * H) * e
    if step == "attn_out_gemm":
        if folded:
            return 2.0 * T * H * H, ((3 * T * H + H * H) * e + (T * H * 4 if f32res else 0)
                                     + fold_stats_bytes(shape))
        return 2.0 * T * H * H, (T * H + H * H) * e + T * H * ea
    if step == "ffn1_gemm":
        return 2.0 * T * F * H, ((T * H + F * H + T * F) * e
                                 + (fold_stats_bytes(shape) + 2 * F * 4 if folded else 0))
    if step == "ffn2_gemm":
        return 2.0 * T * H * F, (T * F + H * F) * e + T * H * ea
    if step == "attention":
        return 4.0 * B * S * S * H, 4 * T * H * e
    if step == "qkv_attention":  # Q, K and V stay on chip
        return 2.0 * T * 3 * H * H + 4.0 * B * S * S * H, (T * H + 3 * H * H + T * H) * e
    if step == "ln1":  # bf16: the fp32 branch in, Y1 out in bf16 and fp32
        return 0.0, (T * H * (2 * e + 8) if f32res else 3 * T * H * e)
    if step == "ln2":  # bf16: Y1 (or Z1) and the branch in fp32
        return 0.0, ((T * H * (8 + e) if f32res else 3 * T * H * e)
                     + (fold_stats_bytes(shape) if folded else 0))
    if step == "bias_gelu":
        return 0.0, 2 * T * F * e
    if step == "bias_qkv_split":
        return 0.0, 2 * 3 * T * H * e
    if step == "weight_prefetch":  # W2 read once, nothing written
        return 0.0, H * F * e
    raise KeyError(step)


# ----------------------------------------------------------------- rocprofv3 summaries
# Kernel sources whose hash tags a traffic measurement: traffic figures are reported only
# while these files are unchanged since the counters were taken.
KERNEL_SOURCES = ("transformer_encoder_bert_amd/csrc/gemm.hip",
                  "transformer_encoder_bert_amd/csrc/attention.hip",
                  "transformer_encoder_bert_amd/csrc/elementwise.hip",
                  "transformer_encoder_bert_amd/csrc/device_common.h")


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code: // comments and blank lines are dropped, so editing a
    comment does not mark a measurement stale."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            for line in f:
                code = re.sub(r"//.*$", "", line).rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def classify_dispatches(names):
    """Step class of each kernel dispatch of a forward, from the fixed launch order of a
    layer (the attention-output and FFN-output projections share one kernel symbol)."""
    import re
    steps, prev = [], None
    for n in names:
        st = None
        # the projections run the two-buffer K loop (gemm_kernel) or, for long K, the
        # ping-pong one (gemm_pp_kernel)
        gemm = "gemm_kernel" in n or "gemm_pp_kernel" in n
        if gemm and "EpiQKVAttn" in n:
            st = "qkv_attention"
        elif gemm and "EpiQKV" in n:
            st = "qkv_gemm"
        elif "attention" in n and "ftx" in n:
            st = "attention"
        elif "layernorm_kernel" in n:
            st = "ln1" if prev in ("attn_out_gemm", "attention") else "ln2"
        elif gemm and "EpiLinearResStats" in n:
            st = "attn_out_gemm"  # with the first LayerNorm folded into FFN-in
        elif gemm and "EpiLinearNormIn" in n:
            st = "ffn1_gemm"
        elif gemm and "EpiLinear" in n:
            m = re.search(r"EpiLinearI\w+?Lb([01])E", n)
            gelu = m is not None and m.group(1) == "1"
            if gelu or prev == "ln1":
                st = "ffn1_gemm"
            elif prev in ("attention", "qkv_attention"):
                st = "attn_out_gemm"
            else:
                st = "ffn2_gemm"
        elif "bias_gelu_kernel" in n:
            st = "bias_gelu"
        elif "bias_qkv_split_kernel" in n:
            st = "bias_qkv_split"
        elif "prefetch16_kernel" in n:
            st = "weight_prefetch"
        steps.append(st)
        if st is not None:
            prev = st
    return steps


def profile_commands(wl, calib_mb, name, batch=None):
    """The four rocprofv3 runs a summary is made from (kernel trace, FETCH_SIZE, WRITE_SIZE,
    MFMA-busy counters), and the summarizing call."""
    w = ("" if wl == WORKLOAD_DEFAULT else f" --workload {wl}") + (f" --batch {batch}" if batch else "")
    run = f"python3 bench.py{w} --no-cpu-baseline --no-hbm --copy-calib-mb {calib_mb}"
    short = "--steps 2 --warmup 1 --no-kernel-times"
    return [
        f"rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/prof_trace -o trace -- {run} --steps 5 --warmup 2",
        f"rocprofv3 --pmc FETCH_SIZE -f csv -d gpurun_out/prof_fetch -o fetch -- {run} {short}",
        f"rocprofv3 --pmc WRITE_SIZE -f csv -d gpurun_out/prof_write -o write -- {run} {short}",
        f"rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES -f csv -d gpurun_out/prof_mfma -o mfma -- {run} {short}",
        f"python3 bench.py{w} --copy-calib-mb {calib_mb} --summarize-rocprof gpurun_out/prof_trace "
        f"gpurun_out/prof_fetch gpurun_out/prof_write gpurun_out/prof_mfma --summary-name {name}",
    ]


# what each ftx kernel symbol is, for the kernel-trace summaries (demangling by hand: the
# host's c++filt predates the _Float16 mangling)
KERNEL_ROLES = (
    ("splitk_layernorm", "split-K partial sum + bias + residual + LayerNorm"),
    ("splitk_reduce_kernelINS_6EpiQKV", "split-K reduction + bias + head split (Q/K/V)"),
    ("splitk_reduce_kernelINS_9EpiLinearIDF16_Lb1", "split-K reduction + bias + GELU (FFN-in)"),
    ("splitk_reduce_kernelINS_9EpiLinearIDF16bLb1", "split-K reduction + bias + GELU (FFN-in)"),
    ("splitk_reduce", "split-K reduction + the projection's epilogue"),
    ("EpiQKVAttn", "Q/K/V projection with the attention in its epilogue"),
    ("EpiQKV", "Q/K/V (or Q-only, K/V-only) projection with bias + head split"),
    ("EpiLinearResStats", "attention-output projection + bias + residual, with per-tile row statistics (LayerNorm 1 folded)"),
    ("EpiLinearNormIn", "FFN-in on the un-normalised rows, LayerNorm 1 applied in the epilogue, + bias + GELU"),
    ("fold_ln_weights", "LayerNorm weight folding (set_weights, not in the forward)"),
    ("EpiLinearIDF16_Lb1", "projection with bias + GELU (FFN-in)"),
    ("EpiLinearIDF16bLb1", "projection with bias + GELU (FFN-in)"),
    ("EpiLinear", "projection (attention output, FFN-out)"),
    ("EpiPartial", "split-K partial products"),
    ("attention", "attention (scores, masked softmax, context)"),
    ("ELb1ELb1EEEvPKT0_", "bias + residual + LayerNorm (LayerNorm 2, residual rebuilt from the folded LayerNorm 1)"),
    ("layernorm", "bias + residual + LayerNorm"),
    ("transpose", "weight repacking (set_weights, not in the forward)"),
    ("prefetch16_kernel", "read of the FFN-out weights into the last-level cache"),
)


def summarize_trace(args):
    """Summarise the kernel statistics of a rocprofv3 --kernel-trace --stats run of this
    benchmark into profiles/<name>.md (ftx kernels only)."""
    import csv
    fs = [os.path.join(args.summarize_trace, f) for f in os.listdir(args.summarize_trace)
          if f.endswith("_kernel_stats.csv")]
    if len(fs) != 1:
        raise SystemExit(f"expected one *_kernel_stats.csv in {args.summarize_trace}")
    rows = [r for r in csv.DictReader(open(fs[0])) if "ftx" in r["Name"]]
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    wl = args.workload or WORKLOAD_DEFAULT
    import synthetic_inputs as si
    batches = si.DECODER_WORKLOAD["batches"] if wl == si.DECODER_WORKLOAD["name"] else si.WORKLOADS[wl].batches
    batch = args.batch or max(batches)
    flags = (f" --workload {wl}" if wl != WORKLOAD_DEFAULT else "") + (f" --batch {args.batch}" if args.batch else "")
    d = os.path.relpath(os.path.abspath(args.summarize_trace), ROOT)
    lines = [f"# Kernel time per forward -- {wl}, batch {batch}", "",
             "Commands (from the repository root, on one MI355X, with TMPDIR=/tmp):", "", "```",
             f"rocprofv3 --kernel-trace --stats -f csv -d {d} -o trace -- python3 bench.py"
             f"{flags} --steps 5 --warmup 2 --no-cpu-baseline",
             f"python3 bench.py{flags} --summarize-trace {d} --summary-name {args.summary_name}",
             "```", "",
             "The run makes 2 warm-up forwards, one forward that reads the launch counts, 5 timed",
             "forwards, 5 latency-timed forwards and 5 with per-launch events.", "",
             "| kernel | role | calls | avg us | share of ftx kernel time % |", "|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        role = next((v for k, v in KERNEL_ROLES if k in r["Name"]), "")
        lines.append(f"| `{r['Name']}` | {role} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{100 * float(r['TotalDurationNs']) / total:.1f} |")
    lines += ["", f"Kernel source hash: `{kernel_source_hash()}`"]
    path = os.path.join(ROOT, "profiles", args.summary_name + ".md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)


def summarize_rocprof(args):
    """Summarise a rocprofv3 kernel trace plus FETCH_SIZE / WRITE_SIZE counter runs of this
    benchmark (made with --copy-calib-mb) into profiles/<name>.md and profiles/<name>_traffic.json."""
    import csv
    if len(args.summarize_rocprof) not in (3, 4):
        raise SystemExit("--summarize-rocprof takes TRACE_DIR FETCH_DIR WRITE_DIR [MFMA_DIR]")
    trace_dir, fetch_dir, write_dir = args.summarize_rocprof[:3]
    mfma_dir = args.summarize_rocprof[3] if len(args.summarize_rocprof) == 4 else None
    def one(d, suffix):
        fs = [os.path.join(d, f) for f in os.listdir(d) if f.endswith(suffix)]
        if len(fs) != 1:
            raise SystemExit(f"expected one *{suffix} in {d}")
        return list(csv.DictReader(open(fs[0])))
    trace = one(trace_dir, "_kernel_trace.csv")
    trace.sort(key=lambda r: int(r["Dispatch_Id"]))
    steps = classify_dispatches([r["Kernel_Name"] for r in trace])
    dur = {}
    sym = {}
    for r, st in zip(trace, steps):
        if st is None:
            continue
        dur.setdefault(st, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
        sym[st] = r["Kernel_Name"]
    calib_bytes = args.copy_calib_mb * (1 << 20)
    counters = {}
    scale = {}
    for name, d, suffix in (("FETCH_SIZE", fetch_dir, "_counter_collection.csv"),
                            ("WRITE_SIZE", write_dir, "_counter_collection.csv")):
        rows = one(d, suffix)
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        cal = [float(r["Counter_Value"]) for r in rows if "neg_kernel" in r["Kernel_Name"]]
        if not cal:
            raise SystemExit("no calibration copy kernel in the counter run")
        scale[name] = calib_bytes / (sum(cal) / len(cal) * 1024.0)  # true bytes per counted byte
        st_rows = classify_dispatches([r["Kernel_Name"] for r in rows])
        for r, st in zip(rows, st_rows):
            if st is None:
                continue
            counters.setdefault(st, {}).setdefault(name, []).append(float(r["Counter_Value"]) * 1024.0 * scale[name])
    mfma = {}
    if mfma_dir:
        # one row per (dispatch, counter): MFMA-busy cycles summed over every SIMD
        rows = one(mfma_dir, "_counter_collection.csv")
        per_dispatch = {}
        for r in rows:
            if r["Counter_Name"] == "SQ_VALU_MFMA_BUSY_CYCLES":
                per_dispatch[int(r["Dispatch_Id"])] = (r["Kernel_Name"], float(r["Counter_Value"]))
        ids = sorted(per_dispatch)
        for i, st in zip(ids, classify_dispatches([per_dispatch[i][0] for i in ids])):
            if st is not None:
                mfma.setdefault(st, []).append(per_dispatch[i][1])
    wl = WORKLOAD_DEFAULT if args.workload is None else args.workload
    import synthetic_inputs as si
    w = si.WORKLOADS[wl]
    shape = w.shape(args.batch or max(w.batches))
    out = {"workload": wl, "batch": shape.batch, "kernel_source_hash": kernel_source_hash(),
           "scale": scale, "simds": SIMDS, "clock_hz": CLOCK_HZ, "steps": {}}
    commands = args.summary_commands or profile_commands(wl, args.copy_calib_mb, args.summary_name,
                                                         args.batch)
    lines = [f"# Kernel time and HBM traffic per step -- {wl}, batch {shape.batch}", "",
             "Commands (from the repository root, on one MI355X, with TMPDIR=/tmp):", "", "```",
             *commands, "```", "",
             f"FETCH_SIZE and WRITE_SIZE are scaled by what they read for a plain copy kernel "
             f"(torch.neg over {args.copy_calib_mb} MiB of fp16): true bytes per counted byte "
             f"{scale['FETCH_SIZE']:.3f} (fetch) and {scale['WRITE_SIZE']:.3f} (write).",
             "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES (summed over the SIMDs) / "
             f"({SIMDS} SIMDs x {CLOCK_HZ / 1e9:.1f} GHz x avg us); frac = algorithmic TFLOP/s / "
             f"{PEAK_MFMA_TFLOPS[shape.dtype]} (dense MFMA peak).", "",
             "| step | launches | avg us | algorithmic MB | fetched MB | written MB | traffic / algorithmic | "
             "algorithmic TFLOP/s | frac of peak | MFMA busy % | algorithmic GB/s |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    folded = "EpiLinearResStats" in sym.get("attn_out_gemm", "")
    per_layer = {k: len(v) for k, v in dur.items()}
    for st in ("qkv_attention", "qkv_gemm", "bias_qkv_split", "attention", "attn_out_gemm", "ln1", "ffn1_gemm",
               "bias_gelu", "weight_prefetch", "ffn2_gemm", "ln2"):
        if st not in dur:
            continue
        avg = sum(dur[st]) / len(dur[st])
        fl, by = step_work(shape, st, folded)
        ch = launches_per_layer(per_layer, st)  # the FFN block in row chunks: work per launch
        fl, by = fl / ch, by / ch
        c = counters.get(st, {})
        fetch = sum(c.get("FETCH_SIZE", [0])) / max(1, len(c.get("FETCH_SIZE", [])))
        write = sum(c.get("WRITE_SIZE", [0])) / max(1, len(c.get("WRITE_SIZE", [])))
        busy = None
        if st in mfma:
            busy = sum(mfma[st]) / len(mfma[st]) / (SIMDS * CLOCK_HZ * avg * 1e-6)
        tfl = fl / (avg * 1e-6) / 1e12 if fl else 0.0
        out["steps"][st] = {"symbol": sym[st], "avg_us": avg, "launches": len(dur[st]),
                            "fetch_bytes": fetch, "write_bytes": write,
                            "algorithmic_bytes": by, "flops": fl, "mfma_busy": busy,
                            "frac": tfl / PEAK_MFMA_TFLOPS[shape.dtype] if fl else None}
        lines.append(f"| {st} | {len(dur[st])} | {avg:.1f} | {by / 1e6:.1f} | {fetch / 1e6:.1f} | "
                     f"{write / 1e6:.1f} | {(fetch + write) / by:.2f} | {tfl:.1f} | "
                     f"{tfl / PEAK_MFMA_TFLOPS[shape.dtype]:.3f} | "
                     f"{'' if busy is None else f'{100 * busy:.1f}'} | {by / (avg * 1e-6) / 1e9:.0f} |")
    lines += ["", "Kernel symbols:", ""]
    lines += [f"- {st}: `{v['symbol']}`" for st, v in out["steps"].items()]
    lines += ["", f"Kernel source hash: `{out['kernel_source_hash']}`"]
    base = os.path.join(ROOT, "profiles", args.summary_name)
    os.makedirs(os.path.dirname(base), exist_ok=True)
    with open(base + ".md", "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(base + "_traffic.json", "w") as f:
        json.dump(out, f, indent=1)
    print(base + ".md")


HBM_KERNELS = (("layernorm_kernel", "bias_residual_layernorm", lambda T, H, F, e: 3 * T * H * e),
               ("bias_gelu_kernel", "bias_gelu", lambda T, H, F, e: 2 * T * F * e),
               ("bias_qkv_split_kernel", "bias_qkv_split", lambda T, H, F, e: 6 * T * H * e))


def summarize_hbm(args):
    """Kernel times of the element-wise kernels in a rocprofv3 --kernel-trace run of
    --hbm-only (each launch after the MALL flush) into profiles/<name>.md: algorithmic bytes
    over the traced kernel time, against 8 TB/s."""
    import csv
    fs = [os.path.join(args.summarize_hbm, f) for f in os.listdir(args.summarize_hbm)
          if f.endswith("_kernel_trace.csv")]
    if len(fs) != 1:
        raise SystemExit(f"expected one *_kernel_trace.csv in {args.summarize_hbm}")
    rows = sorted(csv.DictReader(open(fs[0])), key=lambda r: int(r["Dispatch_Id"]))
    import synthetic_inputs as si
    wl = args.workload or WORKLOAD_DEFAULT
    shape = si.WORKLOADS[wl].shape(args.batch)
    e = 4 if shape.dtype == "fp32" else 2
    d = os.path.relpath(os.path.abspath(args.summarize_hbm), ROOT)
    flags = (f" --workload {wl}" if wl != WORKLOAD_DEFAULT else "") + (f" --batch {args.batch}" if args.batch else "")
    lines = [f"# Element-wise kernels from HBM (MALL flushed) -- {wl}, batch {shape.batch}", "",
             "Commands (from the repository root, on one MI355X, with TMPDIR=/tmp):", "", "```",
             f"rocprofv3 --kernel-trace -f csv -d {d} -o hbm -- python3 bench.py{flags} --hbm-only",
             f"python3 bench.py{flags} --summarize-hbm {d} --summary-name {args.summary_name}",
             "```", "",
             f"Each launch runs alone after a reduction that reads {FLUSH_BYTES >> 20} MiB (four times the "
             "256 MB MALL), so its inputs come from HBM.  The first launch of each kernel (a warm-up "
             "without the flush) is left out.  GB/s = algorithmic bytes (inputs once, output once) / "
             "traced kernel time.", "",
             "| kernel | launches | algorithmic MB | median us | min us | GB/s (median) | % of 8 TB/s |",
             "|---|---|---|---|---|---|---|"]
    for sym_part, name, nbytes in HBM_KERNELS:
        t = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3 for r in rows
             if sym_part in r["Kernel_Name"] and "ftx" in r["Kernel_Name"]][1:]
        if not t:
            continue
        by = nbytes(shape.tokens, shape.hidden, shape.ffn, e)
        med = float(np.median(t))
        lines.append(f"| {name} | {len(t)} | {by / 1e6:.1f} | {med:.1f} | {min(t):.1f} | "
                     f"{by / (med * 1e-6) / 1e9:.0f} | {100 * by / (med * 1e-6) / 1e9 / PEAK_HBM_GBS:.1f} |")
    lines += ["", f"Kernel source hash: `{kernel_source_hash()}`"]
    path = os.path.join(ROOT, "profiles", args.summary_name + ".md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)


def measured_profile(workload: str, batch: int, step: str):
    """What the committed rocprofv3 summary of this workload says of `step` (kernel time,
    HBM bytes, MFMA busy), or None when there is none or the kernel sources changed since it
    was taken."""
    rel = os.path.join("profiles", f"{workload}_b{batch}_traffic.json")
    path = os.path.join(ROOT, rel)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash() or step not in t.get("steps", {}):
        return None
    s = dict(t["steps"][step])
    s["traffic"] = s["fetch_bytes"] + s["write_bytes"]
    s["source"] = rel.replace("_traffic.json", ".md")
    return s


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(case, target_s: float):
    """The fp64 oracle, as it stands, on the first n sequences of the same workload."""
    import oracle
    layers = list(case.layers())
    n = 1
    t0 = time.perf_counter()
    oracle.encoder_rows(case.x, layers, case.lens, case.shape.head_num, list(range(n)))
    one = time.perf_counter() - t0
    n = int(max(1, min(case.shape.batch, target_s / max(one, 1e-3))))
    t0 = time.perf_counter()
    oracle.encoder_rows(case.x, layers, case.lens, case.shape.head_num, list(range(n)))
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "sequences/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"first {n} of {case.shape.batch} sequences, all {case.shape.num_layers} layers, "
                      f"numpy float64 ({dt:.1f} s)",
            "cpu": platform.processor() or platform.machine()}


DECODER_METRIC = "sequences/sec + TFLOPS (% MFMA peak), 12-layer decoder fp16, 32 positions over a 32-position memory"


def dec_step_work(shape, step: str):
    """Algorithmic work of ONE launch of a decoder step class: (flops, bytes)."""
    B, Sd, Se, H, F = shape.batch, shape.tgt_len, shape.mem_len, shape.hidden, shape.ffn
    T, Tm = B * Sd, B * Se
    e = 4 if shape.dtype == "fp32" else 2
    if step == "self_qkv_gemm":
        return 2.0 * T * 3 * H * H, (T * H + 3 * H * H + 3 * T * H) * e
    if step in ("self_out_gemm", "cross_out_gemm", "cross_q_gemm"):
        return 2.0 * T * H * H, (2 * T * H + H * H) * e
    if step == "cross_kv_gemm":
        return 2.0 * Tm * 2 * H * H, (Tm * H + 2 * H * H + 2 * Tm * H) * e
    if step == "ffn1_gemm":
        return 2.0 * T * F * H, (T * H + F * H + T * F) * e
    if step == "ffn2_gemm":
        return 2.0 * T * H * F, (T * F + H * F + T * H) * e
    if step == "self_attention":
        return 4.0 * B * Sd * Sd * H, 4 * T * H * e
    if step == "self_qkv_attention":  # Q, K and V stay on chip
        return 2.0 * T * 3 * H * H + 4.0 * B * Sd * Sd * H, (2 * T * H + 3 * H * H) * e
    if step == "cross_attention":
        return 4.0 * B * Sd * Se * H, (2 * T * H + 2 * Tm * H) * e
    if step in ("ln1", "ln2", "ln3"):
        return 0.0, 3 * T * H * e
    raise KeyError(step)


def bench_decoder(args):
    """The decoder forward (the article's roadmap item): same timing and JSON fields as the
    encoder's bench line, on the decoder workload of synthetic_inputs."""
    import torch
    import synthetic_inputs as si
    from transformer_encoder_bert_amd import ftx

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    wd = si.DECODER_WORKLOAD
    batch = args.batch or max(wd["batches"])
    shape = si.DecoderShape(batch, wd["tgt_len"], wd["mem_len"], wd["head_num"], wd["size_per_head"],
                            wd["num_layers"], wd["dtype"])
    case = si.make_decoder_case(shape, wd["seed"], mem_lens_range=wd["mem_lens_range"])
    dt, dev = shape.dtype, "cuda:0"
    torch.cuda.set_device(0)

    def up(a):
        return torch.from_numpy(si.host_array(a, dt)).to(dev)

    dec = ftx.Decoder(batch, shape.tgt_len, shape.mem_len, shape.head_num, shape.size_per_head,
                      shape.num_layers, dt)
    dec.set_option(ftx.FTX_OPT_FUSED_ATTENTION, args.fused_attention)
    for l, w in enumerate(case.layers()):
        dec.set_weights(l, {k: up(w[k]) for k in si.DECODER_WEIGHT_NAMES})
    x, mem = up(case.x), up(case.mem)
    lens = None if case.mem_lens is None else torch.from_numpy(case.mem_lens).to(dev)
    out = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        dec.forward(x, mem, lens, out)
    torch.cuda.synchronize()
    # which self-attention path the handle takes (one forward with launch counts, untimed)
    dec.set_option(ftx.FTX_OPT_KERNEL_TIMING, 1)
    dec.forward(x, mem, lens, out)
    attn_fused = dec.kernel_times()["self_qkv_attention"][1] > 0
    dec.set_option(ftx.FTX_OPT_KERNEL_TIMING, 0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dec.forward(x, mem, lens, out)
    torch.cuda.synchronize()
    ms_per_step = 1e3 * (time.perf_counter() - t0) / args.steps
    tflops = shape.flops() / (ms_per_step * 1e-3) / 1e12
    result = {
        "metric": DECODER_METRIC, "value": batch / (ms_per_step * 1e-3), "unit": "sequences/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": DTYPE_TAG[dt],
        "data": "synthetic",
        "config": {"workload": f"{wd['name']}: {wd['description']}", "global_batch": batch,
                   "tgt_len": shape.tgt_len, "mem_len": shape.mem_len, "layers": shape.num_layers,
                   "heads": shape.head_num, "size_per_head": shape.size_per_head,
                   "parallelism": "none (1 GPU)",
                   "self_attention": ("in the Q/K/V projection's epilogue" if attn_fused
                                      else "own kernel")},
        "tflops": tflops, "frac_mfma_peak": tflops / PEAK_MFMA_TFLOPS[dt],
        "roofline": None, "cpu_baseline": None,
    }
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        dec.forward(x, mem, lens, out)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    lat = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    result["latency_ms"] = {q: float(np.percentile(lat, v)) for q, v in (("p10", 10), ("p50", 50), ("p90", 90))}
    if not args.no_kernel_times:
        dec.set_option(ftx.FTX_OPT_KERNEL_TIMING, 1)
        dec.kernel_times()
        for _ in range(args.steps):
            dec.forward(x, mem, lens, out)
        torch.cuda.synchronize()
        times = dec.kernel_times()
        dec.set_option(ftx.FTX_OPT_KERNEL_TIMING, 0)
        kernels = {}
        for name, (ms, cnt) in times.items():
            if cnt:
                fl, by = dec_step_work(shape, name)
                avg = ms / cnt
                kernels[name] = {"avg_us": 1e3 * avg, "launches": cnt, "share": 0.0,
                                 "tflops": fl / (avg * 1e-3) / 1e12 if fl else None,
                                 "gbs_algorithmic": by / (avg * 1e-3) / 1e9}
        total = sum(v["avg_us"] * v["launches"] for v in kernels.values())
        for v in kernels.values():
            v["share"] = v["avg_us"] * v["launches"] / total
        dom = max(kernels, key=lambda k: kernels[k]["avg_us"] * kernels[k]["launches"])
        fl, by = dec_step_work(shape, dom)
        avg_s = kernels[dom]["avg_us"] * 1e-6
        if fl > 0 and "attention" not in dom:
            achieved, peak, unit, bound = fl / avg_s / 1e12, PEAK_MFMA_TFLOPS[dt], "TFLOP/s", "mfma"
        else:
            achieved, peak, unit, bound = by / avg_s / 1e9, PEAK_HBM_GBS, "GB/s", "hbm"
        result["roofline"] = {"kernel": dom, "bound": bound, "achieved": achieved, "peak": peak,
                              "unit": unit, "frac": achieved / peak, "traffic": None,
                              "traffic_gbs": None, "work_per_launch": fl if bound == "mfma" else by,
                              "avg_launch_us": kernels[dom]["avg_us"]}
        result["kernels"] = kernels
    dec.close()
    if not args.no_cpu_baseline:
        import oracle
        layers = list(case.layers())

        def run(n):
            ml = None if case.mem_lens is None else case.mem_lens[:n]
            oracle.decoder(case.x[:n], case.mem[:n], layers, ml, shape.head_num)
        t0 = time.perf_counter()
        run(1)
        one = time.perf_counter() - t0
        n = int(max(1, min(batch, args.cpu_seconds / max(one, 1e-3))))
        t0 = time.perf_counter()
        run(n)
        el = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": n / el, "unit": "sequences/s", "cores": blas_threads(),
                                  "kind": "oracle",
                                  "sample": f"first {n} of {batch} sequences, all {shape.num_layers} "
                                            f"layers, numpy float64 ({el:.1f} s)",
                                  "cpu": platform.processor() or platform.machine()}
    print(json.dumps(result), flush=True)


def main():
    args = parse()
    if args.summarize_rocprof or args.summarize_trace or args.summarize_hbm or args.summarize_calibration:
        if not args.summary_name:
            raise SystemExit("--summary-name is required")
        if args.summarize_calibration:
            summarize_calibration(args)
        elif args.summarize_rocprof:
            summarize_rocprof(args)
        elif args.summarize_hbm:
            summarize_hbm(args)
        else:
            summarize_trace(args)
        return
    if args.workload is None:
        args.workload = WORKLOAD_DEFAULT
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py measures one GPU: the encoder forward shards by data parallelism with no "
              f"collective, so the one-GPU figure times each GPU's share (asked: --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import synthetic_inputs as si
    if args.workload == si.DECODER_WORKLOAD["name"]:
        return bench_decoder(args)
    import torch
    from transformer_encoder_bert_amd import ftx

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    wl = si.WORKLOADS[args.workload]
    batch = args.batch or max(wl.batches)
    if args.calibrate_gemm:
        return calibrate_gemm(args, wl, batch)
    if args.hbm_only:
        shape = wl.shape(batch)
        res = {"workload": wl.name, "batch": batch, "elementwise_hbm": elementwise_hbm(shape, args.hbm_reps)}
        print(json.dumps(res), flush=True)
        return
    case = si.make_case(wl, batch)
    shape = case.shape
    dt = shape.dtype
    dev = "cuda:0"
    torch.cuda.set_device(0)

    def up(a):
        h = si.host_array(a, dt)
        if dt == "bf16":
            return torch.from_numpy(h.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(h).to(dev)

    enc = ftx.Encoder(shape.batch, shape.seq_len, shape.head_num, shape.size_per_head,
                      shape.num_layers, dt)
    for l, w in enumerate(case.layers()):
        enc.set_weights(l, {k: up(w[k]) for k in si.WEIGHT_NAMES})
    if args.unfused:
        enc.set_option(ftx.FTX_OPT_FUSED_EPILOGUES, 0)
    enc.set_option(ftx.FTX_OPT_FUSED_ATTENTION, args.fused_attention)
    if args.no_fold_layernorm:
        enc.set_option(ftx.FTX_OPT_FOLD_LAYERNORM, 0)
    if args.no_prefetch_weights:
        enc.set_option(ftx.FTX_OPT_PREFETCH_WEIGHTS, 0)
    if args.graph:
        enc.set_option(ftx.FTX_OPT_GRAPH, 1)
    x = up(case.x)
    lens = None if case.lens is None else torch.from_numpy(case.lens).to(dev)
    out = torch.empty_like(x)
    stream = torch.cuda.current_stream()

    if args.copy_calib_mb > 0:
        n = args.copy_calib_mb * (1 << 20) // 2
        src = torch.ones(n, dtype=torch.float16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.neg(src, out=dst)  # reads and writes exactly n * 2 bytes
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        enc.forward(x, lens, out)
    torch.cuda.synchronize()
    # which attention path the handle takes (one forward with launch counts, untimed)
    enc.set_option(ftx.FTX_OPT_KERNEL_TIMING, 1)
    enc.forward(x, lens, out)
    counts = enc.kernel_times()
    attn_fused = counts["qkv_attention"][1] > 0
    # (hidden 128 also has no LayerNorm-1 launch: it runs in the projection's epilogue)
    ln_folded = counts["ln1"][1] == 0 and shape.hidden in (768, 1024)
    w2_prefetch = counts["weight_prefetch"][1] > 0
    enc.set_option(ftx.FTX_OPT_KERNEL_TIMING, 0)
    torch.cuda.synchronize()

    # timed region: K forwards between a synchronize on each side
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        enc.forward(x, lens, out)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = 1e3 * wall / args.steps
    seqs = shape.batch / (ms_per_step * 1e-3)
    flops = shape.flops()
    tflops = flops / (ms_per_step * 1e-3) / 1e12

    result = {
        "metric": METRIC, "value": seqs, "unit": "sequences/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": DTYPE_TAG[dt], "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.description}", "global_batch": shape.batch,
                   "seq_len": shape.seq_len, "layers": shape.num_layers,
                   "heads": shape.head_num, "size_per_head": shape.size_per_head,
                   "parallelism": "none (1 GPU)",
                   "epilogues": "standalone" if args.unfused else "fused",
                   "attention": "in the Q/K/V projection's epilogue" if attn_fused else "own kernel",
                   "layernorm1": "folded into the FFN-in projection" if ln_folded else "own kernel",
                   "w2_prefetch": w2_prefetch,
                   "launch": "hip graph" if args.graph else "stream"},
        "tflops": tflops, "frac_mfma_peak": tflops / PEAK_MFMA_TFLOPS[dt],
        "gpu_event_ms_per_step": gpu_ms / args.steps,
        "roofline": None, "cpu_baseline": None,
    }

    # latency distribution: the same K forwards again, each between its own event pair on the
    # forward's stream (after the timed region, so the headline figure carries no extra events)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        enc.forward(x, lens, out)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    lat = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    result["latency_ms"] = {"p10": float(np.percentile(lat, 10)), "p50": float(np.percentile(lat, 50)),
                            "p90": float(np.percentile(lat, 90))}

    if not args.no_kernel_times:
        # the same K forwards again, with a HIP event pair around every launch on `stream`
        enc.set_option(ftx.FTX_OPT_KERNEL_TIMING, 1)
        enc.kernel_times()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            enc.forward(x, lens, out)
        torch.cuda.synchronize()
        timed_wall = time.perf_counter() - t0
        times = enc.kernel_times()
        enc.set_option(ftx.FTX_OPT_KERNEL_TIMING, 0)
        kernels = {}
        counts = {name: cnt for name, (ms, cnt) in times.items()}
        for name, (ms, cnt) in times.items():
            if cnt == 0:
                continue
            avg = ms / cnt
            fl, by = step_work(shape, name, ln_folded)
            ch = launches_per_layer(counts, name)
            fl, by = fl / ch, by / ch
            kernels[name] = {"avg_us": 1e3 * avg, "launches": cnt, "share": 0.0,
                             "tflops": fl / (avg * 1e-3) / 1e12 if fl else None,
                             "gbs_algorithmic": by / (avg * 1e-3) / 1e9}
        total = sum(v["avg_us"] * v["launches"] for v in kernels.values())
        for v in kernels.values():
            v["share"] = v["avg_us"] * v["launches"] / total
        dom = max(kernels, key=lambda k: kernels[k]["avg_us"] * kernels[k]["launches"])
        fl, by = step_work(shape, dom, ln_folded)
        ch = launches_per_layer(counts, dom)
        fl, by = fl / ch, by / ch
        avg_s = kernels[dom]["avg_us"] * 1e-6
        if fl > 0 and dom != "attention":
            achieved, peak, unit, bound = fl / avg_s / 1e12, PEAK_MFMA_TFLOPS[dt], "TFLOP/s", "mfma"
        else:
            achieved, peak, unit, bound = by / avg_s / 1e9, PEAK_HBM_GBS, "GB/s", "hbm"
        prof = measured_profile(wl.name, shape.batch, dom)
        traffic = None if prof is None else prof["traffic"]
        result["roofline"] = {
            "kernel": dom, "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
            "frac": achieved / peak, "traffic": traffic,
            "work_per_launch": fl if bound == "mfma" else by,
            "avg_launch_us": kernels[dom]["avg_us"],
            "timing": "HIP event pair around every launch on the forward's stream, "
                      f"{args.steps} forwards after the timed region",
            # the committed rocprofv3 summary of the same kernel code (null when the kernels
            # changed since): its own kernel time, and HBM traffic and MFMA busy over that time
            "profile": None if prof is None else {
                "source": prof["source"], "avg_us": prof["avg_us"],
                "frac": (fl if bound == "mfma" else by) / (prof["avg_us"] * 1e-6)
                        / (1e12 if bound == "mfma" else 1e9) / peak,
                "mfma_busy": prof.get("mfma_busy"),
                "traffic_over_algorithmic": prof["traffic"] / prof["algorithmic_bytes"],
                "traffic_gbs": prof["traffic"] / (prof["avg_us"] * 1e-6) / 1e9},
        }
        result["kernels"] = kernels
        result["ms_per_step_with_kernel_events"] = 1e3 * timed_wall / args.steps

    enc.close()
    if case.lens is not None:
        # the same forward counted on the valid tokens only: projections on sum(len_b) rows,
        # attention over len_b queries and keys
        valid = shape.valid_flops(case.lens)
        result["effective_tflops"] = valid / (ms_per_step * 1e-3) / 1e12
        result["valid_token_fraction"] = float(np.sum(case.lens)) / shape.tokens
    if not args.no_hbm:
        result["elementwise_hbm"] = elementwise_hbm(shape, args.hbm_reps)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def calibrate_gemm(args, wl, batch):
    """The projection GEMMs of one layer, alone: the ftx kernel against the vendor library
    (torch.matmul, which calls hipBLASLt) on the same operands in the same layout (W^T, N x K),
    as a practical ceiling next to the MFMA peak.  The library runs without an epilogue; ftx
    runs plain and, for FFN-in, with its fused bias + GELU.  Each time is the mean of 50
    back-to-back launches after a warm-up of at least 150 ms, from stream events."""
    import torch
    from transformer_encoder_bert_amd import ftx
    shape = wl.shape(batch)
    T, H, F = shape.tokens, shape.hidden, shape.ffn
    tdt = {"fp16": torch.float16, "bf16": torch.bfloat16, "fp32": torch.float32}[shape.dtype]
    dev = "cuda:0"
    g = torch.Generator(device=dev).manual_seed(7)

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.15:
            for _ in range(10):
                fn()
            torch.cuda.synchronize()
        e0.record()
        for _ in range(50):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / 50

    rows = []
    for name, M, N, K in (("Q/K/V projection", T, 3 * H, H), ("attention-output projection", T, H, H),
                          ("FFN-in", T, F, H), ("FFN-out", T, H, F)):
        a = torch.randn(M, K, device=dev, dtype=tdt, generator=g)
        w_t = torch.randn(N, K, device=dev, dtype=tdt, generator=g) * 0.05
        bias = torch.randn(N, device=dev, dtype=tdt, generator=g) * 0.1
        c = torch.empty(M, N, device=dev, dtype=tdt)
        flops = 2.0 * M * N * K
        r = {"gemm": name, "M": M, "N": N, "K": K,
             "ftx_plain_us": timed(lambda: ftx.ftx_step_linear(a, w_t, None, False, c)),
             "library_plain_us": timed(lambda: torch.matmul(a, w_t.t()))}
        if name == "FFN-in":
            r["ftx_bias_gelu_us"] = timed(lambda: ftx.ftx_step_linear(a, w_t, bias, True, c))
        for k in [k for k in r if k.endswith("_us")]:
            r[k.replace("_us", "_tflops")] = flops / r[k] * 1e-6
        rows.append(r)
        del a, w_t, bias, c
    res = {"workload": wl.name, "batch": batch, "dtype": shape.dtype, "library": "torch.matmul (hipBLASLt)",
           "kernel_source_hash": kernel_source_hash(), "gemm_calibration": rows}
    print(json.dumps(res), flush=True)


def summarize_calibration(args):
    """profiles/<name>.md from the JSON line of a --calibrate-gemm run."""
    res = json.loads([l for l in open(args.summarize_calibration) if l.startswith("{")][-1])
    wl, batch = res["workload"], res["batch"]
    flags = (f" --workload {wl}" if wl != WORKLOAD_DEFAULT else "") + f" --batch {batch}"
    src = os.path.relpath(os.path.abspath(args.summarize_calibration), ROOT)
    lines = [f"# Projection GEMMs alone: ftx against the library -- {wl}, batch {batch}, {res['dtype']}", "",
             "Commands (from the repository root, on one MI355X):", "", "```",
             f"python3 bench.py{flags} --calibrate-gemm > {src}",
             f"python3 bench.py --summarize-calibration {src} --summary-name {args.summary_name}", "```", "",
             "Mean of 50 back-to-back launches after a 150 ms warm-up, stream events.  The library",
             "(torch.matmul, which calls hipBLASLt) multiplies the same operands in the same layout",
             "(A row-major M x K, weights as W^T, N x K) without an epilogue; ftx runs plain and, for",
             "FFN-in, with its fused bias + GELU.  TFLOP/s against the 2516.6 dense peak.", "",
             "| GEMM | M x N x K | ftx plain us (TFLOP/s) | library us (TFLOP/s) | ftx with bias+GELU us (TFLOP/s) |",
             "|---|---|---|---|---|"]
    for r in res["gemm_calibration"]:
        gl = (f"{r['ftx_bias_gelu_us']:.1f} ({r['ftx_bias_gelu_tflops']:.0f})" if "ftx_bias_gelu_us" in r else "")
        lines.append(f"| {r['gemm']} | {r['M']} x {r['N']} x {r['K']} | {r['ftx_plain_us']:.1f} "
                     f"({r['ftx_plain_tflops']:.0f}) | {r['library_plain_us']:.1f} ({r['library_plain_tflops']:.0f}) | {gl} |")
    lines += ["", f"Kernel source hash: `{res['kernel_source_hash']}`"]
    path = os.path.join(ROOT, "profiles", args.summary_name + ".md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)


def elementwise_hbm(shape, reps: int):
    """HBM GB/s of the element-wise kernels (bias + residual + LayerNorm, standalone bias +
    GELU, standalone bias + head split) at this workload's shape, each launch timed alone with
    the last-level cache flushed first: FLUSH_BYTES are read before every timed launch, so
    the kernel's inputs come from HBM, not from the 256 MB MALL or the L2s.  Algorithmic
    bytes (inputs read once, output written once) over the median event time.  An event pair
    around one launch adds a few microseconds; the kernel trace of --hbm-only
    (--summarize-hbm) gives the kernel time itself."""
    import torch
    from transformer_encoder_bert_amd import ftx
    dev = "cuda:0"
    dt = {"fp16": torch.float16, "bf16": torch.bfloat16, "fp32": torch.float32}[shape.dtype]
    e = 4 if shape.dtype == "fp32" else 2
    T, H, F = shape.tokens, shape.hidden, shape.ffn
    g = torch.Generator(device=dev)
    g.manual_seed(7)

    def rnd(*sz):
        return torch.randn(*sz, generator=g, device=dev, dtype=torch.float32).to(dt)

    x, a, y = rnd(T, H), rnd(T, H), torch.empty(T, H, dtype=dt, device=dev)
    bias, gamma, beta = rnd(H), rnd(H), rnd(H)
    u, bias_f, gel = rnd(T, F), rnd(F), torch.empty(T, F, dtype=dt, device=dev)
    qkv, bias3 = rnd(T, 3 * H), rnd(3 * H)
    q, k, vt = (torch.empty(T * H, dtype=dt, device=dev) for _ in range(3))
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    B, S, n, d = shape.batch, shape.seq_len, shape.head_num, shape.size_per_head
    kernels = {
        "bias_residual_layernorm": (lambda: ftx.ftx_step_bias_residual_layernorm(x, a, bias, gamma, beta, y),
                                    3 * T * H * e),
        "bias_gelu": (lambda: ftx.ftx_step_bias_gelu(u, bias_f, gel), 2 * T * F * e),
        "bias_qkv_split": (lambda: ftx.ftx_step_bias_qkv_split(B, S, n, d, qkv, bias3, q, k, vt),
                           6 * T * H * e),
    }
    stream = torch.cuda.current_stream()
    out = {}
    for name, (fn, nbytes) in kernels.items():
        fn()
        torch.cuda.synchronize()
        times = []
        for r in range(reps):
            torch.sum(flush, dim=0, out=sink)  # reads FLUSH_BYTES
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1) * 1e-3)
        med = float(np.median(times))
        out[name] = {"bytes": nbytes, "median_us": med * 1e6, "min_us": min(times) * 1e6,
                     "gbs": nbytes / med / 1e9, "frac_of_hbm_peak": nbytes / med / 1e9 / PEAK_HBM_GBS}
    out["method"] = (f"each launch alone after reading {FLUSH_BYTES >> 20} MiB (4x the MALL); "
                     f"HIP events around the launch, median of {reps}; algorithmic bytes")
    del flush
    torch.cuda.synchronize()
    return out


if __name__ == "__main__":
    main()
