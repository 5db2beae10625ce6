#!/usr/bin/env python3
"""Bench: FP4-KV decode step on one MI355X, against the FP8/BF16 KV baselines and
the CPU oracle.

One step is one pass of the hot path over a batch: append the new token of every
sequence to the paged cache (rotate + quantize + pack for FP4) and run decode
attention over the whole context (query rotation to E4M3, split-K attention,
merge + inverse rotation).  The FP4 step is one launch of the fused entry point
(uq_append_decode_attention) when every sequence adds one token; the FP4 step with
the PV on the scaled FP4 x FP8 matrix instruction (UQ_FLAG_PV_SCALED) and the
FP8 / BF16 baselines (append kernel, then decode kernel) are reported beside it.
Workloads: 64 sequences x 8,192 context (the headline), 8 x 65,536 and 128 ragged
sequences with 256-token appends; 64 (32) query heads / 8 (4) KV heads,
head_dim 128, 16-token pages randomly permuted.

Prints one JSON line.  Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 / bf16 matrix peak, vendor figure
METRIC = "FP4-KV decode-attn us/step & HBM GB/s (% peak), 64 seq x 8K ctx GQA"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="before the warm-up steps, run steps for this long so that the GPU clocks reach their "
                         "sustained-load state (a cold start reads ~5%% slow)")
    ap.add_argument("--workloads", default="decode_gqa,long,ragged",
                    help="decode workloads to time, comma-separated; the first is the headline")
    ap.add_argument("--no-baselines", action="store_true", help="skip the FP8/BF16 KV kernels")
    ap.add_argument("--no-pv-scaled", action="store_true",
                    help="skip the FP4 step with the PV on the scaled FP4 x FP8 MFMA (UQ_FLAG_PV_SCALED)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the chunked-prefill measurement")
    ap.add_argument("--no-append", action="store_true", help="skip the append-only measurement")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="time each oracle worker may spend building its pairs' caches before the timed step")
    ap.add_argument("--scrub-mb", type=int, default=1024,
                    help="read a buffer of this size before every scrubbed step, so that the 256 MB last-level "
                         "cache holds no cache page; the headline is the scrubbed step")
    ap.add_argument("--oracle-times", action="store_true",
                    help="time only the CPU oracle on every configuration (tiny, the 65,536 x 8 append, "
                         "decode_gqa, long, ragged) on this host's cores and print one JSON line; no GPU")
    ap.add_argument("--pmc-pass", choices=sorted(PMC_KINDS),
                    help="run only one kernel's calls and a 1 GiB device copy (for rocprofv3 --pmc runs)")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="ARG",
                    help="KIND CSV [CSV ...]: write the counter summary of one --pmc-pass kind from rocprofv3 "
                         "counter_collection.csv files into profiles/")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("KIND", "STATS_CSV", "TRACE_CSV"),
                    help="write the kernel-trace summary of one kind (decode, prefill) from a rocprofv3 "
                         "--kernel-trace --stats run into profiles/")
    return ap.parse_args()


def make_workload(name):
    from bit_kv_cache_wht_amd import workloads as W
    if name == "decode_gqa":
        return W.decode_gqa(new=1)
    if name == "long":
        return W.long_context(new=1)
    if name == "ragged":
        return W.ragged()
    return W.tiny()


# the kernel sources and the compiler flags (build.py) that fix the decode binary
DECODE_SOURCES = ["bit_kv_cache_wht_amd/csrc/uq_decode.hip", "bit_kv_cache_wht_amd/csrc/uq_device.h",
                  "bit_kv_cache_wht_amd/csrc/uq_fp4_row.h", "bit_kv_cache_wht_amd/csrc/uq_internal.h",
                  "bit_kv_cache_wht_amd/build.py"]
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_SUMMARY = os.path.join(PROFILES, "decode_fp4_64x8192_hbm_traffic.md")
COPY_BYTES = 1 << 30


def decode_source_sha():
    import hashlib
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per launch of the FP4 decode kernel from the committed counter
    summary, or None if it is missing or was taken on other kernel sources."""
    try:
        with open(TRAFFIC_SUMMARY) as fh:
            text = fh.read()
    except OSError:
        return None
    fields = dict(line.split(":", 1) for line in text.splitlines() if line.startswith(("source_sha256:", "traffic_bytes_per_launch:")))
    if fields.get("source_sha256", "").strip() != decode_source_sha():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"].strip())
    except (KeyError, ValueError):
        return None


# Counter passes (rocprofv3 --pmc), one kernel per kind.  Each pass runs the
# kernel's calls and then a device copy of COPY_BYTES, which calibrates
# FETCH_SIZE / WRITE_SIZE; the summary is written by --summarize-pmc.
PMC_KINDS = {
    "decode": dict(match=("decode_kernel", "Fp4PairPol"), workload="decode_gqa_64x8192, fused FP4 step",
                   out="decode_fp4_64x8192_counters.md"),
    "append": dict(match=("append_fp4_stream_kernel",), workload="append_65536x8x128, bf16 K/V",
                   out="append_fp4_65536x8_counters.md"),
    "prefill": dict(match=("prefill_kernel",), workload="ragged_128, 256-token chunks",
                    out="prefill_fp4_ragged_counters.md"),
}
PMC_PASSES = [["FETCH_SIZE"], ["WRITE_SIZE"],
              ["SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"],
              ["SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_VALU_MFMA_MOPS_F6F4", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES"]]
MI355X_CUS = 256
MI355X_XCDS = 8


def read_counters(paths, match):
    """{counter: [value per dispatch]} of the kernel whose name holds every string
    of `match`, and {counter: largest value} of the runtime's copy kernel."""
    import csv
    kern, copy = {}, {}
    for path in paths:
        with open(path, newline="") as fh:
            for row in csv.DictReader(fh):
                name, counter, value = row.get("Kernel_Name", ""), row.get("Counter_Name"), row.get("Counter_Value")
                if counter is None or value is None:
                    continue
                if all(m in name for m in match):
                    kern.setdefault(counter, []).append(float(value))
                elif "copyBuffer" in name:
                    copy[counter] = max(copy.get(counter, 0.0), float(value))
    return kern, copy


def summarize_counters(kind, paths):
    """Writes profiles/<kind summary>: per-dispatch means of every counter of the
    kind's kernel, HBM bytes (FETCH_SIZE / WRITE_SIZE scaled by the copy of
    COPY_BYTES), MFMA busy fraction and instruction mix.  For the decode it also
    writes the traffic summary the bench's roofline reports."""
    k = PMC_KINDS[kind]
    kern, copy = read_counters(paths, k["match"])
    if not kern:
        raise SystemExit(f"no dispatches of {' '.join(k['match'])} in {paths}")
    mean = {c: float(np.mean(v)) for c, v in kern.items()}
    lines = [f"# Counters of the {kind} kernel on {k['workload']}", "",
             "Each counter set is one rocprofv3 run of the same program; then",
             f"`python3 bench.py --summarize-pmc {kind} <csv files>`:", ""]
    for ctrs in PMC_PASSES:
        lines.append(f"    rocprofv3 --pmc {' '.join(ctrs)} --output-format csv -d <dir> -o <name> -- "
                     f"python3 bench.py --pmc-pass {kind}")
    lines += ["", "| counter | dispatches | mean per dispatch |", "|---|---|---|"]
    for c in sorted(mean):
        lines.append(f"| {c} | {len(kern[c])} | {mean[c]:.6g} |")
    lines += ["", "Derived (per dispatch):", ""]
    derived = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        if c in mean and copy.get(c):
            factor = COPY_BYTES / (copy[c] * 1024.0)
            derived[c] = mean[c] * 1024.0 * factor
            lines.append(f"- {c}: {mean[c]:.0f} KiB x {factor:.4f} (a {COPY_BYTES}-byte copy reads "
                         f"{copy[c]:.0f} KiB) = {derived[c]:.4g} bytes")
    if "FETCH_SIZE" in derived and "WRITE_SIZE" in derived:
        derived["traffic"] = derived["FETCH_SIZE"] + derived["WRITE_SIZE"]
        lines.append(f"- HBM traffic: {derived['traffic']:.4g} bytes")
    if "GRBM_GUI_ACTIVE" in mean:
        # GRBM_GUI_ACTIVE is summed over the 8 XCDs: elapsed cycles = value / 8
        cycles = mean["GRBM_GUI_ACTIVE"] / MI355X_XCDS
        lines.append(f"- elapsed: GRBM_GUI_ACTIVE / {MI355X_XCDS} XCDs = {cycles:.4g} cycles "
                     f"({cycles / 2.4e3:.1f} us at 2.4 GHz)")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
            busy = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * MI355X_CUS * 4)
            derived["mfma_busy"] = busy
            lines.append(f"- MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (elapsed cycles x {MI355X_CUS} CUs x 4 SIMDs) = "
                         f"{busy:.2%}")
    if mean.get("SQ_INSTS_MFMA"):
        lines.append(f"- VALU : MFMA instructions = {mean['SQ_INSTS_VALU'] / mean['SQ_INSTS_MFMA']:.2f}")
    mops = sum(mean.get(c, 0.0) for c in ("SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_VALU_MFMA_MOPS_F6F4"))
    if mops:
        lines.append(f"- MFMA work counted: {mops * 512:.4g} flops (MOPS x 512: f16 "
                     f"{mean.get('SQ_INSTS_VALU_MFMA_MOPS_F16', 0):.4g}, f8f6f4 "
                     f"{mean.get('SQ_INSTS_VALU_MFMA_MOPS_F6F4', 0):.4g}; the block-scaled FP4 x FP8 MFMAs of "
                     f"the QK product read 0 in these MOPS counters)")
    if kind == "append" and "SQ_INSTS_VALU" in mean:
        elems = 65536 * 8 * 2 * 128
        lines.append(f"- VALU lane instructions per element: SQ_INSTS_VALU x 64 / {elems} = "
                     f"{mean['SQ_INSTS_VALU'] * 64 / elems:.2f}")
    lines += ["", f"source_sha256: {decode_source_sha()}", ""]
    out = os.path.join(PROFILES, k["out"])
    with open(out, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))
    if kind == "decode" and "traffic" in derived:
        write_traffic_summary(derived, kern, copy)
    return derived


def write_traffic_summary(derived, kern, copy):
    lines = ["# HBM traffic of the FP4 decode kernel (fused step) on decode_gqa", "",
             "From the FETCH_SIZE and WRITE_SIZE passes of `python3 bench.py --pmc-pass decode` (see",
             "decode_fp4_64x8192_counters.md), each scaled by what the counter reads for a device copy of",
             f"{COPY_BYTES} bytes.", "",
             "| counter | decode dispatches | decode bytes |", "|---|---|---|"]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        lines.append(f"| {c} | {len(kern[c])} | {derived[c]:.4g} |")
    lines += ["", f"source_sha256: {decode_source_sha()}", f"traffic_bytes_per_launch: {int(round(derived['traffic']))}",
              ""]
    with open(TRAFFIC_SUMMARY, "w") as fh:
        fh.write("\n".join(lines))


TRACE_KINDS = {
    "decode": dict(match="Fp4PairPol", out="decode_fp4_64x8192_kernel_trace.md",
                   cmd="rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o trace -- python3 -u bench.py "
                       "--workloads decode_gqa --no-cpu-baseline --no-prefill --no-append",
                   title="decode_gqa 64 x 8192 (64 q / 8 kv heads, d 128), FP4 step = one fused launch"),
    "prefill": dict(match="prefill_kernel", out="prefill_fp4_ragged_kernel_trace.md",
                    cmd="rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o trace -- python3 -u bench.py "
                        "--workloads ragged --no-cpu-baseline --no-baselines --no-pv-scaled --no-append",
                    title="chunked prefill on ragged_128 (128 sequences, 256-token chunks, 32 q / 4 kv heads, d 128)"),
}


def _csv_rows(path):
    import csv
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def summarize_trace(kind, stats_csv, trace_csv):
    """profiles/ summary of a rocprofv3 --kernel-trace --stats run of the command in
    TRACE_KINDS[kind]: the per-kernel statistics, and for the decode the FP4 launches
    of bench.py's passes taken from the dispatch order (the last `steps` of them are
    the event-pair pass after a 1 GiB read each, the `steps` before that the
    whole-step pass after the same read, the `steps` before those the warm pass)."""
    k = TRACE_KINDS[kind]
    stats = _csv_rows(stats_csv)
    pick = lambda row, *names: next(row[n] for n in names if n in row)
    lines = [f"# Kernel trace: {k['title']}", "", "Command (from the repository root):", "", f"    {k['cmd']}", "",
             f"then `python3 bench.py --summarize-trace {kind} <dir>/trace_kernel_stats.csv "
             "<dir>/trace_kernel_trace.csv`.", "",
             "| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---|---|---|---|---|"]
    rows = sorted(stats, key=lambda r: -float(pick(r, "TotalDurationNs")))
    for r in rows[:12]:
        name = pick(r, "Name", "KernelName")
        name = name if len(name) <= 100 else name[:97] + "..."
        lines.append(f"| `{name}` | {pick(r, 'Calls')} | {float(pick(r, 'AverageNs')) / 1e3:.2f} | "
                     f"{float(pick(r, 'MinNs')) / 1e3:.2f} | {float(pick(r, 'MaxNs')) / 1e3:.2f} | "
                     f"{float(pick(r, 'Percentage')):.2f} |")
    trace = _csv_rows(trace_csv)
    durs = [(int(pick(r, "Start_Timestamp")), (int(pick(r, "End_Timestamp")) - int(pick(r, "Start_Timestamp"))) / 1e3)
            for r in trace if k["match"] in pick(r, "Kernel_Name", "KernelName")]
    durs = [d for _, d in sorted(durs)]
    lines.append("")
    if kind == "decode" and len(durs) >= 300:
        n = 100
        warm, whole, ev = durs[-3 * n:-2 * n], durs[-2 * n:-n], durs[-n:]
        lines += [f"FP4 decode launches ({k['match']}, {len(durs)} in all), the last three passes of {n}:", "",
                  f"- warm (back to back): mean {np.mean(warm):.2f} us, median {np.median(warm):.2f} us",
                  f"- whole steps after a 1 GiB read each: mean {np.mean(whole):.2f} us, median "
                  f"{np.median(whole):.2f} us",
                  f"- event-pair and clock pass after a 1 GiB read each: mean {np.mean(ev):.2f} us, median "
                  f"{np.median(ev):.2f} us (bench `roofline.kernel_us` is the mean of the kernel's own clock "
                  "span over the same launches)"]
    elif durs:
        lines += [f"`{k['match']}` launches: {len(durs)}, mean {np.mean(durs):.2f} us, median {np.median(durs):.2f} us"]
    lines.append("")
    with open(os.path.join(PROFILES, k["out"]), "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def stream_read_gbs(reps=20):
    """Read bandwidth of the library's plain streaming-read kernel (uq_stream_read)
    in the same process: a 2 GiB buffer, each byte loaded once, HIP events around
    `reps` back-to-back launches after 5 untimed ones; also the same for torch's
    max over that buffer (another read-only kernel, for comparison)."""
    import torch
    import bit_kv_cache_wht_amd as uq
    x = torch.ones((2 << 30) // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {}
    for name, fn in (("uq_stream_read", lambda: uq.uq_stream_read(x, sink)), ("torch_max", lambda: x.max())):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = x.numel() * 4 / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
    del x, sink
    torch.cuda.empty_cache()
    return res


def append_throughput(steps, warmup, settle_s):
    """The FP4 write path alone on the append workload (65,536 tokens x 8 KV heads x
    head_dim 128, bf16, permuted pages): quantized tokens/s and HBM GB/s of one
    uq_quantize_append call (HIP events around the K timed calls, one launch each)."""
    import torch
    import bit_kv_cache_wht_amd as uq
    from bit_kv_cache_wht_amd import workloads as W
    wl = W.append_only()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    k = dev(wl.k.view(np.int16)).view(torch.bfloat16)
    v = dev(wl.v.view(np.int16)).view(torch.bfloat16)
    slots = dev(wl.slot_mapping)
    cache = uq.KvCache.allocate(uq.UQ_KV_FP4, wl.num_pages, wl.num_kv_heads, wl.head_dim)
    call = lambda: uq.uq_quantize_append(cache, k, v, slots)
    t = time.perf_counter()
    while time.perf_counter() - t < settle_s:
        for _ in range(20):
            call()
        torch.cuda.synchronize()
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / steps * 1e3
    T, H, d = wl.total_tokens, wl.num_kv_heads, wl.head_dim
    algo = T * H * 2 * (2 * d + fp4_kv_bytes_per_token_head(d) // 2) + T * 4   # bf16 K/V in, codes+scales out, slots
    return {"workload": f"{wl.name}: {T} tokens x {H} kv heads x head_dim {d}, bf16, permuted pages",
            "us_per_call": round(us, 2), "quantized_tokens_per_s": round(T / (us * 1e-6)),
            "token_heads_per_s": round(T * H / (us * 1e-6)), "gbs": round(algo / (us * 1e-6) / 1e9, 1),
            "frac_hbm_peak": round(algo / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "algo_bytes_per_call": algo}


def prefill_throughput(reps, warmup):
    """Chunked-prefill attention over the FP4 cache on the ragged workload (128
    sequences of 1k..32k tokens, 32 q heads / 4 kv heads, head_dim 128, bf16; the
    last 256 tokens of every sequence are the chunk): one uq_prefill_attention call
    per rep, HIP events around the `reps` timed calls.  Useful flops count only the
    causal (row, key) pairs: 4 * head_dim flops each (QK and PV)."""
    import torch
    import bit_kv_cache_wht_amd as uq
    from bit_kv_cache_wht_amd import workloads as W
    wl = W.ragged()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    bf = lambda a: dev(a.view(np.int16)).view(torch.bfloat16)
    cache = uq.KvCache.allocate(uq.UQ_KV_FP4, wl.num_pages, wl.num_kv_heads, wl.head_dim)
    for i in range(0, wl.total_tokens, 1 << 18):
        j = np.arange(i, min(i + (1 << 18), wl.total_tokens))
        uq.uq_quantize_append(cache, bf(wl.k[j]), bf(wl.v[j]), dev(wl.slot_mapping[j]))
    q, cu = W.prefill_queries(wl)
    qd, cud, pt, sl = bf(q), dev(cu), dev(wl.page_table), dev(wl.seq_lens)
    out = torch.empty((q.shape[0], wl.num_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
    scale = float(np.float32(1.0 / np.sqrt(wl.head_dim)))
    call = lambda: uq.uq_prefill_attention(cache, qd, cud, pt, sl, scale, out)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    ql = np.diff(cu).astype(np.int64)
    L = wl.seq_lens.astype(np.int64)
    pairs = int(sum((L[b] - ql[b] + np.arange(1, ql[b] + 1)).sum() for b in range(wl.batch))) * wl.num_q_heads
    tflops = 4 * wl.head_dim * pairs / (ms * 1e-3) / 1e12
    del cache, qd, out
    torch.cuda.empty_cache()
    return {"workload": f"{wl.name}: {wl.batch} seq, {int(ql[0])}-token chunk after each prefix "
                        f"({int(L.min())}..{int(L.max())} tokens), {wl.num_q_heads} q heads / {wl.num_kv_heads} kv heads, "
                        f"head_dim {wl.head_dim}, bf16 queries, FP4 cache",
            "ms_per_call": round(ms, 3), "query_tokens_per_s": round(int(cu[-1]) / (ms * 1e-3)),
            "causal_pairs": pairs, "useful_tflops": round(tflops, 1),
            "peak_tflops_f16_mfma": MFMA_F16_PEAK_TFLOPS,
            "frac_f16_peak": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
            "note": "PV runs as two f16 products (P split hi/lo), so the MFMA work is 1.5x the useful flops"}


def pmc_pass(args):
    """One kernel's calls (the --pmc-pass kind), then a plain device copy of
    COPY_BYTES that calibrates the traffic counters."""
    import torch
    torch.cuda.set_device(0)
    if args.pmc_pass == "decode":
        r = Runner("fp4", make_workload("decode_gqa"), fused=True)
        for _ in range(args.warmup + args.steps):
            r.step()
        torch.cuda.synchronize()
        del r
    elif args.pmc_pass == "append":
        append_throughput(args.steps, args.warmup, 0.0)
    else:
        prefill_throughput(max(3, args.steps // 10), 1)
    torch.cuda.empty_cache()
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"pmc pass ({args.pmc_pass}) done")


def fp4_kv_bytes_per_token_head(d):
    return 2 * (d // 2 + d // 32)            # K + V, 17 bytes per 32 elements each


KV_BYTES = {"fp4": lambda d: fp4_kv_bytes_per_token_head(d), "fp8": lambda d: 2 * d, "bf16": lambda d: 4 * d}


class HipEvents:
    """hipEvent_t pairs created and read through the HIP runtime, so that events
    recorded inside libuq (on the kernel's stream) can be timed."""

    def __init__(self, n):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pairs = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(a)) == 0 and self.hip.hipEventCreate(ctypes.byref(b)) == 0
            self.pairs.append((a.value, b.value))

    def elapsed_ms(self, i):
        ms = self.ct.c_float()
        st = self.hip.hipEventElapsedTime(self.ct.byref(ms), self.pairs[i][0], self.pairs[i][1])
        assert st == 0, f"hipEventElapsedTime failed ({st})"
        return ms.value

    def close(self):
        for a, b in self.pairs:
            self.hip.hipEventDestroy(a)
            self.hip.hipEventDestroy(b)


class Runner:
    """Holds device buffers for one format and runs steps through the C ABI."""

    def __init__(self, fmt, wl, fused=False, flags=0):
        import torch
        import bit_kv_cache_wht_amd as uq
        self.fmt, self.wl, self.uq, self.torch, self.flags = fmt, wl, uq, torch, flags
        fid = {"fp4": uq.UQ_KV_FP4, "fp8": uq.UQ_KV_FP8, "bf16": uq.UQ_KV_BF16}[fmt]
        self.append = {"fp4": uq.uq_quantize_append, "fp8": uq.uq_append_fp8, "bf16": uq.uq_append_bf16}[fmt]
        self.decode = {"fp4": uq.uq_decode_attention, "fp8": uq.uq_decode_attention_fp8,
                       "bf16": uq.uq_decode_attention_bf16}[fmt]
        d = wl.head_dim
        self.cache = uq.KvCache.allocate(fid, wl.num_pages, wl.num_kv_heads, d)
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        kv = (lambda a: dev(a.view(np.int16)).view(torch.bfloat16)) if wl.in_dtype == "bf16" else dev
        new = wl.new_token_index()
        pre = wl.prefix_token_index()
        # untimed prefill of the prefix, in chunks to bound host->device staging
        for i in range(0, len(pre), 1 << 18):
            idx = pre[i:i + (1 << 18)]
            self.append(self.cache, kv(wl.k[idx]), kv(wl.v[idx]), dev(wl.slot_mapping[idx]))
        self.k_new, self.v_new = kv(wl.k[new]), kv(wl.v[new])
        self.slots_new = dev(wl.slot_mapping[new])
        self.q = kv(wl.q)
        self.page_table = dev(wl.page_table)
        self.seq_lens = dev(wl.seq_lens)
        self.out = torch.empty((wl.batch, wl.num_q_heads, d), dtype=torch.float32, device="cuda")
        self.ws = torch.zeros(uq.uq_decode_workspace_bytes(self.cache, wl.batch, wl.num_q_heads,
                                                           wl.page_table.shape[1]), dtype=torch.uint8, device="cuda")
        self.sm_scale = float(np.float32(1.0 / np.sqrt(d)))
        # the fused step writes one token per sequence, at position seq_lens[b] - 1
        self.fused = fused and fmt == "fp4" and bool(np.all(wl.new_lens == 1))
        if self.fused:
            self.k_new = self.k_new.reshape(wl.batch, wl.num_kv_heads, d)
            self.v_new = self.v_new.reshape(wl.batch, wl.num_kv_heads, d)
        torch.cuda.synchronize()

    def step(self, ev=None, ev_app=None, clk=None):
        """One step; `ev`: a hipEvent_t pair the library records around its decode
        kernel; `ev_app`: torch events recorded around the append launch; `clk`: a
        device pair the decode kernel fills with its wall-clock span."""
        if clk is not None:
            self.clock_khz = self.uq.uq_profile_next_decode_clock(clk)
        if self.fused:
            if ev is not None:
                self.uq.uq_profile_next_decode(ev[0], ev[1])
            self.uq.uq_append_decode_attention(self.cache, self.k_new, self.v_new, self.q, self.page_table,
                                               self.seq_lens, self.sm_scale, self.out, self.ws, flags=self.flags)
            return
        if ev_app is not None:
            ev_app[0].record()
        self.append(self.cache, self.k_new, self.v_new, self.slots_new)
        if ev_app is not None:
            ev_app[1].record()
        if ev is not None:
            self.uq.uq_profile_next_decode(ev[0], ev[1])
        self.decode(self.cache, self.q, self.page_table, self.seq_lens, self.sm_scale, self.out, self.ws,
                    flags=self.flags)

    def run(self, steps, warmup, scrub=None, settle_s=0.0):
        """After `settle_s` seconds of untimed steps and `warmup` more:
        - warm: `steps` whole steps back to back between two HIP events (nothing
          else in the timed region);
        - scrubbed: `steps` steps each preceded by a read of `scrub` (a device
          tensor larger than the last-level cache, outside the timed events),
          timed in three passes by events on the launch stream: around the
          whole step, around the decode kernel alone (recorded by the library)
          and around the append launch of a two-launch step."""
        torch = self.torch
        t_settle = time.perf_counter()
        while time.perf_counter() - t_settle < settle_s:
            for _ in range(20):
                self.step()
            torch.cuda.synchronize()
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        ev = lambda: torch.cuda.Event(enable_timing=True)
        t0, t1 = ev(), ev()
        wall0 = time.perf_counter()
        t0.record()
        for _ in range(steps):
            self.step()
        t1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        res = dict(warm_ms_per_step=t0.elapsed_time(t1) / steps, wall_ms_per_step=1e3 * wall / steps)
        # whole steps and single kernels are timed in separate passes, so that no
        # step carries more than one pair of events
        whole = [(ev(), ev()) for _ in range(steps)]
        for i in range(steps):
            if scrub is not None:
                scrub.max()                        # a read: evicts without leaving dirty lines
            whole[i][0].record()
            self.step()
            whole[i][1].record()
        torch.cuda.synchronize()
        evs = HipEvents(steps)
        clocks = torch.zeros((steps, 2), dtype=torch.int64, device="cuda")
        clocks[:, 0] = -1                          # the unsigned maximum
        for i in range(steps):
            if scrub is not None:
                scrub.max()
            self.step(evs.pairs[i], clk=clocks[i])
        torch.cuda.synchronize()
        ticks = clocks.cpu().numpy().view(np.uint64).astype(np.float64)
        app = None
        if not self.fused:
            app = [(ev(), ev()) for _ in range(steps)]
            for i in range(steps):
                if scrub is not None:
                    scrub.max()
                self.step(None, app[i])
            torch.cuda.synchronize()
        stat = lambda v: dict(mean=float(np.mean(v)), median=float(np.median(v)), p10=float(np.percentile(v, 10)),
                              p90=float(np.percentile(v, 90)))
        res["step_ms"] = stat([a.elapsed_time(b) for a, b in whole])
        res["decode_ms"] = stat([evs.elapsed_ms(i) for i in range(steps)])
        res["decode_clock_ms"] = stat(list((ticks[:, 1] - ticks[:, 0]) / self.clock_khz))
        if app is not None:
            res["append_ms"] = stat([a.elapsed_time(b) for a, b in app])
        evs.close()
        return res

    def kernel_bytes(self):
        """Algorithmic bytes of one decode launch -- every cached K/V byte of every
        context token once, the query as read, the output written, the page-table
        entries of the context, and for the fused step the new tokens' K/V rows
        read and their cache bytes written -- and of one append launch of a
        two-launch step (new rows read, cache bytes and slots); split partials
        are overhead and not counted."""
        wl = self.wl
        d = wl.head_dim
        in_bytes = 2 if wl.in_dtype == "bf16" else 4
        lens = wl.seq_lens.astype(np.int64)
        kv = int(lens.sum()) * wl.num_kv_heads * KV_BYTES[self.fmt](d)
        q = wl.batch * wl.num_q_heads * d * in_bytes
        out = wl.batch * wl.num_q_heads * d * 4
        pt = int(((lens + 15) // 16).sum()) * 4
        new_rows = int(wl.new_lens.astype(np.int64).sum()) * wl.num_kv_heads
        row_write = KV_BYTES[self.fmt](d)                 # K and V cache bytes of one (token, head)
        new = new_rows * (2 * d * in_bytes + row_write)
        decode = kv + q + out + pt + (new if self.fused else 0)
        append = 0 if self.fused else new + int(wl.new_lens.sum()) * 4
        return dict(decode=decode, append=append, kv=kv, new_rows=new_rows)


def _oracle_pair_prepare(wl, pair):
    """Oracle cache of one (sequence, KV head) pair holding the prefix (untimed)."""
    import oracle as O
    b, hk = divmod(int(pair), wl.num_kv_heads)
    L, d = int(wl.seq_lens[b]), wl.head_dim
    npg = (L + 15) // 16
    t0, n_new = int(wl.tok_offsets[b]), int(wl.new_lens[b])
    kp, vp = O.new_pool(O.FMT_FP4, npg, 1, d), O.new_pool(O.FMT_FP4, npg, 1, d)
    if L > n_new:                                        # a prefix (the tiny config has none)
        O.append(O.FMT_FP4, kp, vp, wl.k[t0:t0 + L - n_new, hk:hk + 1], wl.v[t0:t0 + L - n_new, hk:hk + 1],
                 np.arange(L - n_new, dtype=np.int32), in_dtype=wl.in_dtype)
    return b, hk, kp, vp


def _oracle_pair_step(wl, prepared):
    """The step for one pair: append of its new token(s), decode of its query heads."""
    import oracle as O
    b, hk, kp, vp = prepared
    G, d = wl.num_q_heads // wl.num_kv_heads, wl.head_dim
    L, t0, n_new = int(wl.seq_lens[b]), int(wl.tok_offsets[b]), int(wl.new_lens[b])
    O.append(O.FMT_FP4, kp, vp, wl.k[t0 + L - n_new:t0 + L, hk:hk + 1], wl.v[t0 + L - n_new:t0 + L, hk:hk + 1],
             np.arange(L - n_new, L, dtype=np.int32), in_dtype=wl.in_dtype)
    O.decode_attention_rows(O.FMT_FP4, kp, vp, 1, d, wl.q[b:b + 1, hk * G:(hk + 1) * G],
                            np.arange((L + 15) // 16)[None], np.array([L]), float(np.float32(1 / np.sqrt(d))),
                            [(0, g) for g in range(G)], in_dtype=wl.in_dtype)


def _oracle_worker(wl, pairs, budget_s, barrier, out):
    import threadpoolctl
    with threadpoolctl.threadpool_limits(1):
        t = time.perf_counter()
        prepared = []
        for pair in pairs:
            prepared.append(_oracle_pair_prepare(wl, pair))
            if time.perf_counter() - t > budget_s:
                break
        barrier.wait()
        t0 = time.perf_counter()
        for p in prepared:
            _oracle_pair_step(wl, p)
        t1 = time.perf_counter()
    out.put((len(prepared), t0, t1))


def oracle_cores():
    """Host cores for the oracle: those this process may run on, at most 16 (a
    one-GPU share of a GPU host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_baseline(wl, budget_s):
    """The oracle as it stands, on the host cores this process may use: one forked
    worker per core, each with BLAS pinned to one thread, takes (sequence, KV
    head) pairs in a seeded random order and builds their caches with the prefix
    (untimed, within the budget); then all workers run the step on their pairs
    at once (append of the new token(s), decode of the pair's query heads).  The
    wall time of that phase, scaled by all pairs / pairs run, is the value.  Runs
    before this process touches the GPU (the workers are forks)."""
    import multiprocessing as mp
    import platform
    cores = oracle_cores()
    total_pairs = wl.batch * wl.num_kv_heads
    order = np.random.default_rng(0).permutation(total_pairs)
    ctx = mp.get_context("fork")
    barrier, out = ctx.Barrier(cores), ctx.Queue()
    procs = [ctx.Process(target=_oracle_worker, args=(wl, order[w::cores], budget_s, barrier, out))
             for w in range(cores)]
    for p in procs:
        p.start()
    res = [out.get() for _ in procs]
    for p in procs:
        p.join()
    done = sum(r[0] for r in res)
    wall = max(r[2] for r in res) - min(r[1] for r in res)
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        cpu = platform.processor() or cpu
    G = wl.num_q_heads // wl.num_kv_heads
    return {"value": wall * total_pairs / done * 1e6, "unit": "us/step", "cores": cores, "kind": "oracle",
            "cpu": cpu,
            "sample": f"{done} of {total_pairs} (sequence, KV head) pairs on {cores} worker processes at once: "
                      f"append of the new token(s) + decode of its {G} query heads over the full context, "
                      f"float64 numpy; wall time scaled to the whole step (prefix quantization untimed)"}


def _oracle_append_worker(wl, lo, hi, barrier, out):
    import threadpoolctl
    import oracle as O
    with threadpoolctl.threadpool_limits(1):
        kp = O.new_pool(O.FMT_FP4, wl.num_pages, wl.num_kv_heads, wl.head_dim)
        vp = O.new_pool(O.FMT_FP4, wl.num_pages, wl.num_kv_heads, wl.head_dim)
        barrier.wait()
        t0 = time.perf_counter()
        if hi > lo:
            O.append(O.FMT_FP4, kp, vp, wl.k[lo:hi], wl.v[lo:hi], wl.slot_mapping[lo:hi], in_dtype=wl.in_dtype)
        t1 = time.perf_counter()
    out.put((hi - lo, t0, t1))


def cpu_append_baseline(wl):
    """The oracle's FP4 append of the whole workload, its tokens split into one
    contiguous slice per host core (forked workers, BLAS on one thread, each
    with a pool of its own); the wall time from the common start to the last
    worker's end."""
    import multiprocessing as mp
    cores = oracle_cores()
    T = wl.total_tokens
    cuts = [T * w // cores for w in range(cores + 1)]
    ctx = mp.get_context("fork")
    barrier, out = ctx.Barrier(cores), ctx.Queue()
    procs = [ctx.Process(target=_oracle_append_worker, args=(wl, cuts[w], cuts[w + 1], barrier, out))
             for w in range(cores)]
    for p in procs:
        p.start()
    res = [out.get() for _ in procs]
    for p in procs:
        p.join()
    wall = max(r[2] for r in res) - min(r[1] for r in res)
    return {"value": round(wall * 1e6, 1), "unit": "us/call", "cores": cores, "kind": "oracle",
            "tokens_per_s": round(T / wall),
            "sample": f"all {T} tokens x {wl.num_kv_heads} KV heads, one slice of tokens per worker process, "
                      f"float64 numpy"}


def oracle_times(args):
    """The oracle alone on every configuration, on the host cores this process
    may use (no GPU): the whole step of the tiny config, the 65,536 x 8 append,
    and the decode step (append of the new token(s) + decode) of decode_gqa,
    long and ragged, each as cpu_baseline measures it."""
    import platform
    from bit_kv_cache_wht_amd import workloads as W
    res = {}
    for name in ("tiny", "decode_gqa", "long", "ragged"):
        log(f"oracle: generating {name}")
        wl = make_workload(name)
        log(f"oracle: {describe(wl)}")
        res[name] = cpu_baseline(wl, args.cpu_seconds)
        log(f"oracle: {name} {res[name]['value'] / 1e3:.1f} ms per step")
        del wl
    log("oracle: generating the append workload")
    wl = W.append_only()
    res["append_65536x8x128"] = cpu_append_baseline(wl)
    log(f"oracle: append {res['append_65536x8x128']['value'] / 1e3:.1f} ms per call")
    cpu = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    print(json.dumps({"oracle_times": res, "cores": oracle_cores(), "cpu": cpu}), flush=True)


def describe(wl):
    lens = wl.seq_lens
    ctx = f"{int(lens.min())}..{int(lens.max())}" if lens.min() != lens.max() else f"{int(lens.max())}"
    new = int(wl.new_lens.max())
    return (f"{wl.name}: {wl.batch} seq x {ctx} ctx, {wl.num_q_heads} q heads / {wl.num_kv_heads} kv heads, "
            f"head_dim {wl.head_dim}, 16-token pages permuted; step = append of {new} new token(s) per seq + decode")


def time_workload(args, wl, fmts, torch):
    """Per format: the step timed warm and scrubbed (see Runner.run), with the
    decode kernel's rate against the HBM peak."""
    import bit_kv_cache_wht_amd as uq
    out = {}
    for key in fmts:
        # fp4_pv_scaled: the FP4 step with the PV on the scaled FP4 x FP8 MFMA
        fmt, flags = ("fp4", uq.UQ_FLAG_PV_SCALED) if key == "fp4_pv_scaled" else (key, 0)
        log(f"{wl.name} {key}: prefill + timing")
        r = Runner(fmt, wl, fused=fmt == "fp4", flags=flags)
        scrub = torch.ones((args.scrub_mb << 20) // 4, dtype=torch.int32, device="cuda") if args.scrub_mb else None
        res = r.run(args.steps, args.warmup, scrub, settle_s=args.settle_ms * 1e-3)
        by = r.kernel_bytes()
        dec_us = res["decode_clock_ms"]["mean"] * 1e3
        e = {
            "us_per_step": round(res["step_ms"]["median"] * 1e3, 2),
            "us_per_step_p10_p90": [round(res["step_ms"]["p10"] * 1e3, 2), round(res["step_ms"]["p90"] * 1e3, 2)],
            "us_per_step_warm": round(res["warm_ms_per_step"] * 1e3, 2),
            "fused": r.fused,
            "decode_kernel_us": round(dec_us, 2),
            "decode_kernel_us_median": round(res["decode_clock_ms"]["median"] * 1e3, 2),
            "decode_kernel_us_event_pairs": round(res["decode_ms"]["mean"] * 1e3, 2),
            "decode_algo_bytes": by["decode"],
            "decode_gbs": round(by["decode"] / (dec_us * 1e-6) / 1e9, 1),
            "frac_hbm_peak": round(by["decode"] / (dec_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "kv_bytes": by["kv"],
        }
        if r.fused:
            # one launch per step: the warm region times the kernel back to back
            e["decode_gbs_warm"] = round(by["decode"] / (res["warm_ms_per_step"] * 1e-3) / 1e9, 1)
            e["frac_hbm_peak_warm"] = round(e["decode_gbs_warm"] / HBM_PEAK_GBS, 4)
        if "append_ms" in res:
            app_us = res["append_ms"]["mean"] * 1e3
            toks = int(wl.new_lens.sum())
            e["append_us"] = round(app_us, 2)
            e["append_tokens_per_s"] = round(toks / (app_us * 1e-6))
            e["append_algo_bytes"] = by["append"]
            e["append_gbs"] = round(by["append"] / (app_us * 1e-6) / 1e9, 1)
        out[key] = e
        log(f"{wl.name} {key}: {e['us_per_step']} us/step scrubbed ({e['us_per_step_warm']} warm), decode kernel "
            f"{e['decode_kernel_us']} us = {e['decode_gbs']} GB/s ({e['frac_hbm_peak']:.1%})"
            + (f", append {e['append_us']} us" if "append_us" in e else ""))
        del r, scrub
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_counters(args.summarize_pmc[0], args.summarize_pmc[1:])
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.oracle_times:
        oracle_times(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this hot path needs no "
              f"collectives and is benchmarked at N=1", file=sys.stderr)
        sys.exit(2)
    if args.pmc_pass:
        pmc_pass(args)
        return
    names = [w for w in args.workloads.split(",") if w]
    log(f"generating workload {names[0]}")
    t = time.perf_counter()
    wl = make_workload(names[0])
    log(f"workload ready in {time.perf_counter() - t:.1f}s: B={wl.batch} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} "
        f"d={wl.head_dim} tokens={wl.total_tokens}")
    cpu = None
    if not args.no_cpu_baseline:
        log(f"cpu baseline (oracle on {oracle_cores()} host cores; before the GPU is touched)")
        cpu = cpu_baseline(wl, args.cpu_seconds)
    import torch
    torch.cuda.set_device(0)
    fmts = ["fp4"] + ([] if args.no_pv_scaled else ["fp4_pv_scaled"]) + ([] if args.no_baselines else ["fp8", "bf16"])
    results, descr, shape = {}, {}, {}
    for i, name in enumerate(names):
        if i > 0:
            log(f"generating workload {name}")
            wl = make_workload(name)
        descr[name] = describe(wl)
        shape[name] = (int(wl.batch), int(wl.seq_lens.max()))
        results[name] = time_workload(args, wl, fmts, torch)
        del wl
    head = results[names[0]]["fp4"]
    fused = head["fused"]
    traffic = recorded_traffic() if names[0] == "decode_gqa" else None
    line = {
        "metric": METRIC,
        "value": head["us_per_step"],
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(head["us_per_step"] * 1e-3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4_e2m1xfp8_e4m3->f32 (f16 PV)",
        "data": "synthetic (seeded Gaussian K/V with outlier channels, permuted pages)",
        "timing": (f"value: median over {args.steps} steps, each preceded by a read of a {args.scrub_mb} MB buffer "
                   "(outside the timed events) so that no cache page is in the 256 MB last-level cache; HIP "
                   "events on the launch stream around each whole step.  value_warm: the same steps back to "
                   "back, HIP events around all of them"),
        "value_warm": head["us_per_step_warm"],
        "config": {"workload": descr[names[0]] + (" in one fused launch" if fused else ""),
                   "global_batch": shape[names[0]][0], "seq_len": shape[names[0]][1],
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": head["decode_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": head["frac_hbm_peak"], "traffic": traffic,
                     "kernel": "decode_kernel<Fp4PairPol<128>> (KV-head pairs" + (", fused append)" if fused else ")"),
                     "kernel_us": head["decode_kernel_us"],
                     "timing": "mean over the scrubbed steps of the kernel's own span: the device's constant "
                               "wall clock read by the first workgroup as it starts and by the last as it ends "
                               "(uq_profile_next_decode_clock); HIP events the library records around the same "
                               "launches read more (kernel_us_event_pairs: launch overhead included)",
                     "kernel_us_event_pairs": head["decode_kernel_us_event_pairs"],
                     "achieved_warm": head.get("decode_gbs_warm"), "frac_warm": head.get("frac_hbm_peak_warm"),
                     "algo_bytes_per_launch": head["decode_algo_bytes"]},
        "baselines": {f: {"us_per_step": results[names[0]][f]["us_per_step"],
                          "us_per_step_warm": results[names[0]][f]["us_per_step_warm"],
                          "decode_kernel_us": results[names[0]][f]["decode_kernel_us"],
                          "kernel_gbs": results[names[0]][f]["decode_gbs"],
                          "frac_hbm_peak": results[names[0]][f]["frac_hbm_peak"]}
                      for f in fmts if f not in ("fp4", "fp4_pv_scaled")},
        "workloads": {n: dict(description=descr[n], **results[n]) for n in names},
    }
    sr = stream_read_gbs()
    line["roofline"]["stream_read_gbs"] = round(sr["uq_stream_read"], 1)
    line["roofline"]["torch_max_read_gbs"] = round(sr["torch_max"], 1)
    line["roofline"]["frac_of_stream_read"] = round(head["decode_gbs"] / sr["uq_stream_read"], 4)
    log(f"streaming read reference: {sr['uq_stream_read']:.0f} GB/s (torch max {sr['torch_max']:.0f}); "
        f"FP4 decode at {head['decode_gbs'] / sr['uq_stream_read']:.2%} of it")
    if not args.no_append:
        log("append throughput (FP4 write path alone)")
        line["append"] = append_throughput(args.steps, args.warmup, args.settle_ms * 1e-3)
        log(f"append: {line['append']['us_per_call']} us per call, "
            f"{line['append']['quantized_tokens_per_s'] / 1e6:.1f} M tokens/s, {line['append']['gbs']} GB/s")
        torch.cuda.empty_cache()
    if not args.no_prefill:
        log("chunked prefill over the FP4 cache (ragged workload)")
        line["prefill"] = prefill_throughput(max(5, args.steps // 10), 3)
        log(f"prefill: {line['prefill']['ms_per_call']} ms per call, {line['prefill']['useful_tflops']} TFLOP/s useful")
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
