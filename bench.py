"""Prefill and decode throughput of the decoder forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Workload (default): the Qwen3-0.6B shape with bf16 weights and an f16 KV cache, random
seeded weights and token ids; one step = one dec_prefill of 32 sequences x 1,024 prompt
tokens (last-token logits and greedy next ids) followed by 256 greedy dec_decode_step calls
at batch 32 (next ids passed on the device). W untimed steps, then exactly K timed steps
between two device synchronisations. ``value`` is whole-job tokens/s (prompt + generated
tokens per second); prefill and decode rates are reported beside it. Prefill-only workloads
(the 8 x 2,048 prompts in 512-token chunks; the float32 188-token full path with the logits of
every row) make a step of their prefill calls alone.

``prefill_phase`` / ``decode_phase``: the whole phase against its roofline -- the prefill's
algorithmic flops (projections, the causal half of attention, the LM head rows) per prefill
time against the MFMA peak of the products' type, and a decode step's algorithmic bytes (every
weight byte once, every visible key and value once, the logits) per step time against HBM.
``prefill_kernels``: per kernel class, its launches' mean duration and algorithmic flops, from
one pass of the prefill calls with every launch timed, made before the timed steps.

``roofline``: the kernel with the largest share of the timed region's GPU time (decode
attention, HBM-bound, with the combine kernel of rows split into segments; for prefill-only
workloads the largest prefill product), timed live on the library's stream with HIP events
that the launch itself records at the kernel's start and end -- for the decode attention on
the launches of every 32nd decode step of the timed steps; achieved = mean algorithmic bytes
(flops) per launch / mean duration. ``traffic``: HBM bytes per launch from the committed
hardware-counter summary. ``roofline_prefill``: the same for the largest prefill product,
timed on every launch of the timed steps. ``cpu_baseline``: the float64 CPU oracle on a
bounded sample of the same workload (one sequence's prefill and a few decode steps), timed
on this host.

Summaries for profiles/ (no GPU work): --summarize-stats (rocprofv3 --kernel-trace --stats),
--summarize-counters (FETCH_SIZE / WRITE_SIZE runs: the decode attention's HBM traffic),
--summarize-mfma (MFMA busy and MFMA flops executed per prefill kernel, from a --prefill-only
counter run).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFS = 2516.6    # dense bf16 MFMA: 256 CUs x 4096 flop/clk x 2.4 GHz

METRIC = "prefill & decode tokens/s on 1 MI355X; % MFMA / HBM roofline"
MAX_ROWS = 32768               # prompt tokens per prefill call


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="q06b_bf16_b32_p1024_d256")
    ap.add_argument("--no-sampler", action="store_true", help="skip the seeded-sampler timing after the run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--time-every", type=int, default=32,
                    help="time the attention launches of every N-th decode step (0: none)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="first run one device-to-device copy of this many MiB (a reference dispatch of known "
                         "traffic for hardware-counter runs)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE, "
                         "each with --copy-mb) into the profiles/ traffic summary of the decode attention kernel")
    ap.add_argument("--prefill-only", action="store_true",
                    help="run the prefill calls of the workload and no decode step (for counter runs)")
    ap.add_argument("--summarize-mfma", metavar="PMC_DIR",
                    help="no GPU work: turn a rocprofv3 --pmc run of the MFMA counters over this script (with "
                         "--prefill-only) into the profiles/ MFMA-utilisation summary of the prefill kernels")
    ap.add_argument("--summarize-line", metavar="JSON_FILE",
                    help="no GPU work: turn a saved bench line of --workload into its profiles/ summary")
    ap.add_argument("--summarize-stats", metavar="STATS_DIR",
                    help="no GPU work: turn a rocprofv3 --kernel-trace --stats run of this script into the "
                         "profiles/ kernel-time summary")
    return ap.parse_args()


ATTN_SOURCES = ["decoder_forward_pass_amd/csrc/k_attn.hip", "decoder_forward_pass_amd/csrc/common.h",
                "decoder_forward_pass_amd/csrc/kernels.h"]
TRAFFIC_KERNEL = "attn_decode_kernel"


def _sources_sha256(paths):
    import hashlib
    h = hashlib.sha256()
    for src in paths:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _csv_rows(directory, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True))
    if not files:
        sys.exit(f"no *{suffix} under {directory}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def summarize_counters(fetch_dir, write_dir, wl_name, copy_mb):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of every kernel, scaled by what the same counter
    reads for the reference copy of known size, and the decode attention's bytes per launch."""
    from collections import defaultdict
    per = {}
    ref = {}
    for name, directory in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        sums = defaultdict(float)
        for r in _csv_rows(directory, "counter_collection.csv"):
            if r["Counter_Name"] == name:
                sums[(r["Kernel_Name"], r["Dispatch_Id"])] += float(r["Counter_Value"])
        copies = [v for (k, _), v in sums.items() if "copyBuffer" in k]
        ref[name] = max(copies)  # the reference copy is the largest copy dispatch
        agg = defaultdict(list)
        for (k, _), v in sums.items():
            agg[k].append(v)
        per[name] = agg
    ref_bytes = copy_mb << 20
    fscale, wscale = ref_bytes / ref["FETCH_SIZE"], ref_bytes / ref["WRITE_SIZE"]
    rows = []
    for k, vals in per["FETCH_SIZE"].items():
        if "copyBuffer" in k or "fillBuffer" in k:
            continue
        w = per["WRITE_SIZE"].get(k, [0.0])
        rows.append((k, len(vals), np.mean(vals) * fscale, np.mean(w) * wscale, np.mean(vals), np.mean(w)))
    rows.sort(key=lambda r: -(r[1] * (r[2] + r[3])))
    attn = [r for r in rows if TRAFFIC_KERNEL in r[0]]
    if not attn:
        sys.exit("the decode attention kernel is not in the counter runs")
    k, n, fb, wb, fk, wk = attn[0]
    wl = __import__("synthetic").WORKLOADS[wl_name]
    shape = __import__("synthetic").MODELS[wl.model]
    per_key = shape.n_kv_heads * shape.head_dim * 2 * (2 if shape.kv_dtype == "f16" else 4)
    lens = prompt_lengths(wl)
    alg = float(np.mean([attention_bytes(lens, t, per_key) for t in range(wl.decode_steps)]))
    summary = {
        "kernel": k, "workload": f"{wl_name} (decode steps)", "sources": ATTN_SOURCES,
        "source_sha256": _sources_sha256(ATTN_SOURCES), "dispatches": n,
        "fetch_kib_mean": fk, "write_kib_mean": wk, "copy_reference_bytes": ref_bytes,
        "copy_fetch_kib": ref["FETCH_SIZE"], "copy_write_kib": ref["WRITE_SIZE"],
        "fetch_scale": fscale / 1024, "write_scale": wscale / 1024,
        "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb, "traffic_bytes_per_launch": fb + wb,
        "algorithmic_bytes_per_launch": alg,
    }
    base = os.path.join(ROOT, "profiles", f"{TRAFFIC_KERNEL}_{wl_name}_pmc")
    with open(base + ".json", "w") as f:
        json.dump(summary, f, indent=1)
    cmd = ("rocprofv3 --pmc {c} -d gpurun_out/{d} -o run --output-format csv -- python -u bench.py --steps 1 "
           f"--warmup 0 --no-cpu-baseline --copy-mb {copy_mb} --workload {wl_name}")
    lines = [
        f"# HBM traffic: `{TRAFFIC_KERNEL}` on {wl_name} (decode steps)", "",
        "Commands (one MI355X, repo root; one counter per run), then the summary:", "", "```",
        cmd.format(c="FETCH_SIZE", d="pmc_fetch"), cmd.format(c="WRITE_SIZE", d="pmc_write"),
        f"python bench.py --summarize-counters gpurun_out/pmc_fetch gpurun_out/pmc_write --workload {wl_name} "
        f"--copy-mb {copy_mb}", "```", "",
        f"Per-dispatch `Counter_Value` (KiB), averaged over each kernel's dispatches. Calibration: the "
        f"{copy_mb} MiB device-to-device copy that `--copy-mb` runs first (the largest copy dispatch; "
        f"{ref_bytes:,} bytes read and written).", "",
        "| counter | reference copy (KiB) | bytes per KiB | attention mean (KiB/dispatch) | bytes per launch |",
        "|---|---:|---:|---:|---:|",
        f"| FETCH_SIZE | {ref['FETCH_SIZE']:.1f} | {fscale:.1f} | {fk:.1f} | {fb / 1e6:.2f} MB |",
        f"| WRITE_SIZE | {ref['WRITE_SIZE']:.1f} | {wscale:.1f} | {wk:.1f} | {wb / 1e6:.3f} MB |", "",
        f"Dispatches: {n}. Algorithmic bytes per launch (every visible key and value read once): "
        f"{alg / 1e6:.2f} MB, the mean over the decode steps. Measured traffic {(fb + wb) / 1e6:.2f} MB = "
        f"{100 * (fb + wb) / alg:.1f}% of it (the rest: query rows, block tables, output rows, the new keys "
        "and values).", "",
        "All kernels of the run (scaled fetch / write per dispatch):", "",
        "| kernel | dispatches | fetch MB | write MB |", "|---|---:|---:|---:|",
    ]
    for k2, n2, f2, w2, _, _ in rows[:16]:
        lines.append(f"| `{k2.split('(')[0]}` | {n2} | {f2 / 1e6:.1f} | {w2 / 1e6:.2f} |")
    lines += ["", f"Source hash (sha256 of {', '.join(ATTN_SOURCES)}) at measurement: "
              f"`{summary['source_sha256']}`; `bench.py` reports `traffic` only while it matches."]
    with open(base + ".md", "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {base}.json/.md: {(fb + wb) / 1e6:.2f} MB per launch ({100 * (fb + wb) / alg:.1f}% of algorithmic)")


def summarize_stats(stats_dir, wl_name, steps):
    """Kernel time table from rocprofv3 --kernel-trace --stats."""
    rows = _csv_rows(stats_dir, "kernel_stats.csv")
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    cmd = (f"rocprofv3 --kernel-trace --stats -d gpurun_out/prof -o bench --output-format csv -- python -u bench.py "
           f"--steps {steps} --warmup 0 --no-cpu-baseline --workload {wl_name}")
    lines = [f"# Kernel times: bench.py on {wl_name}", "", "Commands (one MI355X, repo root):", "", "```", cmd,
             f"python bench.py --summarize-stats gpurun_out/prof --workload {wl_name} --steps {steps}", "```", "",
             f"{steps} timed step(s) (the workload's prefill calls, then its decode steps), no warm-up; before "
             "them the bench runs the prefill calls once more, untimed, for its per-kernel breakdown, so each "
             "prefill kernel appears once per step plus once.", "",
             "| kernel | calls | total ms | mean us | share |", "|---|---:|---:|---:|---:|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        t = float(r["TotalDurationNs"])
        lines.append(f"| `{r['Name'].split('(')[0]}` | {r['Calls']} | {t / 1e6:.2f} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{100 * t / total:.1f}% |")
    path = os.path.join(ROOT, "profiles", f"bench_{wl_name}_kernel_stats.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {path}")


MFMA_COUNTERS = ["MfmaUtil", "MfmaFlopsBF16", "MfmaFlopsF16", "MfmaFlopsF32", "GRBM_GUI_ACTIVE"]


def summarize_mfma(pmc_dir, wl_name):
    """Per prefill kernel, from one rocprofv3 --pmc run of MFMA_COUNTERS over the prefill-only bench
    step: MFMA busy (MfmaUtil = MFMA busy cycles / (GPU active cycles x SIMDs)), MFMA flops executed
    (the MOPS counters x 512) and the algorithmic flops of the same dispatches."""
    from collections import defaultdict
    from decoder_forward_pass_amd import binding as B
    from synthetic import MODELS, WORKLOADS
    vals = defaultdict(lambda: defaultdict(float))  # (kernel, dispatch) -> counter -> value
    for r in _csv_rows(pmc_dir, "counter_collection.csv"):
        vals[(r["Kernel_Name"], r["Dispatch_Id"])][r["Counter_Name"]] += float(r["Counter_Value"])
    per = defaultdict(list)
    for (k, _), c in vals.items():
        if "copyBuffer" in k or "fillBuffer" in k or "Fill" in k:
            continue
        per[k.split("(")[0]].append(c)
    wl = WORKLOADS[wl_name]
    shape = MODELS[wl.model]
    lens = prompt_lengths(wl)
    per_class, total = prefill_flops(shape, prefill_plan(wl, lens), B)
    L = shape.n_layers
    rows = []
    for k, cs in per.items():
        util = float(np.mean([c.get("MfmaUtil", 0.0) for c in cs]))
        fl = float(np.mean([c.get("MfmaFlopsBF16", 0) + c.get("MfmaFlopsF16", 0) + c.get("MfmaFlopsF32", 0) for c in cs]))
        rows.append((k, len(cs), util, fl))
    rows.sort(key=lambda r: -r[1] * r[3])
    # algorithmic flops per dispatch of the kernels that carry one product each
    import re
    by_epi = {"3": per_class[K_QKV] / L, "2": per_class[K_GATEUP] / L, "1": (per_class[K_O] + per_class[K_DOWN]) / (2 * L)}

    def alg_of(k):  # gemm_big<weight format, epilogue, ...>: the epilogue names the product
        m = re.search(r"gemm_big<\d+, (\d+),", k)
        if m:
            return by_epi.get(m.group(1))
        return per_class[K_ATTN_PF] / L if "attn_prefill_kernel" in k else None
    summary = {"workload": wl_name, "counters": MFMA_COUNTERS, "kernels": []}
    lines = [f"# Prefill MFMA utilisation: {wl_name}", "",
             "Commands (one MI355X, repo root), then the summary:", "", "```",
             f"rocprofv3 --pmc {' '.join(MFMA_COUNTERS)} -d gpurun_out/pmc_mfma -o run --output-format csv -- "
             f"python -u bench.py --steps 1 --warmup 0 --no-cpu-baseline --prefill-only --workload {wl_name}",
             f"python bench.py --summarize-mfma gpurun_out/pmc_mfma --workload {wl_name}", "```", "",
             "`MfmaUtil` is rocprofv3's derived counter: MFMA busy cycles summed over the SIMDs / (GPU active "
             "cycles x SIMDs), in percent, per dispatch. Flops executed are the MFMA MOPS counters x 512. "
             "Algorithmic flops: 2 per multiply-add of the product the kernel computes (the causal half of "
             "attention); the O and down projections share one kernel instantiation, so their mean is shown.", "",
             "| kernel | dispatches | MFMA busy (MfmaUtil) | MFMA TFLOP executed / dispatch | algorithmic TFLOP / dispatch | executed / algorithmic |",
             "|---|---:|---:|---:|---:|---:|"]
    for k, n, util, fl in rows:
        a = alg_of(k)
        ratio = f"{fl / a:.3f}" if a else "-"
        lines.append(f"| `{k}` | {n} | {util:.1f}% | {fl / 1e12:.4f} | {a / 1e12 if a else 0:.4f} | {ratio} |")
        summary["kernels"].append({"kernel": k, "dispatches": n, "mfma_util_pct": util, "mfma_flops_per_dispatch": fl,
                                   "algorithmic_flops_per_dispatch": a})
    lines += ["", "The fraction of the MFMA peak each kernel reaches by its measured duration is in the bench line's "
              "`prefill_kernels` (`frac`) and in the kernel-time summary."]
    base = os.path.join(ROOT, "profiles", f"prefill_mfma_{wl_name}")
    with open(base + ".json", "w") as f:
        json.dump(summary, f, indent=1)
    with open(base + ".md", "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {base}.json/.md")


def summarize_line(path, wl_name, steps, warmup):
    """A bench line saved by `python bench.py --workload W --steps K --warmup W > file` as a
    profiles/ summary: the command, the phase fractions, the per-kernel table and the line."""
    with open(path) as f:
        line = [l for l in f if l.startswith("{")][-1]
    d = json.loads(line)
    cmd = f"python bench.py --workload {wl_name} --steps {steps} --warmup {warmup} > gpurun_out/line_{wl_name}.json"
    lines = [f"# Bench line: {wl_name}", "", "Commands (one MI355X, repo root):", "", "```", cmd,
             f"python bench.py --summarize-line gpurun_out/line_{wl_name}.json --workload {wl_name} --steps {steps} "
             f"--warmup {warmup}", "```", "",
             f"- value: {d['value']:,} {d['unit']} ({d['config']})",
             f"- prefill: {d['prefill_ms']} ms, {d['prefill_tok_s']:,} tok/s; whole phase {d['prefill_phase']['achieved']} "
             f"{d['prefill_phase']['unit']} = {100 * d['prefill_phase']['frac']:.1f}% of {d['prefill_phase']['peak']} "
             f"({d['prefill_phase']['algorithmic_tflop']} TFLOP per step)"]
    if "decode_phase" in d:
        lines.append(f"- decode: {d['decode_ms_per_step']} ms per step, {d['decode_tok_s']:,} tok/s; whole phase "
                     f"{d['decode_phase']['achieved']} GB/s = {100 * d['decode_phase']['frac']:.1f}% of HBM")
    r = d["roofline"]
    lines.append(f"- roofline kernel ({r['kernel']}): {r['achieved']} {r['unit']} = {100 * r['frac']:.1f}% of {r['peak']}")
    if "hardware" in d:
        h = d["hardware"]
        lines.append(f"- device: {h['device']} ({h['arch']}), {h['compute_units']} compute units, clock "
                     f"{h['clock_mhz']} MHz reported; device-to-device copy of {h['stream_copy_mib']} MiB: "
                     f"{h['stream_copy_gbs']} GB/s (read + write) against the 8,000 GB/s peak")
    if "cpu_baseline" in d:
        c = d["cpu_baseline"]
        rates = f"prefill {c['prefill_tok_s']:.1f} tok/s" if "prefill_tok_s" in c else ""
        if "decode_tok_s" in c:
            rates += f", decode {c['decode_tok_s']:.2f} tok/s"
        host = c.get("host") or {}
        lines.append(f"- CPU oracle: {c['value']:.1f} {c['unit']} ({rates}; {c['sample']}) on {c['cores']} cores"
                     + (f", {host.get('cpu_model')}, BLAS {host.get('blas')}" if host else ""))
    lines += ["", "| prefill kernel class | launches | mean us | TFLOP/s | fraction of peak | share of prefill |",
              "|---|---:|---:|---:|---:|---:|"]
    for k, v in d["prefill_kernels"].items():
        lines.append(f"| {k} | {v['launches']} | {v['avg_launch_us']} | {v.get('achieved_tflops', '-')} | "
                     f"{v.get('frac', '-')} | {v['share_of_prefill']} |")
    lines += ["", "The line:", "", "```json", line.strip(), "```"]
    out = os.path.join(ROOT, "profiles", f"bench_{wl_name}_line.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {out}")


def measured_traffic(name):
    """Bytes per launch from the committed hardware-counter summary, or None when the kernel's
    sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name)
    try:
        with open(path) as f:
            d = json.load(f)
        h = hashlib.sha256()
        for src in d["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        return d["traffic_bytes_per_launch"] if h.hexdigest() == d["source_sha256"] else None
    except (OSError, KeyError, ValueError):
        return None


SAMPLER_PARAMS = dict(temperature=0.8, top_k=50, top_p=0.95, repetition_penalty=1.1)


def time_sampler(s, logits, prompts, reps=10):
    """dec_sample over the last decode step's logits (one row per sequence, its prompt as the
    history) with SAMPLER_PARAMS: mean microseconds per call, outside the timed region."""
    import torch
    from decoder_forward_pass_amd import binding as B
    S = logits.shape[0]
    p = B.dec_sampling()
    p.temperature, p.top_k, p.top_p = SAMPLER_PARAMS["temperature"], SAMPLER_PARAMS["top_k"], SAMPLER_PARAMS["top_p"]
    p.min_p, p.repetition_penalty = 0.0, SAMPLER_PARAMS["repetition_penalty"]
    hist = []
    off = 0
    for pr in prompts:
        h = B.dec_history()
        h.prompt_offset, h.prompt_len, h.output_offset, h.output_len = off, len(pr), off + len(pr), 0
        off += len(pr)
        hist.append(h)
    ids = torch.tensor(np.concatenate(prompts), dtype=torch.int32, device="cuda")
    rng = torch.tensor([list(B.dec_rng_stream(i)) for i in range(S)], dtype=torch.uint64, device="cuda")
    for _ in range(2):
        s.sample(logits, [p] * S, hist, ids, rng)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        s.sample(logits, [p] * S, hist, ids, rng)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    return {"kernel": "sample_kernel (seeded sampling, float64)", "rows": S, "vocab": int(logits.shape[1]),
            "params": SAMPLER_PARAMS, "us_per_call": round(us, 1),
            "bound": "fp64 VALU (exp) of one workgroup per row"}


def prompt_lengths(wl):
    """Prompt length of every sequence of a workload: all equal, or the seeded ragged lengths."""
    from synthetic import make_context_lengths
    if wl.prompt_len is not None:
        return np.full(wl.n_seqs, wl.prompt_len, np.int64)
    return np.asarray(make_context_lengths(wl), np.int64)


def prefill_calls(lens, max_rows=MAX_ROWS):
    """Consecutive sequences grouped into prefill calls of at most max_rows prompt tokens (a
    longer prompt alone in its call): a list of (first, end, rows)."""
    calls, i, S = [], 0, len(lens)
    while i < S:
        j, rows = i, 0
        while j < S and (j == i or rows + int(lens[j]) <= max_rows):
            rows += int(lens[j])
            j += 1
        calls.append((i, j, rows))
        i = j
    return calls


def attention_bytes(lens, t, per_key):
    """Algorithmic bytes of one decode attention launch at decode step t: every visible key and
    value once (the keys before each sequence's position, and the new one)."""
    return int((np.asarray(lens, np.int64) + t + 1).sum()) * per_key


def cpu_baseline(wl, shape, weights, prompts, decode_steps=8):
    """The oracle as it is, on a bounded sample of the workload, timed on this host: one sequence
    (the first; with ragged prompts the shortest) -- its prefill (in the workload's chunks, with
    the workload's logits) and, for decode workloads, a few greedy decode steps."""
    import oracle.model as om
    threads = len(os.sched_getaffinity(0))
    which = int(np.argmin([len(p) for p in prompts])) if wl.prompt_len is None else 0
    plen = len(prompts[which])
    decode_steps = decode_steps if wl.decode_steps else 0
    dec = om.OracleDecoder(weights)
    c = dec.new_cache(capacity=plen + decode_steps)
    t0 = time.perf_counter()
    chunk = wl.chunk or plen
    for c0 in range(0, plen, chunk):
        lg = dec.forward([(prompts[which][c0:c0 + chunk], c)], logits="all" if wl.split else "last")
    t_pre = time.perf_counter() - t0
    tok = int(np.argmax(lg[-1]))
    for _ in range(decode_steps):
        lg = dec.forward([(np.array([tok]), c)], logits="last")
        tok = int(np.argmax(lg[0]))
    dt = time.perf_counter() - t0
    n = plen + decode_steps
    which_s = "" if wl.prompt_len is not None else " (the shortest)"
    what = f"{plen}-token prefill" + (f" in {chunk}-token chunks" if wl.chunk else "") + \
        (" (logits of every row)" if wl.split else "")
    if decode_steps:
        what += f" + {decode_steps} greedy decode steps"
    out = {"value": n / dt, "unit": "tok/s", "cores": threads, "kind": "oracle",
           "sample": f"1 of {wl.n_seqs} sequences{which_s}: {what}, float64 numpy, {dt:.1f} s",
           "prefill_tok_s": plen / t_pre, "host": host_description(threads)}
    if decode_steps:
        out["decode_tok_s"] = decode_steps / (dt - t_pre)
    return out


def host_description(threads):
    """The host the oracle ran on: CPU model, core counts, numpy's BLAS."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    blas = None
    try:
        cfg = np.show_config(mode="dicts")
        dep = cfg.get("Build Dependencies", {}).get("blas", {})
        blas = " ".join(str(dep[k]) for k in ("name", "version") if dep.get(k))
    except Exception:  # (numpy builds differ in what they report)
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity_cores": threads, "blas": blas}


def hardware_line(torch, copy_mib=1024):
    """The device as the runtime reports it, and a measured device-to-device copy beside the
    8 TB/s peak (read + write bytes over the copy's event time; outside the timed region)."""
    import ctypes
    p = torch.cuda.get_device_properties(0)
    clock_khz = ctypes.c_int(0)
    try:  # hipDeviceGetAttribute(hipDeviceAttributeClockRate = 5 in hip_runtime_api.h): peak clock, kHz
        if ctypes.CDLL("libamdhip64.so").hipDeviceGetAttribute(ctypes.byref(clock_khz), 5, 0) != 0:
            clock_khz.value = 0
    except OSError:
        pass
    hw = {"device": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
          "clock_mhz": clock_khz.value / 1000 if clock_khz.value else None,
          "hbm_gib": round(p.total_memory / 2**30, 1)}
    src = torch.empty(copy_mib << 18, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for _ in range(2):
        dst.copy_(src)
    ev[0].record()
    for _ in range(5):
        dst.copy_(src)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / 5
    hw["stream_copy_gbs"] = round(2 * src.numel() * 4 / (ms * 1e-3) / 1e9, 1)
    hw["stream_copy_mib"] = copy_mib
    del src, dst
    return hw


# kernel classes of the library's per-launch timing (dec.h DEC_K_*) timed over a prefill
K_RMSNORM, K_QKV, K_ATTN_PF, K_ROWS, K_COMBINE, K_O, K_GATEUP, K_DOWN, K_LMHEAD = 1, 2, 4, 5, 6, 7, 8, 9, 10
K_WIDEN = 12
PREFILL_CLASSES = {K_QKV: "gemm_qkv", K_ATTN_PF: "attn_prefill", K_ROWS: "attn_rows", K_COMBINE: "attn_combine",
                   K_O: "gemm_o", K_GATEUP: "gemm_gateup", K_DOWN: "gemm_down", K_LMHEAD: "gemm_lmhead",
                   K_RMSNORM: "rmsnorm", K_WIDEN: "widen_q4"}
FP32_MFMA_PEAK_TFS = 157.3  # dense fp32 MFMA: 256 CUs x 256 flop/clk x 2.4 GHz


def prefill_plan(wl, lens):
    """The prefill calls of one bench step: a list of (seqs [(index, start, n)], logits mode).
    Decode workloads: consecutive sequences in calls of at most MAX_ROWS prompt tokens, each
    sequence's last row gets logits. Chunked workloads: one call per chunk of every sequence,
    logits of the last rows in the last call. Cached-split workloads: the full path, logits of
    every row."""
    from decoder_forward_pass_amd import binding as B
    if wl.chunk:
        L = int(lens.max())
        n_chunks = -(-L // wl.chunk)
        return [([(i, c * wl.chunk, min(wl.chunk, int(lens[i]) - c * wl.chunk)) for i in range(len(lens))
                  if c * wl.chunk < lens[i]], B.DEC_LOGITS_LAST if c == n_chunks - 1 else B.DEC_LOGITS_NONE)
                for c in range(n_chunks)]
    if wl.split:
        return [([(i, 0, int(lens[i])) for i in range(len(lens))], B.DEC_LOGITS_ALL)]
    return [([(k, 0, int(lens[k])) for k in range(i, j)], B.DEC_LOGITS_LAST) for i, j, _ in prefill_calls(lens)]


def prefill_flops(shape, plan, B):
    """Algorithmic flops (2 per multiply-add) of the prefill plan, per kernel class and in total.
    Linear layers: every row through every projection; attention: the causal part only (a row
    at position p sees p + 1 keys), 4 H D flops per (row, visible key); LM head: the rows that
    get logits."""
    d, qw, kvw, ff, V, L = shape.d_model, shape.q_width, shape.kv_width, shape.ff_hidden, shape.vocab, shape.n_layers
    per = {K_QKV: 0.0, K_ATTN_PF: 0.0, K_O: 0.0, K_GATEUP: 0.0, K_DOWN: 0.0, K_LMHEAD: 0.0}
    for seqs, mode in plan:
        N = sum(n for _, _, n in seqs)
        keys = sum((st + 1) * n + n * (n - 1) // 2 for _, st, n in seqs)
        per[K_QKV] += 2.0 * N * d * (qw + 2 * kvw) * L
        per[K_O] += 2.0 * N * qw * d * L
        per[K_GATEUP] += 2.0 * N * d * 2 * ff * L
        per[K_DOWN] += 2.0 * N * ff * d * L
        per[K_ATTN_PF] += 4.0 * shape.n_heads * shape.head_dim * keys * L
        n_out = N if mode == B.DEC_LOGITS_ALL else (len(seqs) if mode == B.DEC_LOGITS_LAST else 0)
        per[K_LMHEAD] += 2.0 * n_out * d * V
    return per, sum(per.values())


def decode_step_bytes(shape, lens, t, weight_bytes):
    """Algorithmic HBM bytes of decode step t: every weight byte once, every visible key and value
    once (the new ones counted as written), the float32 logits written."""
    kv_el = 2 if shape.kv_dtype == "f16" else 4
    per_key = shape.n_kv_heads * shape.head_dim * 2 * kv_el
    return weight_bytes + attention_bytes(lens, t, per_key) * shape.n_layers + len(lens) * shape.vocab * 4


def compute_dtype(shape):
    """The arithmetic type of the products: float32 MFMA for float32 weights, bf16 MFMA otherwise
    (4-bit weights are dequantised to bf16 operands)."""
    return "f32" if shape.weight_dtype == "f32" else "bf16"


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.workload, args.copy_mb or 512)
        return
    if args.summarize_stats:
        summarize_stats(args.summarize_stats, args.workload, args.steps)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma, args.workload)
        return
    if args.summarize_line:
        summarize_line(args.summarize_line, args.workload, args.steps, args.warmup)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (sharding the batch by "
              "sequence would run these kernels unchanged on each GPU's share; it is not implemented).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from decoder_forward_pass_amd import binding as B
    from decoder_forward_pass_amd.session import BlockAllocator, Session
    from synthetic import MODELS, WORKLOADS, make_prompts, make_weights

    wl = WORKLOADS[args.workload]
    shape = MODELS[wl.model]
    weights = make_weights(shape)
    prompts = make_prompts(wl)
    S = wl.n_seqs
    steps = 0 if args.prefill_only else wl.decode_steps
    lens = prompt_lengths(wl)
    ctx = int(lens.max()) + max(steps, 1)
    n_blocks = sum(math.ceil((int(n) + max(steps, 1)) / shape.block_tokens) for n in lens)
    plan = prefill_plan(wl, lens)
    max_rows = max(sum(n for _, _, n in seqs) for seqs, _ in plan)
    s = Session(shape, weights, max_context=ctx, n_blocks=n_blocks, max_rows=max_rows, max_seqs=S)
    alloc = BlockAllocator(n_blocks, shape.block_tokens, seed=1)
    for i in range(S):
        alloc.ensure(i, int(lens[i]) + max(steps, 1))
    tbl = alloc.table_array(list(range(S)))
    call_args = []
    for seqs, mode in plan:
        idx = [i for i, _, _ in seqs]
        toks = np.concatenate([prompts[i][st:st + n] for i, st, n in seqs])
        n_out = sum(n for _, _, n in seqs) if mode == B.DEC_LOGITS_ALL else (len(seqs) if mode == B.DEC_LOGITS_LAST
                                                                             else 0)
        out = torch.empty((n_out, shape.vocab), dtype=torch.float32, device="cuda") if n_out else None
        call_args.append(([st for _, st, _ in seqs], [n for _, _, n in seqs], toks, alloc.table_array(idx), mode,
                          out, idx))
    hist = torch.zeros((steps + 1, S), dtype=torch.int32, device="cuda")
    logits = torch.empty((S, shape.vocab), dtype=torch.float32, device="cuda")
    positions = [(lens + t).astype(np.int32) for t in range(steps)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    if args.copy_mb:
        src = torch.empty(args.copy_mb << 18, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    TIME_EVERY = args.time_every
    decode_mask = (1 << K_ROWS) | (1 << K_COMBINE)

    def prefill_calls_once():
        for st, nn, toks, ctbl, mode, out, idx in call_args:
            # (decode workloads: a call's sequences are consecutive, so their next ids are a view)
            nxt = hist[0, idx[0]:idx[-1] + 1] if mode == B.DEC_LOGITS_LAST and steps else None
            s.prefill(st, nn, toks, ctbl, mode, logits=out, next_tokens=nxt)

    def one_step(timed, prefill_mask=0):
        # in the timed steps the launches of one prefill kernel class (the dominant one) are timed,
        # with events the launch records at the kernel's own start and end, and of the decode steps
        # the attention launches of every TIME_EVERY-th step (a timed launch costs a little)
        if timed:
            ev[0].record()
            B.dec_timing_enable(s.ctx, prefill_mask)
        prefill_calls_once()
        if timed:
            ev[1].record()
            B.dec_timing_enable(s.ctx, 0)
        for t in range(steps):
            on = timed and TIME_EVERY and t % TIME_EVERY == 0
            if on:
                B.dec_timing_enable(s.ctx, decode_mask)
            s.decode_step(positions[t], tbl, tokens_device=hist[t], logits=logits, next_tokens=hist[t + 1])
            if on:
                B.dec_timing_enable(s.ctx, 0)
        if timed:
            ev[2].record()

    for _ in range(args.warmup):
        one_step(False)
    # per-class breakdown of the prefill, untimed for the value: one more pass of the prefill calls
    # with every launch of every class timed; its largest product class is then timed live
    torch.cuda.synchronize()
    B.dec_timing_enable(s.ctx, sum(1 << k for k in PREFILL_CLASSES))
    prefill_calls_once()
    B.dec_timing_enable(s.ctx, 0)
    breakdown = {k: B.dec_timing_read(s.ctx, k) for k in PREFILL_CLASSES}
    top_class = max((k for k in (K_QKV, K_ATTN_PF, K_O, K_GATEUP, K_DOWN, K_LMHEAD) if breakdown[k][1]),
                    key=lambda k: breakdown[k][0])
    torch.cuda.synchronize()

    pre, dec = [], []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_step(True, 1 << top_class)
        pre.append((ev[0], ev[1]))
        dec.append((ev[1], ev[2]))
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    phases = [(a.elapsed_time(b), c.elapsed_time(d)) for (a, b), (c, d) in zip(pre, dec)]
    timing = {k: B.dec_timing_read(s.ctx, k) for k in PREFILL_CLASSES}  # the timed steps' launches
    weight_bytes = B.dec_weight_bytes(s.cfg)
    sampler = None if (args.no_sampler or not steps) else time_sampler(s, logits, prompts)
    s.close()

    prompt_tokens = int(lens.sum())
    tok_per_step = prompt_tokens + S * steps
    value = tok_per_step * args.steps / elapsed
    pre_ms = float(np.mean([p[0] for p in phases]))
    dec_ms = float(np.mean([p[1] for p in phases]))
    mfma_peak = FP32_MFMA_PEAK_TFS if shape.weight_dtype == "f32" else MFMA_BF16_PEAK_TFS

    # prefill: algorithmic flops per kernel class against the launches of that class, from the
    # breakdown pass (one pass of the prefill calls)
    per_class, pre_flops = prefill_flops(shape, plan, B)
    kernels = {}
    for k, name in PREFILL_CLASSES.items():
        ms, n = breakdown[k]
        if not n:
            continue
        row = {"launches": n, "avg_launch_us": round(ms / n * 1e3, 2), "share_of_prefill": round(ms / pre_ms, 4)}
        if per_class.get(k):
            tfs = per_class[k] / n / (ms / n * 1e-3) / 1e12
            row.update(algorithmic_flops_per_launch=per_class[k] / n, achieved_tflops=round(tfs, 1),
                       frac=round(tfs / mfma_peak, 4))
        kernels[name] = row
    # the dominant class, timed live over the timed steps
    top_ms, top_n = timing[top_class]
    top_flops = per_class[top_class] / max(breakdown[top_class][1], 1)
    top_tfs = top_flops / (top_ms / max(top_n, 1) * 1e-3) / 1e12
    pre_tfs = pre_flops / (pre_ms * 1e-3) / 1e12
    roofline_prefill = {"kernel": PREFILL_CLASSES[top_class], "bound": "mfma", "achieved": round(top_tfs, 1),
                        "peak": mfma_peak, "unit": "TFLOP/s", "frac": round(top_tfs / mfma_peak, 4),
                        "launches": top_n, "avg_launch_us": round(top_ms / max(top_n, 1) * 1e3, 2),
                        "algorithmic_flops_per_launch": top_flops}

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": compute_dtype(shape),
        "data": "synthetic",
        "config": {"workload": wl.name, "model": "Qwen3-0.6B shape, random init" if shape.d_model == 1024 else shape.name,
                   "global_batch": S,
                   "prompt_len": wl.prompt_len if wl.prompt_len is not None else f"U[{wl.ctx_lo}, {wl.ctx_hi}]",
                   "prefill_chunk": wl.chunk, "logits": "every row" if wl.split else "last row",
                   "decode_steps": steps, "weights": shape.weight_dtype,
                   "kv_cache": shape.kv_dtype, "parallelism": "none (1 GPU)"},
        "prefill_tok_s": round(prompt_tokens / (pre_ms * 1e-3), 1),
        "prefill_ms": round(pre_ms, 3),
        "prefill_phase": {"bound": "mfma", "algorithmic_tflop": round(pre_flops / 1e12, 4),
                          "achieved": round(pre_tfs, 1), "peak": mfma_peak, "unit": "TFLOP/s",
                          "frac": round(pre_tfs / mfma_peak, 4)},
        "prefill_kernels": kernels,
    }
    if steps:
        rows_ms, rows_n = timing[K_ROWS]
        comb_ms, comb_n = timing[K_COMBINE]
        kv_el = 2 if shape.kv_dtype == "f16" else 4
        per_key = shape.n_kv_heads * shape.head_dim * 2 * kv_el
        timed_steps = list(range(0, steps, TIME_EVERY or steps))
        rows_launch_bytes = float(np.mean([attention_bytes(lens, t, per_key) for t in timed_steps]))
        rows_launches_expected = args.steps * len(timed_steps) * shape.n_layers if TIME_EVERY else 0
        # a split row's segments are merged by the combine kernel: its time counts with the attention's
        rows_avg_ms = (rows_ms + comb_ms) / max(rows_n, 1)
        achieved = rows_launch_bytes / (rows_avg_ms * 1e-3) / 1e9 if rows_n else None
        step_bytes = float(np.mean([decode_step_bytes(shape, lens, t, weight_bytes) for t in range(steps)]))
        dec_step_ms = dec_ms / steps
        dec_gbs = step_bytes / (dec_step_ms * 1e-3) / 1e9
        result.update({
            "decode_tok_s": round(S * steps / (dec_ms * 1e-3), 1),
            "decode_ms_per_step": round(dec_step_ms, 4),
            "decode_phase": {"bound": "hbm", "algorithmic_bytes_per_step": step_bytes, "achieved": round(dec_gbs, 1),
                             "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4)},
            "roofline": {
                "kernel": "attn_decode_kernel (decode attention, q/k norm + RoPE + KV write fused)"
                          + (" + attn_decode_combine_kernel" if comb_n else ""),
                "bound": "hbm", "achieved": round(achieved, 1) if achieved else None, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4) if achieved else None,
                "traffic": measured_traffic(f"attn_decode_kernel_{wl.name}_pmc.json"),
                "launches": rows_n, "launches_expected": rows_launches_expected, "combine_launches": comb_n,
                "avg_launch_us": round(rows_avg_ms * 1e3, 2), "algorithmic_bytes_per_launch": rows_launch_bytes,
            },
            "roofline_prefill": roofline_prefill,
        })
    else:
        # prefill-only workload: its dominant kernel is the roofline
        result["roofline"] = dict(roofline_prefill, traffic=None)
    if sampler:
        result["sampler"] = sampler
    if not args.copy_mb:
        # (not in the counter runs: their reference copy must stay the largest copy dispatch)
        result["hardware"] = hardware_line(torch)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, shape, weights, prompts)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
