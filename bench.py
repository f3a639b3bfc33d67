"""Prefill and decode throughput of the decoder forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Workload (default): the Qwen3-0.6B shape with bf16 weights and an f16 KV cache, random
seeded weights and token ids; one step = one dec_prefill of 32 sequences x 1,024 prompt
tokens (last-token logits and greedy next ids) followed by 256 greedy dec_decode_step calls
at batch 32 (next ids passed on the device). W untimed steps, then exactly K timed steps
between two device synchronisations. ``value`` is whole-job tokens/s (prompt + generated
tokens per second); prefill and decode rates are reported beside it.

``roofline``: the kernel with the largest share of the timed region's GPU time (decode
attention, HBM-bound), timed live on the library's stream with HIP events that the launch
itself records at the kernel's start and end, on the attention launches of every 32nd decode
step of the timed steps; achieved = their mean algorithmic bytes per launch / their mean
duration. ``traffic``: HBM bytes per launch from the committed hardware-counter summary.
``roofline_prefill``: the same for the largest prefill GEMM (MFMA-bound). ``cpu_baseline``:
the float64 CPU oracle on a bounded sample of the same workload (one sequence's prefill and
a few decode steps), timed on this host.
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
             f"{steps} step(s), no warm-up: one prefill of the batch plus its decode steps.", "",
             "| kernel | calls | total ms | mean us | share |", "|---|---:|---:|---:|---:|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        t = float(r["TotalDurationNs"])
        lines.append(f"| `{r['Name'].split('(')[0]}` | {r['Calls']} | {t / 1e6:.2f} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{100 * t / total:.1f}% |")
    path = os.path.join(ROOT, "profiles", f"bench_{wl_name}_kernel_stats.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {path}")


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
    """The oracle as it is, on one sequence (the first; with ragged prompts the shortest): its
    prefill, then a few greedy decode steps."""
    import oracle.model as om
    threads = len(os.sched_getaffinity(0))
    which = int(np.argmin([len(p) for p in prompts])) if wl.prompt_len is None else 0
    plen = len(prompts[which])
    dec = om.OracleDecoder(weights)
    c = dec.new_cache(capacity=plen + decode_steps)
    t0 = time.perf_counter()
    lg = dec.forward([(prompts[which], c)], logits="last")
    tok = int(np.argmax(lg[0]))
    for _ in range(decode_steps):
        lg = dec.forward([(np.array([tok]), c)], logits="last")
        tok = int(np.argmax(lg[0]))
    dt = time.perf_counter() - t0
    n = plen + decode_steps
    which_s = "" if wl.prompt_len is not None else " (the shortest)"
    return {"value": n / dt, "unit": "tok/s", "cores": threads, "kind": "oracle",
            "sample": f"1 of {wl.n_seqs} sequences{which_s}: {plen}-token prefill + {decode_steps} greedy decode "
                      f"steps, float64 numpy, {dt:.1f} s"}


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.workload, args.copy_mb or 512)
        return
    if args.summarize_stats:
        summarize_stats(args.summarize_stats, args.workload, args.steps)
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
    if wl.decode_steps == 0:
        sys.exit(f"workload {wl.name} is a parity case, not a bench workload")
    shape = MODELS[wl.model]
    weights = make_weights(shape)
    prompts = make_prompts(wl)
    S, steps = wl.n_seqs, wl.decode_steps
    lens = prompt_lengths(wl)
    ctx = int(lens.max()) + steps
    n_blocks = sum(math.ceil((int(n) + steps) / shape.block_tokens) for n in lens)
    # prefill calls of consecutive sequences, each at most MAX_ROWS prompt tokens (one call for
    # 32 x 1,024)
    calls = prefill_calls(lens)
    s = Session(shape, weights, max_context=ctx, n_blocks=n_blocks, max_rows=max(c[2] for c in calls), max_seqs=S)
    alloc = BlockAllocator(n_blocks, shape.block_tokens, seed=1)
    for i in range(S):
        alloc.ensure(i, int(lens[i]) + steps)
    tbl = alloc.table_array(list(range(S)))
    call_args = [(np.concatenate(prompts[i:j]), alloc.table_array(list(range(i, j)))) for i, j, _ in calls]
    hist = torch.zeros((steps + 1, S), dtype=torch.int32, device="cuda")
    last = torch.empty((S, shape.vocab), dtype=torch.float32, device="cuda")
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

    # kernel classes timed live over the timed region: the prefill's gate/up GEMM and the
    # decode steps' attention
    K_ROWS, K_GATEUP = 5, 8
    TIME_EVERY = args.time_every

    def one_step(phase_times=None):
        timed = phase_times is not None
        if timed:
            ev[0].record()
            B.dec_timing_enable(s.ctx, 1 << K_GATEUP)
        for (i, j, _), (toks, ctbl) in zip(calls, call_args):
            s.prefill([0] * (j - i), lens[i:j], toks, ctbl, B.DEC_LOGITS_LAST, logits=last[i:j],
                      next_tokens=hist[0, i:j])
        if timed:
            ev[1].record()
            B.dec_timing_enable(s.ctx, 0)
        for t in range(steps):
            # the attention launches of every TIME_EVERY-th decode step are timed (a timed launch
            # records its events at the kernel's own start and end, which costs a little)
            if timed and TIME_EVERY and t % TIME_EVERY == 0:
                B.dec_timing_enable(s.ctx, 1 << K_ROWS)
            s.decode_step(positions[t], tbl, tokens_device=hist[t], logits=logits, next_tokens=hist[t + 1])
            if timed and TIME_EVERY and t % TIME_EVERY == 0:
                B.dec_timing_enable(s.ctx, 0)
        if timed:
            ev[2].record()
            phase_times.append(None)

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()

    phases = []
    pre, dec = [], []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_step(phases)
        # the phase events of this step are read after the next step is queued
        pre.append((ev[0], ev[1]))
        dec.append((ev[1], ev[2]))
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    phases = [(a.elapsed_time(b), c.elapsed_time(d)) for (a, b), (c, d) in zip(pre, dec)]
    rows_ms, rows_n = B.dec_timing_read(s.ctx, K_ROWS)
    gu_ms, gu_n = B.dec_timing_read(s.ctx, K_GATEUP)
    sampler = None if args.no_sampler else time_sampler(s, logits, prompts)
    s.close()

    tok_per_step = int(lens.sum()) + S * steps
    value = tok_per_step * args.steps / elapsed
    pre_ms = float(np.mean([p[0] for p in phases]))
    dec_ms = float(np.mean([p[1] for p in phases]))

    # decode attention: algorithmic bytes = every visible key and value once (f16), plus q and
    # the output partial sums are negligible; per layer and step: sum over sequences of
    # (context length) x H_kv x D x 2 (K, V) x 2 bytes.
    kv_el = 2 if shape.kv_dtype == "f16" else 4
    per_key = shape.n_kv_heads * shape.head_dim * 2 * kv_el
    bytes_per_step_layer = [attention_bytes(lens, t, per_key) for t in range(0, steps, TIME_EVERY or steps)]
    rows_launch_bytes = float(np.mean(bytes_per_step_layer))
    rows_launches_expected = args.steps * len(bytes_per_step_layer) * shape.n_layers if TIME_EVERY else 0
    rows_avg_ms = rows_ms / max(rows_n, 1)
    # (--time-every 0 times no launch: the roofline figures are then absent)
    achieved = rows_launch_bytes / (rows_avg_ms * 1e-3) / 1e9 if rows_n else None
    # gate/up GEMM of the prefill: 2 * M * (2 ff) * d flops per launch (M = the call's rows;
    # every call has the same number of launches, all timed)
    gu_prefill_flops = float(np.mean([2.0 * rows * 2 * shape.ff_hidden * shape.d_model for _, _, rows in calls]))
    # (only prefill launches of that class are timed)

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
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "model": "Qwen3-0.6B shape, random init", "global_batch": S,
                   "prompt_len": wl.prompt_len if wl.prompt_len is not None else f"U[{wl.ctx_lo}, {wl.ctx_hi}]",
                   "decode_steps": steps, "weights": shape.weight_dtype,
                   "kv_cache": shape.kv_dtype, "parallelism": "none (1 GPU)"},
        "prefill_tok_s": round(int(lens.sum()) / (pre_ms * 1e-3), 1),
        "decode_tok_s": round(S * steps / (dec_ms * 1e-3), 1),
        "prefill_ms": round(pre_ms, 3),
        "decode_ms_per_step": round(dec_ms / steps, 4),
        "roofline": {
            "kernel": "attn_decode_kernel (decode attention, q/k norm + RoPE + KV write fused)",
            "bound": "hbm", "achieved": round(achieved, 1) if achieved else None, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4) if achieved else None,
            "traffic": measured_traffic(f"attn_decode_kernel_{wl.name}_pmc.json"),
            "launches": rows_n, "launches_expected": rows_launches_expected,
            "avg_launch_us": round(rows_avg_ms * 1e3, 2), "algorithmic_bytes_per_launch": rows_launch_bytes,
        },
    }
    gu_avg_ms = gu_ms / max(gu_n, 1)
    gu_tfs = gu_prefill_flops / (gu_avg_ms * 1e-3) / 1e12
    result["roofline_prefill"] = {
        "kernel": "gemm_gateup (prefill, SwiGLU epilogue)", "bound": "mfma",
        "achieved": round(gu_tfs, 2), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
        "frac": round(gu_tfs / MFMA_BF16_PEAK_TFS, 4), "launches": gu_n,
        "avg_launch_us": round(gu_avg_ms * 1e3, 2), "algorithmic_flops_per_launch": gu_prefill_flops,
    }
    if sampler:
        result["sampler"] = sampler
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, shape, weights, prompts)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
