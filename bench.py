"""Prefill and decode throughput of the decoder forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Workload (default): the Qwen3-0.6B shape with bf16 weights and an f16 KV cache, random
seeded weights and token ids; one step = one dec_prefill of 32 sequences x 1,024 prompt
tokens (last-token logits and greedy next ids) followed by 256 greedy dec_decode_step calls
at batch 32 (next ids passed on the device). W untimed steps, then exactly K timed steps
between two device synchronisations. ``value`` is whole-job tokens/s (prompt + generated
tokens per second); prefill and decode rates are reported beside it.

``roofline``: the kernel with the largest share of the timed region's GPU time (decode
attention, HBM-bound), timed live with HIP events around its launches on the library's
stream; achieved = its algorithmic bytes per launch / its mean launch duration.
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="q06b_bf16_b32_p1024_d256")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="first run one device-to-device copy of this many MiB (a reference dispatch of known "
                         "traffic for hardware-counter runs)")
    return ap.parse_args()


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


def cpu_baseline(wl, shape, weights, prompts, decode_steps=8):
    """The oracle as it is, on one sequence: its prefill, then a few greedy decode steps."""
    import oracle.model as om
    threads = len(os.sched_getaffinity(0))
    dec = om.OracleDecoder(weights)
    c = dec.new_cache(capacity=wl.prompt_len + decode_steps)
    t0 = time.perf_counter()
    lg = dec.forward([(prompts[0], c)], logits="last")
    tok = int(np.argmax(lg[0]))
    for _ in range(decode_steps):
        lg = dec.forward([(np.array([tok]), c)], logits="last")
        tok = int(np.argmax(lg[0]))
    dt = time.perf_counter() - t0
    n = wl.prompt_len + decode_steps
    return {"value": n / dt, "unit": "tok/s", "cores": threads, "kind": "oracle",
            "sample": f"1 of {wl.n_seqs} sequences: {wl.prompt_len}-token prefill + {decode_steps} greedy decode "
                      f"steps, float64 numpy, {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(data-parallel sharding by sequence is described in DESIGN.md but not built).", file=sys.stderr)
        sys.exit(2)

    import torch
    from decoder_forward_pass_amd import binding as B
    from decoder_forward_pass_amd.session import BlockAllocator, Session
    from synthetic import MODELS, WORKLOADS, make_prompts, make_weights

    wl = WORKLOADS[args.workload]
    if wl.prompt_len is None or wl.decode_steps == 0:
        sys.exit(f"workload {wl.name} is a parity case, not a bench workload")
    shape = MODELS[wl.model]
    weights = make_weights(shape)
    prompts = make_prompts(wl)
    S, P, steps = wl.n_seqs, wl.prompt_len, wl.decode_steps
    ctx = P + steps
    n_blocks = S * math.ceil(ctx / shape.block_tokens)
    s = Session(shape, weights, max_context=ctx, n_blocks=n_blocks, max_rows=S * P, max_seqs=S)
    alloc = BlockAllocator(n_blocks, shape.block_tokens, seed=1)
    for i in range(S):
        alloc.ensure(i, ctx)
    tbl = alloc.table_array(list(range(S)))
    tokens = np.concatenate(prompts)
    hist = torch.zeros((steps + 1, S), dtype=torch.int32, device="cuda")
    last = torch.empty((S, shape.vocab), dtype=torch.float32, device="cuda")
    logits = torch.empty((S, shape.vocab), dtype=torch.float32, device="cuda")
    positions = [np.full(S, P + t, np.int32) for t in range(steps)]
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

    def one_step(phase_times=None):
        timed = phase_times is not None
        if timed:
            ev[0].record()
            B.dec_timing_enable(s.ctx, 1 << K_GATEUP)
        s.prefill([0] * S, [P] * S, tokens, tbl, B.DEC_LOGITS_LAST, logits=last, next_tokens=hist[0])
        if timed:
            ev[1].record()
            B.dec_timing_enable(s.ctx, 1 << K_ROWS)
        for t in range(steps):
            s.decode_step(positions[t], tbl, tokens_device=hist[t], logits=logits, next_tokens=hist[t + 1])
        if timed:
            B.dec_timing_enable(s.ctx, 0)
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
    s.close()

    tok_per_step = S * P + S * steps
    value = tok_per_step * args.steps / elapsed
    pre_ms = float(np.mean([p[0] for p in phases]))
    dec_ms = float(np.mean([p[1] for p in phases]))

    # decode attention: algorithmic bytes = every visible key and value once (f16), plus q and
    # the output partial sums are negligible; per layer and step: sum over sequences of
    # (context length) x H_kv x D x 2 (K, V) x 2 bytes.
    kv_el = 2 if shape.kv_dtype == "f16" else 4
    per_key = shape.n_kv_heads * shape.head_dim * 2 * kv_el
    bytes_per_step_layer = [S * (P + t + 1) * per_key for t in range(steps)]
    rows_launch_bytes = float(np.mean(bytes_per_step_layer))
    rows_launches_expected = args.steps * steps * shape.n_layers
    rows_avg_ms = rows_ms / max(rows_n, 1)
    achieved = rows_launch_bytes / (rows_avg_ms * 1e-3) / 1e9
    # gate/up GEMM of the prefill: 2 * M * (2 ff) * d flops per launch
    gu_prefill_flops = 2.0 * S * P * 2 * shape.ff_hidden * shape.d_model
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
                   "prompt_len": P, "decode_steps": steps, "weights": shape.weight_dtype,
                   "kv_cache": shape.kv_dtype, "parallelism": "none (1 GPU)"},
        "prefill_tok_s": round(S * P / (pre_ms * 1e-3), 1),
        "decode_tok_s": round(S * steps / (dec_ms * 1e-3), 1),
        "prefill_ms": round(pre_ms, 3),
        "decode_ms_per_step": round(dec_ms / steps, 4),
        "roofline": {
            "kernel": "attn_decode_kernel (decode attention, q/k norm + RoPE + KV write fused)",
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
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
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, shape, weights, prompts)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
