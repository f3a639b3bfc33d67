"""Host-side arithmetic of bench.py (no GPU): the grouping of prompts into prefill calls and the
decode attention's algorithmic bytes, including the ragged-context workloads."""

import numpy as np

import bench
from synthetic import MODELS, WORKLOADS


def test_prefill_calls_cover_every_sequence_once_within_the_row_cap():
    rng = np.random.default_rng(3)
    for cap in (1, 100, 1000, 32768):
        lens = rng.integers(1, 400, 57)
        calls = bench.prefill_calls(lens, cap)
        assert calls[0][0] == 0 and calls[-1][1] == len(lens)
        for (i, j, rows), nxt in zip(calls, calls[1:] + [None]):
            assert j > i and rows == int(lens[i:j].sum())
            assert rows <= cap or j == i + 1  # a longer prompt goes alone
            if nxt is not None:
                assert nxt[0] == j and rows + int(lens[j]) > cap  # greedy: the next one did not fit


def test_headline_workload_is_one_prefill_call():
    wl = WORKLOADS["q06b_bf16_b32_p1024_d256"]
    assert bench.prefill_calls(bench.prompt_lengths(wl)) == [(0, 32, 32768)]


def test_ragged_workload_lengths_and_calls():
    wl = WORKLOADS["q06b_uint4_b64_ragged_d128"]
    lens = bench.prompt_lengths(wl)
    assert len(lens) == 64 and lens.min() >= 512 and lens.max() <= 8192
    calls = bench.prefill_calls(lens)
    assert sum(r for _, _, r in calls) == int(lens.sum())
    assert all(r <= bench.MAX_ROWS for _, _, r in calls)


def test_attention_bytes_count_every_visible_key_once():
    m = MODELS["q06b_bf16"]
    per_key = m.n_kv_heads * m.head_dim * 2 * 2  # K and V, f16
    assert per_key == 4096
    # 32 sequences of 1,024 prompt tokens at decode step 0: 1,025 visible keys each
    assert bench.attention_bytes(np.full(32, 1024), 0, per_key) == 32 * 1025 * 4096
    # ragged: the sum of each sequence's own context
    assert bench.attention_bytes([10, 20], 5, 2) == (16 + 26) * 2


def test_chunked_plan_and_flops_of_the_chunked_workload():
    from decoder_forward_pass_amd import binding as B
    wl = WORKLOADS["q06b_bf16_b8_p2048_c512"]
    plan = bench.prefill_plan(wl, bench.prompt_lengths(wl))
    assert len(plan) == 4
    for c, (seqs, mode) in enumerate(plan):
        assert [(i, st, n) for i, st, n in seqs] == [(i, 512 * c, 512) for i in range(8)]
        assert mode == (B.DEC_LOGITS_LAST if c == 3 else B.DEC_LOGITS_NONE)
    per, total = bench.prefill_flops(MODELS[wl.model], plan, B)
    # 14.43 TFLOP of projections + 3.85 of causal attention (+ 8 rows of LM head)
    assert abs(total / 1e12 - 18.28) < 0.01
    assert abs(per[bench.K_ATTN_PF] / 1e12 - 3.85) < 0.01


def test_flops_of_the_headline_prefill_and_the_fp32_full_path():
    from decoder_forward_pass_amd import binding as B
    wl = WORKLOADS["q06b_bf16_b32_p1024_d256"]
    _, total = bench.prefill_flops(MODELS[wl.model], bench.prefill_plan(wl, bench.prompt_lengths(wl)), B)
    assert abs(total / 1e12 - 32.72) < 0.01
    wl = WORKLOADS["q06b_f32_t188"]
    plan = bench.prefill_plan(wl, bench.prompt_lengths(wl))
    assert plan[0][1] == B.DEC_LOGITS_ALL
    per, total = bench.prefill_flops(MODELS[wl.model], plan, B)
    assert abs(total / 1e9 - 228.2) < 0.3  # every row's logits: 58.5 GFLOP of LM head
    assert abs(per[bench.K_LMHEAD] / 1e9 - 58.5) < 0.1


def test_decode_step_bytes_of_the_headline_workload():
    from decoder_forward_pass_amd.session import make_config
    from decoder_forward_pass_amd import binding as B
    wl = WORKLOADS["q06b_bf16_b32_p1024_d256"]
    m = MODELS[wl.model]
    wb = B.dec_weight_bytes(make_config(m, max_context=2048, n_blocks=1, max_rows=1, max_seqs=1))
    assert abs(wb / 1e9 - 1.192) < 0.001
    lens = bench.prompt_lengths(wl)
    mean = np.mean([bench.decode_step_bytes(m, lens, t, wb) for t in range(wl.decode_steps)])
    assert abs(mean / 1e9 - 5.445) < 0.005
    assert bench.compute_dtype(m) == "bf16" and bench.compute_dtype(MODELS["q06b_f32"]) == "f32"
