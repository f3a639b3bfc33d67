"""Chunked prefill on the cache at full size: the 0.6B shape, bf16 weights, f16 KV cache,
8 prompts of 2,048 seeded tokens run as four calls of 8 x 512 tokens at start = 512c, against
one 8 x 2,048 call ("Candle model runner" 2.4, chunk invariance; "Proving it's the same model",
the cached path must match).

The chunked logits are compared with the single-shot logits at every position (the
library's key tiles are aligned to absolute positions, so they are expected to agree bit for
bit; identical rows are counted and the max difference must stay within the gate), and both
are compared with the float64 oracle on one sequence: the last row of every chunk plus a
seeded sample of 1/16 of the positions. Gate: 2e-2 of each row's oracle logit range.

A third copy prefills the first 600 tokens of every prompt in one call (4,800 rows: not a
multiple of the 128- or 256-row product tiles, and small enough that the output and down
projections take the 128 x 128 tiles); its logits must equal the single-shot ones bit for bit.
"""

import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from gpu_util import compare, report
import oracle.model as om
from synthetic import MODELS, WORKLOADS, make_prompts, make_weights

REL = 2e-2
ORACLE_SEQ = 3
RAGGED = 600  # prompt tokens per sequence of the one-call ragged copy


@pytest.fixture(scope="module")
def run():
    from decoder_forward_pass_amd import binding as B
    from decoder_forward_pass_amd.session import BlockAllocator, Session
    wl = WORKLOADS["q06b_bf16_b8_p2048_c512"]
    shape = MODELS[wl.model]
    w = make_weights(shape)
    prompts = make_prompts(wl)
    S, P, C = wl.n_seqs, wl.prompt_len, wl.chunk
    per_seq = math.ceil(P / shape.block_tokens)
    n_blocks = 3 * S * per_seq
    s = Session(shape, w, max_context=P, n_blocks=n_blocks, max_rows=S * P, max_seqs=S)
    alloc = BlockAllocator(n_blocks, shape.block_tokens, seed=4)
    one = [("one", i) for i in range(S)]
    chk = [("chunk", i) for i in range(S)]
    rag = [("ragged", i) for i in range(S)]
    for a in one + chk + rag:
        alloc.ensure(a, P)
    print(f"[c4] single shot {S}x{P}", flush=True)
    full = s.prefill([0] * S, [P] * S, np.concatenate(prompts), alloc.table_array(one), B.DEC_LOGITS_ALL)
    rng = np.random.default_rng(wl.seed)
    sample = np.sort(np.unique(np.concatenate([np.arange(C - 1, P, C), rng.choice(P, P // 16, replace=False)])))
    identical, worst = 0, 0.0
    chunk_rows = {}
    tbl = alloc.table_array(chk)
    for c0 in range(0, P, C):
        print(f"[c4] chunk at {c0}", flush=True)
        part = s.prefill([c0] * S, [C] * S, np.concatenate([p[c0:c0 + C] for p in prompts]), tbl, B.DEC_LOGITS_ALL)
        ref = full.view(S, P, -1)[:, c0:c0 + C].reshape(S * C, -1)
        identical += int(torch.sum(torch.all(part == ref, dim=1)))
        worst = max(worst, float((part - ref).abs().max()))
        mine = part.view(S, C, -1)[ORACLE_SEQ]
        for p in sample[(sample >= c0) & (sample < c0 + C)]:
            chunk_rows[int(p)] = mine[p - c0].cpu().numpy()
        del part, ref
    print(f"[c4] {S}x{RAGGED} rows in one call", flush=True)
    part = s.prefill([0] * S, [RAGGED] * S, np.concatenate([p[:RAGGED] for p in prompts]), alloc.table_array(rag),
                     B.DEC_LOGITS_ALL)
    ref = full.view(S, P, -1)[:, :RAGGED].reshape(S * RAGGED, -1)
    ragged_identical = int(torch.sum(torch.all(part == ref, dim=1)))
    del part, ref
    full_rows = full.view(S, P, -1)[ORACLE_SEQ][torch.from_numpy(sample).cuda()].cpu().numpy()
    torch.cuda.synchronize()
    del full
    s.close()
    yield (wl, shape, w, prompts, sample, full_rows, np.array([chunk_rows[int(p)] for p in sample]), identical, worst,
           ragged_identical)


def test_chunked_equals_single_shot(run):
    wl, shape, w, prompts, sample, full_rows, chunk_rows, identical, worst, _ = run
    total = wl.n_seqs * wl.prompt_len
    report({"type": "chunk_invariance", "case": wl.name, "identical_rows": identical, "rows": total,
            "max_absolute_error": worst})
    assert identical == total


def test_ragged_row_count_equals_single_shot(run):
    wl, *_, ragged_identical = run
    report({"type": "batch_invariance", "case": f"{wl.name}_first{RAGGED}", "identical_rows": ragged_identical,
            "rows": wl.n_seqs * RAGGED})
    assert ragged_identical == wl.n_seqs * RAGGED


def test_chunked_and_single_shot_match_oracle(run):
    wl, shape, w, prompts, sample, full_rows, chunk_rows, identical, worst, _ = run
    dec = om.OracleDecoder(w)
    print("[c4] oracle", flush=True)
    ref = dec.forward([(prompts[ORACLE_SEQ], dec.new_cache(wl.prompt_len))], rows=sample)
    for path, got in (("single_shot", full_rows), ("chunked", chunk_rows)):
        row = compare(got, ref, rel_range=REL)
        row.update(type="logit_parity", case=wl.name, path=path, seq=ORACLE_SEQ, sampled_positions=len(sample))
        report(row)
        assert row["pass"], row
