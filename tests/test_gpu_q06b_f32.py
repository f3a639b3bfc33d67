"""GPU parity on the Qwen3-0.6B-shaped decoder in float32: 188 prompt tokens, full path and
cached path split at 94, every logit at every position against the float64 oracle, max-abs
<= 1e-3 ("Proving it's the same model": the procedure of ``logits_parity`` and the tolerance
fixed before the first run).

Batch invariance across the float32 paths: the 188-token prompt run alone and inside one call
with a 2,100-token prompt must give bit-identical logits. Alone, every product's grid is small,
so K is split into parts (16 for O and down, 8 for the others) over blocks and a second kernel adds them, and the attention merges
each row's key chunks inside one workgroup. In the 2,288-row call every product adds the parts
inside one block, and the attention (a row of 66 chunks, beyond what the workgroup merge holds)
writes chunk partials that a second kernel merges."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from gpu_util import compare, report
import oracle.model as om
from synthetic import MODELS, WORKLOADS, make_prompts, make_weights

TOL = 1e-3


@pytest.fixture(scope="module")
def case():
    from decoder_forward_pass_amd.session import BlockAllocator, Session
    wl = WORKLOADS["q06b_f32_t188"]
    shape = MODELS[wl.model]
    w = make_weights(shape)
    prompt = make_prompts(wl)[0]
    s = Session(shape, w, max_context=256, n_blocks=64, max_rows=188, max_seqs=2)
    yield wl, shape, w, prompt, s, BlockAllocator(64, shape.block_tokens, seed=9)
    s.close()


def test_full_and_cached_match_oracle(case):
    wl, shape, w, prompt, s, alloc = case
    from decoder_forward_pass_amd.binding import DEC_LOGITS_ALL
    T, split = len(prompt), wl.split
    assert split == T // 2
    alloc.ensure("full", T)
    full = s.prefill([0], [T], prompt, alloc.table_array(["full"]), DEC_LOGITS_ALL).cpu().numpy()
    alloc.ensure("cached", T)
    tbl = alloc.table_array(["cached"])
    a = s.prefill([0], [split], prompt[:split], tbl, DEC_LOGITS_ALL)
    b = s.prefill([split], [T - split], prompt[split:], tbl, DEC_LOGITS_ALL)
    cached = torch.cat([a, b]).cpu().numpy()
    dec = om.OracleDecoder(w)
    ref = dec.forward([(prompt, dec.new_cache())], logits="all")
    assert ref.shape == (188, 151936)
    for path, got in (("full", full), ("cached", cached)):
        row = compare(got, ref, tol=TOL)
        row.update(type="logit_parity", case=wl.name, path=path)
        report(row)
        assert row["pass"], row


def test_batch_invariance_across_product_and_attention_paths(case):
    wl, shape, w, prompt, _, _ = case
    from decoder_forward_pass_amd.binding import DEC_LOGITS_ALL
    from decoder_forward_pass_amd.session import BlockAllocator, Session
    rng = np.random.default_rng(wl.seed + 1)
    T, LONG = len(prompt), 2100
    long_prompt = rng.integers(0, shape.vocab, LONG).astype(np.int32)
    n_blocks = 2 * (LONG + T) // shape.block_tokens + 8
    s = Session(shape, w, max_context=LONG, n_blocks=n_blocks, max_rows=LONG + T, max_seqs=2)
    try:
        alloc = BlockAllocator(n_blocks, shape.block_tokens, seed=10)
        alloc.ensure("long", LONG)
        alloc.ensure("short", T)
        alloc.ensure("alone", T)
        print(f"[f32] {LONG} + {T} rows in one call", flush=True)
        both = s.prefill([0, 0], [LONG, T], np.concatenate([long_prompt, prompt]),
                         alloc.table_array(["long", "short"]), DEC_LOGITS_ALL)
        mine = both[LONG:].cpu().numpy()
        del both
        alone = s.prefill([0], [T], prompt, alloc.table_array(["alone"]), DEC_LOGITS_ALL).cpu().numpy()
    finally:
        s.close()
    same = int(np.sum(np.all(mine.view(np.uint32) == alone.view(np.uint32), axis=1)))
    report({"type": "batch_invariance", "case": f"{wl.name}_with_{LONG}", "identical_rows": same, "rows": T})
    assert same == T
