"""dec_decode_step_static -- the decode step for callers that cannot allocate -- against
dec_decode_step, through the C ABI: the same logits and greedy ids bit for bit, and the same K/V
written to the pool, on two calls in a row (the second with fewer sequences), on the full-width
two-layer decoder (decode GEMMs, LM-head candidates, a row long enough for the split attention's
segment states) and on the tiny float32 decoder (the two-pass argmax; the static array holds
no K-part sums, so its float32 products add the parts inside one block where the workspace
step splits them over blocks). A step whose scratch would not fit the static array is refused
before anything runs."""

import dataclasses

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from synthetic import MODELS, make_weights

CASES = {
    "w1024_bf16": (dataclasses.replace(MODELS["q06b_bf16"], name="static_bf16", n_layers=2),
                   [4200, 700, 33, 1, 150, 2000]),
    "tiny_f32": (dataclasses.replace(MODELS["tiny_f32"], gains="random"), [40, 7, 1, 19]),
}


def _blocks_equal(pool, shape, n_blocks, a_ids, b_ids):
    """The K and V slabs of blocks a_ids equal those of b_ids, byte for byte, in every layer."""
    el = 4 if shape.kv_dtype == "f32" else 2
    slab = shape.n_kv_heads * shape.block_tokens * shape.head_dim * el
    p = pool.view(shape.n_layers * 2, n_blocks, slab)
    a = p[:, torch.as_tensor(a_ids, device=pool.device)]
    b = p[:, torch.as_tensor(b_ids, device=pool.device)]
    return bool(torch.equal(a, b))


@pytest.mark.parametrize("name", list(CASES))
def test_static_decode_step_equals_the_workspace_decode_step(name):
    from decoder_forward_pass_amd import binding as B
    from decoder_forward_pass_amd.session import BlockAllocator, Session
    shape, lens = CASES[name]
    w = make_weights(shape)
    S = len(lens)
    ctx_len = max(lens) + 3
    per = -(-ctx_len // shape.block_tokens)
    n_blocks = 2 * S * per
    s = Session(shape, w, max_context=ctx_len, n_blocks=n_blocks, max_rows=sum(lens), max_seqs=S)
    s.pool.zero_()  # slots past each sequence's position are then equal (zero) in both copies
    alloc = BlockAllocator(n_blocks, shape.block_tokens, seed=21)
    rng = np.random.default_rng(31)
    prompts = [rng.integers(0, shape.vocab, n).astype(np.int32) for n in lens]
    for copy in "AB":
        for i in range(S):
            alloc.ensure((copy, i), ctx_len)
        s.prefill([0] * S, lens, np.concatenate(prompts), alloc.table_array([(copy, i) for i in range(S)]),
                  B.DEC_LOGITS_NONE)
    pos = np.array(lens, np.int32)
    toks = rng.integers(0, shape.vocab, S).astype(np.int32)
    print(f"[static] {name}: call 1, {S} sequences", flush=True)
    results = []
    for rows in (list(range(S)), [2, 0, S - 1]):  # the second call: a smaller batch
        out = {}
        for copy, static in (("A", False), ("B", True)):
            tbl = alloc.table_array([(copy, i) for i in rows])
            nxt = torch.full((len(rows),), -1, dtype=torch.int32, device="cuda")
            lg = s.decode_step(pos[rows], tbl, tokens_host=toks[rows], next_tokens=nxt, static=static)
            torch.cuda.synchronize()
            out[copy] = (lg.cpu().numpy(), nxt.cpu().numpy())
        la, na = out["A"]
        lb, nb = out["B"]
        assert np.array_equal(la.view(np.uint32), lb.view(np.uint32)), f"{name}: logits differ ({len(rows)} rows)"
        assert np.array_equal(na, nb) and np.all(na >= 0)
        assert _blocks_equal(s.pool, shape, n_blocks, [alloc.tables[("A", i)] for i in rows],
                             [alloc.tables[("B", i)] for i in rows])
        results.append(len(rows))
        pos[rows] += 1
        toks[rows] = na
        print(f"[static] {name}: {len(rows)} rows equal", flush=True)
    s.close()
    assert results == [S, 3]


def test_static_decode_step_refuses_a_step_beyond_its_array():
    from decoder_forward_pass_amd import binding as B
    from decoder_forward_pass_amd.session import BlockAllocator, Session
    shape = dataclasses.replace(MODELS["q06b_bf16"], name="static_many", n_layers=1)
    S = 400  # about 60 KB of scratch per sequence at this width: more than 16 MiB
    s = Session(shape, make_weights(shape), max_context=64, n_blocks=S, max_rows=S, max_seqs=S)
    alloc = BlockAllocator(S, shape.block_tokens, seed=2)
    for i in range(S):
        alloc.ensure(i, 1)
    tbl = alloc.table_array(list(range(S)))
    before = s.pool.clone()
    with pytest.raises(B.DecError) as e:
        s.decode_step(np.zeros(S, np.int32), tbl, tokens_host=np.zeros(S, np.int32), static=True)
    assert e.value.code == B.DEC_E_CAPACITY and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.equal(before, s.pool)
    s.close()
