"""Greedy ties go to the lowest id ("Candle model runner" section 2.6: greedy takes the largest
logit, ties to the lowest id), on every greedy path of the library.

Ties are planted in the weights. After a first run finds each row's top id a, the row of the
tied embedding E for a is copied into a lower id b that no input uses: the LM head then gives
b exactly the logit of a (the same row against the same hidden state, by the same per-element
sequence), and nothing else changes. The second run must return b. The two ids are at least
1,024 apart, so on the 151,936-id vocabulary they fall in different LM-head blocks and the
choice is made when the blocks' candidates are merged; on the tiny vocabulary they fall in
different slices of the two-pass argmax. Paths: the prefill call's next ids (logits of the last
rows, two-pass argmax) and the decode step's next ids (per-block candidates of the decode LM
head, or the two-pass argmax where the decode LM head does not apply).
"""

import dataclasses

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from gpu_util import report
from synthetic import MODELS, make_weights
from synthetic.generate import Q4, Q4S

SHAPES = {
    # the full vocabulary and width with two layers: the decode LM head's block candidates
    "v151936_bf16": dataclasses.replace(MODELS["q06b_bf16"], name="ties_bf16", n_layers=2),
    "v151936_uint4": dataclasses.replace(MODELS["q06b_uint4"], name="ties_uint4", n_layers=2),
    "tiny_f32": dataclasses.replace(MODELS["tiny_f32"], gains="random"),
}
S, P = 4, 8


def copy_embed_row(embed, src: int, dst: int):
    if isinstance(embed, (Q4, Q4S)):
        out = type(embed)(*[a.copy() for a in embed])
        for a in out:
            a[dst] = a[src]
        return out
    out = embed.copy()
    out[dst] = out[src]
    return out


def run(shape, w, prompts, dec_tokens):
    from decoder_forward_pass_amd import binding as B
    from decoder_forward_pass_amd.session import BlockAllocator, Session
    s = Session(shape, w, max_context=64, n_blocks=64, max_rows=S * P, max_seqs=S)
    alloc = BlockAllocator(64, shape.block_tokens, seed=9)
    for i in range(S):
        alloc.ensure(i, P + 1)
    tbl = alloc.table_array(list(range(S)))
    nxt_p = torch.full((S,), -1, dtype=torch.int32, device="cuda")
    lp = s.prefill([0] * S, [P] * S, np.concatenate(prompts), tbl, B.DEC_LOGITS_LAST, next_tokens=nxt_p)
    nxt_d = torch.full((S,), -1, dtype=torch.int32, device="cuda")
    ld = s.decode_step([P] * S, tbl, tokens_host=dec_tokens, next_tokens=nxt_d)
    torch.cuda.synchronize()
    out = (lp.cpu().numpy(), nxt_p.cpu().numpy(), ld.cpu().numpy(), nxt_d.cpu().numpy())
    s.close()
    return out


def lowest_of_max(row):
    return int(np.flatnonzero(row == row.max()).min())


@pytest.mark.parametrize("name", list(SHAPES))
def test_greedy_ties_take_the_lowest_id(name):
    shape = SHAPES[name]
    w = make_weights(shape)
    V = shape.vocab
    rng = np.random.default_rng(404)
    prompts = [rng.integers(0, V, P).astype(np.int32) for _ in range(S)]
    dec_tokens = rng.integers(0, V, S).astype(np.int32)
    lp, np_, ld, nd = run(shape, w, prompts, dec_tokens)
    used = set(np.concatenate(prompts).tolist()) | set(dec_tokens.tolist())
    # the planted pairs: each row's top id a (prefill rows, then decode rows) gets a lower twin b
    far = 1024 if V > 4096 else 64
    tops = [int(np.argmax(row)) for row in list(lp) + list(ld)]
    pairs = []
    for a in dict.fromkeys(tops):  # distinct top ids, in row order
        b = a - far
        while b >= 0 and (b in used or b in tops or any(b == p for _, p in pairs)):
            b -= 1
        if b >= 0:
            pairs.append((a, b))
    assert len(pairs) >= 2, "too few rows with a top id far from id 0"
    w2 = dataclasses.replace(w, embed=w.embed)
    for a, b in pairs:
        w2.embed = copy_embed_row(w2.embed, a, b)
    lp2, np2, ld2, nd2 = run(shape, w2, prompts, dec_tokens)
    ties = 0
    for path, logits, nxt in (("prefill", lp2, np2), ("decode", ld2, nd2)):
        for r in range(S):
            row = logits[r]
            top = np.flatnonzero(row == row.max())
            ties += int(len(top) >= 2)
            assert int(nxt[r]) == lowest_of_max(row), (path, r, top[:4], int(nxt[r]))
    # every planted twin holds its original's logit bit for bit, and most rows end in a tie
    for logits in (lp2, ld2):
        for a, b in pairs:
            assert np.array_equal(logits[:, a].view(np.uint32), logits[:, b].view(np.uint32))
    report({"type": "greedy_ties", "case": name, "rows": 2 * S, "rows_with_tie": ties, "pairs": len(pairs)})
    assert ties >= 2
