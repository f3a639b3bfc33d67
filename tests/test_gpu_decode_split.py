"""GPU parity of decode attention on rows split into key segments: a row with more than 4,096
keys before its position is attended by one workgroup per 4,096-key segment, and the segments'
states are merged in order with the new key's ("Candle model runner" 2.4, second equation:
the softmax over every key up to the position, computed here in parts).

On the two-layer tiny decoder: decode steps at positions on both sides of the one-, two- and
three-segment boundaries (4,095 .. 4,097 and 8,191 .. 8,193 keys before the position) against
the oracle's full forward (float32 gate 1e-3, "Proving it's the same model", "Pick the
tolerance before looking"; f16-KV gate 2e-2 of the row's logit range, "Candle model runner"
2.4, "The f16 bound"), and a batch that mixes split and unsplit rows against each row alone,
bit for bit.
"""

import dataclasses

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from gpu_util import compare, report
import oracle.model as om
from synthetic import MODELS, make_weights

VARIANTS = {
    "f32": MODELS["tiny_f32"],
    "bf16_f16kv": dataclasses.replace(MODELS["tiny_f32"], name="tiny_bf16", weight_dtype="bf16", kv_dtype="f16"),
    "gqa8_bf16_f16kv": dataclasses.replace(MODELS["tiny_f32"], name="tiny_gqa8", n_heads=16, n_kv_heads=2,
                                           weight_dtype="bf16", kv_dtype="f16"),
    "gqa4_bf16_f16kv": dataclasses.replace(MODELS["tiny_f32"], name="tiny_gqa4", n_heads=8, n_kv_heads=2,
                                           weight_dtype="bf16", kv_dtype="f16"),
    "mha_bf16_f16kv": dataclasses.replace(MODELS["tiny_f32"], name="tiny_mha", n_kv_heads=4, weight_dtype="bf16",
                                          kv_dtype="f16"),
}
T = 8194          # prompt tokens of the long sequence (positions 0 .. 8193)
FIRST = (4095, 4096, 4097)
SECOND = (8191, 8192, 8193)
MAX_CTX = 8300
N_BLOCKS = 2200


def gate(name):
    return dict(tol=1e-3) if name == "f32" else dict(rel_range=2e-2)


@pytest.fixture(scope="module", params=list(VARIANTS))
def setup(request):
    from decoder_forward_pass_amd.session import BlockAllocator, Session
    shape = VARIANTS[request.param]
    w = make_weights(shape)
    print(f"[split] variant {request.param}", flush=True)
    s = Session(shape, w, max_context=MAX_CTX, n_blocks=N_BLOCKS, max_rows=MAX_CTX, max_seqs=4)
    yield request.param, shape, w, s, BlockAllocator(N_BLOCKS, shape.block_tokens, seed=9)
    s.close()


@pytest.fixture(scope="module")
def long_prompt():
    return np.random.default_rng(8194).integers(0, MODELS["tiny_f32"].vocab, T).astype(np.int32)


def test_split_decode_matches_oracle(setup, long_prompt):
    name, shape, w, s, alloc = setup
    from decoder_forward_pass_amd.binding import DEC_LOGITS_NONE
    p = long_prompt
    dec = om.OracleDecoder(w)
    ref = dec.forward([(p, dec.new_cache())], logits="all")
    seq = ("split", name)
    alloc.ensure(seq, T)
    tbl = alloc.table_array([seq])
    rows = []
    s.prefill([0], [FIRST[0]], p[:FIRST[0]], tbl, DEC_LOGITS_NONE)
    for pos in FIRST:
        rows.append(s.decode_step([pos], tbl, tokens_host=p[pos:pos + 1]).cpu().numpy()[0])
    s.prefill([FIRST[-1] + 1], [SECOND[0] - FIRST[-1] - 1], p[FIRST[-1] + 1:SECOND[0]], tbl, DEC_LOGITS_NONE)
    for pos in SECOND:
        rows.append(s.decode_step([pos], tbl, tokens_host=p[pos:pos + 1]).cpu().numpy()[0])
    row = compare(np.array(rows), ref[list(FIRST + SECOND)], **gate(name))
    row.update(type="logit_parity", case=f"tiny_{name}_decode_split", path="decode",
               positions=list(FIRST + SECOND))
    report(row)
    assert row["pass"], row


def test_split_rows_batch_invariance_is_bit_exact(setup, long_prompt):
    name, shape, w, s, alloc = setup
    from decoder_forward_pass_amd.binding import DEC_LOGITS_NONE
    lens = [8193, 30, 4097]  # three, one and two segments
    toks = np.array([long_prompt[n] for n in lens], np.int32)
    for tag in ("alone", "batch"):
        for i, n in enumerate(lens):
            seq = (tag, name, i)
            alloc.ensure(seq, n + 1)
            s.prefill([0], [n], long_prompt[:n], alloc.table_array([seq]), DEC_LOGITS_NONE)
    order = [1, 0, 2]
    seqs = [("batch", name, i) for i in order]
    both = s.decode_step([lens[i] for i in order], alloc.table_array(seqs), tokens_host=toks[order]).clone()
    for k, i in enumerate(order):
        one = s.decode_step([lens[i]], alloc.table_array([("alone", name, i)]), tokens_host=toks[i:i + 1])
        torch.cuda.synchronize()
        assert torch.equal(both[k], one[0]), f"decode row of {lens[i]} keys differs when batched"
