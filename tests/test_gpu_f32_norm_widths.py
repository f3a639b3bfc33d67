"""The float32 RMSNorm written by the residual products' combine, at the other vector-norm widths
(d = 256 and 512: one and two float4 per lane), on two-layer float32 decoders with per-channel
gains.

A 96-token prompt alone: every product's 64 x 64 grid is small, so K is split over blocks and
the O and down combines also write the norm that follows. Parity: every logit against the
float64 oracle, max-abs <= 1e-3 ("Proving it's the same model"). Batch invariance: the same
prompt inside one call with a 4,200-token prompt, where no product splits K and each norm is a
launch of its own; the prompt's logits must be the same bits ("Candle model runner" 2.4: a row's
result does not depend on the rows around it). Decode: float32 decode steps take the same
split products and fused norms (one row per step); the prompt's last 8 tokens, fed one step at a
time after a prefill of the rest, against the oracle's logits at those positions.
"""

import dataclasses
import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from gpu_util import compare, report
import oracle.model as om
from synthetic import MODELS, make_weights

T_SMALL, T_BIG = 96, 4200


def shape_for(d):
    return dataclasses.replace(MODELS["tiny_f32"], name=f"f32_d{d}", d_model=d, n_heads=4, n_kv_heads=2,
                               head_dim=64, ff_hidden=2 * d, vocab=1024, gains="random")


@pytest.mark.parametrize("d", [256, 512])
def test_fused_norm_matches_oracle_and_the_unsplit_path(d):
    from decoder_forward_pass_amd.binding import DEC_LOGITS_ALL
    from decoder_forward_pass_amd.session import BlockAllocator, Session
    shape = shape_for(d)
    w = make_weights(shape)
    rng = np.random.default_rng(d)
    small = rng.integers(0, shape.vocab, T_SMALL).astype(np.int32)
    big = rng.integers(0, shape.vocab, T_BIG).astype(np.int32)
    n_blocks = 2 * math.ceil(T_SMALL / shape.block_tokens) + math.ceil(T_BIG / shape.block_tokens) + 8
    s = Session(shape, w, max_context=T_BIG, n_blocks=n_blocks, max_rows=T_SMALL + T_BIG, max_seqs=2)
    try:
        alloc = BlockAllocator(n_blocks, shape.block_tokens, seed=d)
        alloc.ensure("alone", T_SMALL)
        alloc.ensure("small", T_SMALL)
        alloc.ensure("big", T_BIG)
        print(f"[f32 d={d}] {T_SMALL} rows alone, then {T_SMALL} + {T_BIG} rows in one call", flush=True)
        alone = s.prefill([0], [T_SMALL], small, alloc.table_array(["alone"]), DEC_LOGITS_ALL)
        both = s.prefill([0, 0], [T_SMALL, T_BIG], np.concatenate([small, big]),
                         alloc.table_array(["small", "big"]), DEC_LOGITS_ALL)
        mine = both[:T_SMALL].clone()
        del both
        torch.cuda.synchronize()
        same = int(torch.sum(torch.all(mine == alone, dim=1)))
        got = alone.cpu().numpy()
    finally:
        s.close()
    dec = om.OracleDecoder(w)
    ref = dec.forward([(small, dec.new_cache())], logits="all")
    row = compare(got, ref, tol=1e-3)
    row.update(type="logit_parity", case=f"f32_d{d}_t{T_SMALL}", path="split products, fused norm")
    report(row)
    report({"type": "batch_invariance", "case": f"f32_d{d}_{T_SMALL}_in_{T_SMALL + T_BIG}", "identical_rows": same,
            "rows": T_SMALL})
    assert row["pass"], row
    assert same == T_SMALL


@pytest.mark.parametrize("d", [256, 512])
def test_fused_norm_in_decode_steps_matches_oracle(d):
    from decoder_forward_pass_amd.binding import DEC_LOGITS_ALL
    from decoder_forward_pass_amd.session import BlockAllocator, Session
    shape = shape_for(d)
    w = make_weights(shape)
    prompt = np.random.default_rng(d + 1).integers(0, shape.vocab, T_SMALL).astype(np.int32)
    p0 = T_SMALL - 8
    n_blocks = math.ceil(T_SMALL / shape.block_tokens) + 4
    s = Session(shape, w, max_context=T_SMALL, n_blocks=n_blocks, max_rows=T_SMALL, max_seqs=1)
    try:
        alloc = BlockAllocator(n_blocks, shape.block_tokens, seed=d + 1)
        alloc.ensure("dec", T_SMALL)
        tbl = alloc.table_array(["dec"])
        print(f"[f32 d={d}] prefill {p0}, then {T_SMALL - p0} decode steps", flush=True)
        s.prefill([0], [p0], prompt[:p0], tbl, DEC_LOGITS_ALL)
        rows = [s.decode_step([pos], tbl, tokens_host=prompt[pos:pos + 1]).cpu().numpy()[0]
                for pos in range(p0, T_SMALL)]
    finally:
        s.close()
    dec = om.OracleDecoder(w)
    ref = dec.forward([(prompt, dec.new_cache())], logits="all")
    row = compare(np.array(rows), ref[p0:], tol=1e-3)
    row.update(type="logit_parity", case=f"f32_d{d}_t{T_SMALL}", path="decode")
    report(row)
    assert row["pass"], row
