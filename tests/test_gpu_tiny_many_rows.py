"""Batch invariance at many rows on the two-layer tiny decoder: 33 prompts of 1,000 tokens in one
prefill call (33,000 rows) against one of them alone, every logit of that prompt compared bit for
bit.

At that row count the products take paths that small calls never take, on shapes that are not
multiples of the tiles. bf16 weights: the output and down products (N = 64) and gate/up (192
features) run on the 128 x 128 tiles, the LM head on the 256 x 256 tiles. uint4 weights: each
layer's seven matrices (64 to 192 columns) are widened to bf16 first. float32 weights: every
product adds its K parts inside one block, where the lone prompt's products split them
over blocks. The lone prompt (1,000 rows) takes the 64 x 64 tiles, dequantising uint4 in the
products. Expected values: the library's own lone call (the results must not depend on the rows
around a prompt, "Candle model runner" 2.4); the oracle checks the lone path in the other tests.
"""

import dataclasses
import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from gpu_util import report
from synthetic import MODELS, make_weights

_R = dict(gains="random")
VARIANTS = {
    "bf16_f16kv": dataclasses.replace(MODELS["tiny_f32"], name="tiny_bf16", weight_dtype="bf16", kv_dtype="f16", **_R),
    "uint4_f16kv": dataclasses.replace(MODELS["tiny_f32"], name="tiny_uint4", weight_dtype="uint4", kv_dtype="f16",
                                       **_R),
    "f32": dataclasses.replace(MODELS["tiny_f32"], name="tiny_f32_gains", **_R),
}
S, T, PICK = 33, 1000, 17


@pytest.mark.parametrize("name", list(VARIANTS))
def test_many_rows_equal_the_prompt_alone(name):
    from decoder_forward_pass_amd.binding import DEC_LOGITS_ALL
    from decoder_forward_pass_amd.session import BlockAllocator, Session
    shape = VARIANTS[name]
    w = make_weights(shape)
    rng = np.random.default_rng(91)
    prompts = [rng.integers(0, shape.vocab, T).astype(np.int32) for _ in range(S)]
    n_blocks = (S + 1) * math.ceil(T / shape.block_tokens)
    s = Session(shape, w, max_context=T, n_blocks=n_blocks, max_rows=S * T, max_seqs=S)
    try:
        alloc = BlockAllocator(n_blocks, shape.block_tokens, seed=12)
        for i in range(S):
            alloc.ensure(i, T)
        alloc.ensure("alone", T)
        print(f"[tiny {name}] {S} x {T} rows in one call", flush=True)
        both = s.prefill([0] * S, [T] * S, np.concatenate(prompts), alloc.table_array(list(range(S))),
                         DEC_LOGITS_ALL)
        mine = both[PICK * T:(PICK + 1) * T].clone()
        del both
        alone = s.prefill([0], [T], prompts[PICK], alloc.table_array(["alone"]), DEC_LOGITS_ALL)
        torch.cuda.synchronize()
        same = int(torch.sum(torch.all(mine == alone, dim=1)))
    finally:
        s.close()
    report({"type": "batch_invariance", "case": f"tiny_{name}_{S}x{T}", "identical_rows": same, "rows": T})
    assert same == T
