"""Prefix-cache reuse through the forward pass ("Candle model runner" section 2.2, KvPool: full
blocks are indexed by their prefix, released ones are kept in an LRU cache and reacquired by a
lookup, the oldest cached block is evicted first; section 4 tests kv_pool_bounds_and_cache_
lifecycle and kv_pool_evicts_the_oldest_cached_block).

Sequence A prefills its prompt into blocks handed out by the library's block manager and
registers its full blocks under their prefix keys. Sequence B shares A's first three blocks of
tokens: a lookup of each prefix key returns A's block, and B prefills only its own tail at
start = the shared length. B's logits (its tail, then a decode step) must match the oracle's
full forward of B's whole prompt, and A's blocks must be left byte for byte as they were. After
both are released the blocks are cached; an allocation that needs more than the free blocks
evicts the oldest cached ones first, and sequence C, which shares A's prefix again, reacquires
the blocks still cached and gets the oracle's logits.
"""

import dataclasses

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from gpu_util import compare, report
import oracle.model as om
from synthetic import MODELS, make_weights

SHAPE = dataclasses.replace(MODELS["tiny_f32"], name="tiny_prefix", weight_dtype="bf16", kv_dtype="f16",
                            gains="random")
BT = SHAPE.block_tokens
REL = 2e-2


def slab_bytes(s, blk):
    """Every layer's K and V slab of pool block blk, as bytes (a copy)."""
    el = 2
    slab = SHAPE.n_kv_heads * BT * SHAPE.head_dim * el
    p = s.pool.view(SHAPE.n_layers * 2, s.cfg.n_blocks, slab)
    return p[:, blk].clone()


def keys_of(tokens, n_full):
    """Prefix keys of the first n_full blocks: each names its block's tokens and every earlier block."""
    from decoder_forward_pass_amd import binding as B
    keys, parent = [], 0
    for b in range(n_full):
        parent = B.dec_prefix_key(parent, tokens[b * BT:(b + 1) * BT])
        keys.append(parent)
    return keys


def oracle_logits(w, tokens):
    dec = om.OracleDecoder(w)
    return dec.forward([(tokens, dec.new_cache())], logits="all")


def test_prefix_blocks_are_shared_reacquired_and_evicted_oldest_first():
    from decoder_forward_pass_amd import binding as B
    from decoder_forward_pass_amd.session import Session
    w = make_weights(SHAPE)
    n_blocks = 12
    s = Session(SHAPE, w, max_context=128, n_blocks=n_blocks, max_rows=128, max_seqs=2)
    pool = B.BlockPool(n_blocks, BT, prefix_cache=True)
    rng = np.random.default_rng(8)
    shared = rng.integers(0, SHAPE.vocab, 3 * BT).astype(np.int32)
    a_tok = np.concatenate([shared, rng.integers(0, SHAPE.vocab, 9).astype(np.int32)])  # 3 full + 1 partial
    b_tok = np.concatenate([shared, rng.integers(0, SHAPE.vocab, 20).astype(np.int32)])  # tail of 20

    # A: four blocks, prefill, the three full blocks registered under their prefix keys
    a_blk = pool.alloc(4)
    s.prefill([0], [len(a_tok)], a_tok, np.array([a_blk], np.int32), B.DEC_LOGITS_NONE)
    keys = keys_of(a_tok, 3)
    for b, key in zip(a_blk[:3], keys):
        pool.set_fill(b, BT)
        assert pool.register(b, key) == b
    pool.set_fill(a_blk[3], 9)
    torch.cuda.synchronize()
    before = [slab_bytes(s, b) for b in a_blk]

    # B: the shared prefix by lookup, its own blocks for the tail, prefill of the tail only
    b_keys = keys_of(b_tok, 3)
    assert b_keys == keys
    hits = [pool.lookup(k) for k in b_keys]
    assert hits == a_blk[:3]
    assert all(pool.info(b)[1] == 2 for b in hits)  # referenced by A and B
    b_own = pool.alloc(2)
    b_tbl = np.array([hits + b_own], np.int32)
    tail = s.prefill([3 * BT], [20], b_tok[3 * BT:], b_tbl, B.DEC_LOGITS_ALL).cpu().numpy()
    nxt = int(rng.integers(0, SHAPE.vocab))
    step = s.decode_step([len(b_tok)], b_tbl, tokens_host=np.array([nxt], np.int32)).cpu().numpy()
    torch.cuda.synchronize()
    ref = oracle_logits(w, np.concatenate([b_tok, [nxt]]).astype(np.int32))
    row = compare(np.concatenate([tail, step]), ref[3 * BT:], rel_range=REL)
    row.update(type="logit_parity", case="prefix_reuse", path="B tail on A's blocks + decode")
    report(row)
    assert row["pass"], row
    for b, old in zip(a_blk, before):
        assert torch.equal(slab_bytes(s, b), old), f"A's block {b} changed"

    # release both: the registered blocks become cached (oldest first: A's releases come first)
    for b in a_blk:
        pool.release(b)
    for b in hits + b_own:
        pool.release(b)
    st = {b: pool.info(b)[0] for b in a_blk[:3]}
    assert all(v == B.DEC_BLOCK_CACHED for v in st.values())
    n_free, n_used, n_cached = pool.counts()
    assert (n_used, n_cached) == (0, 3)
    # take every free block and one more: the oldest cached block (A's first) is evicted
    taken = pool.alloc(n_free + 1)
    assert a_blk[0] in taken and pool.info(a_blk[1])[0] == B.DEC_BLOCK_CACHED
    assert pool.lookup(keys[0]) == -1  # its key left the index
    for b in taken:
        pool.release(b)

    # C: shares A's prefix; the first block must be recomputed, the next two are reacquired
    c_tok = np.concatenate([shared, rng.integers(0, SHAPE.vocab, 5).astype(np.int32)])
    c_keys = keys_of(c_tok, 3)
    got = [pool.lookup(k) for k in c_keys]
    assert got[0] == -1 and got[1:] == a_blk[1:3]
    assert all(pool.info(b)[:2] == (B.DEC_BLOCK_USED, 1) for b in got[1:])
    # (a prefix is reused only up to its first miss: C recomputes from block 0 into new blocks)
    for b in got[1:]:
        pool.release(b)
    c_blk = pool.alloc(4)
    lg = s.prefill([0], [len(c_tok)], c_tok, np.array([c_blk], np.int32), B.DEC_LOGITS_ALL).cpu().numpy()
    row = compare(lg, oracle_logits(w, c_tok), rel_range=REL)
    row.update(type="logit_parity", case="prefix_reuse", path="C after eviction")
    report(row)
    assert row["pass"], row
    pool.close()
    s.close()


def test_reacquired_cached_blocks_serve_a_later_sequence():
    """A's full blocks, released into the cache, are looked up again by B (reacquired from the
    LRU, not recomputed); B's tail prefill on them matches the oracle."""
    from decoder_forward_pass_amd import binding as B
    from decoder_forward_pass_amd.session import Session
    w = make_weights(SHAPE)
    s = Session(SHAPE, w, max_context=128, n_blocks=10, max_rows=128, max_seqs=1)
    pool = B.BlockPool(10, BT, prefix_cache=True)
    rng = np.random.default_rng(9)
    a_tok = rng.integers(0, SHAPE.vocab, 2 * BT).astype(np.int32)
    a_blk = pool.alloc(2)
    s.prefill([0], [len(a_tok)], a_tok, np.array([a_blk], np.int32), B.DEC_LOGITS_NONE)
    keys = keys_of(a_tok, 2)
    for b, k in zip(a_blk, keys):
        pool.set_fill(b, BT)
        pool.register(b, k)
        pool.release(b)
    assert pool.counts()[2] == 2  # both cached
    b_tok = np.concatenate([a_tok, rng.integers(0, SHAPE.vocab, 7).astype(np.int32)])
    hits = [pool.lookup(k) for k in keys_of(b_tok, 2)]
    assert hits == a_blk and pool.counts()[2] == 0
    own = pool.alloc(1)
    lg = s.prefill([2 * BT], [7], b_tok[2 * BT:], np.array([hits + own], np.int32), B.DEC_LOGITS_ALL).cpu().numpy()
    row = compare(lg, oracle_logits(w, b_tok)[2 * BT:], rel_range=REL)
    row.update(type="logit_parity", case="prefix_reuse", path="B on reacquired cached blocks")
    report(row)
    assert row["pass"], row
    pool.close()
    s.close()
