"""GPU parity on the two-layer tiny decoder (float32, and bf16 / f16-KV / uint4 / symmetric int4
variants).

Every call goes through the C ABI (ctypes binding); expected values come only from the
oracle. Gates: float32 max-abs <= 1e-3 ("Proving it's the same model", "Pick the tolerance
before looking"); bf16 / f16-KV / 4-bit per-row max-abs <= 2e-2 of the row's oracle logit
range ("Candle model runner" 2.4, "The f16 bound": 1e-3 of the largest logit, 2e-2).
"""

import dataclasses

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from gpu_util import compare, report
import oracle.model as om
from oracle import numerics as nx
from oracle import paged
from synthetic import MODELS, WORKLOADS, make_prompts, make_weights

FP32_TOL = 1e-3
REL_RANGE = 2e-2

_R = dict(gains="random")  # per-channel norm gains, uniform in [0.5, 1.5]
VARIANTS = {
    # the two-layer configuration as stated: float32, gains 1.0
    "f32": MODELS["tiny_f32"],
    "f32_gains": dataclasses.replace(MODELS["tiny_f32"], name="tiny_f32_gains", **_R),
    "bf16_f16kv": dataclasses.replace(MODELS["tiny_f32"], name="tiny_bf16", weight_dtype="bf16", kv_dtype="f16", **_R),
    "uint4_f16kv": dataclasses.replace(MODELS["tiny_f32"], name="tiny_uint4", weight_dtype="uint4", kv_dtype="f16",
                                       **_R),
    "int4sym_f16kv": dataclasses.replace(MODELS["tiny_f32"], name="tiny_int4sym", weight_dtype="int4sym",
                                         kv_dtype="f16", **_R),
    "bf16_f32kv": dataclasses.replace(MODELS["tiny_f32"], name="tiny_bf16_f32kv", weight_dtype="bf16", kv_dtype="f32",
                                      **_R),
    # eight query heads per KV head (the largest group the decode attention takes)
    "gqa8_bf16_f16kv": dataclasses.replace(MODELS["tiny_f32"], name="tiny_gqa8", n_heads=16, n_kv_heads=2,
                                           weight_dtype="bf16", kv_dtype="f16", **_R),
    # one KV head per query head: grouped-query attention reduced to multi-head attention
    "mha_bf16_f16kv": dataclasses.replace(MODELS["tiny_f32"], name="tiny_mha", n_kv_heads=4, weight_dtype="bf16",
                                          kv_dtype="f16", **_R),
    # the other block sizes the library accepts
    "bf16_f16kv_b32": dataclasses.replace(MODELS["tiny_f32"], name="tiny_bf16_b32", weight_dtype="bf16",
                                          kv_dtype="f16", block_tokens=32, **_R),
    "bf16_f16kv_b64": dataclasses.replace(MODELS["tiny_f32"], name="tiny_bf16_b64", weight_dtype="bf16",
                                          kv_dtype="f16", block_tokens=64, **_R),
    "f32_b32": dataclasses.replace(MODELS["tiny_f32"], name="tiny_f32_b32", block_tokens=32, **_R),
    # the other head size the library accepts (Q width 256, four times d_model)
    "hd64_bf16_f16kv": dataclasses.replace(MODELS["tiny_f32"], name="tiny_hd64", head_dim=64, weight_dtype="bf16",
                                           kv_dtype="f16", **_R),
    "hd64_f32": dataclasses.replace(MODELS["tiny_f32"], name="tiny_hd64_f32", head_dim=64, **_R),
}


def gate(name):
    return dict(tol=FP32_TOL) if VARIANTS[name].weight_dtype == "f32" and VARIANTS[name].kv_dtype == "f32" \
        else dict(rel_range=REL_RANGE)


@pytest.fixture(scope="module", params=list(VARIANTS))
def setup(request):
    from decoder_forward_pass_amd.session import BlockAllocator, Session
    shape = VARIANTS[request.param]
    w = make_weights(shape)
    s = Session(shape, w, max_context=256, n_blocks=160, max_rows=256, max_seqs=8)
    yield request.param, shape, w, s, BlockAllocator(160, shape.block_tokens, seed=5)
    s.close()


@pytest.fixture(scope="module")
def prompt():
    return make_prompts(WORKLOADS["tiny_f32_t16"])[0]


def oracle_full(w, prompt):
    dec = om.OracleDecoder(w)
    c = dec.new_cache()
    return dec.forward([(prompt, c)], logits="all"), c


def test_full_and_cached_paths_match_oracle(setup, prompt):
    name, shape, w, s, alloc = setup
    from decoder_forward_pass_amd.binding import DEC_LOGITS_ALL
    T = len(prompt)
    split = WORKLOADS["tiny_f32_t16"].split
    ref, _ = oracle_full(w, prompt)
    alloc.ensure(("full", name), T)
    full = s.prefill([0], [T], prompt, alloc.table_array([("full", name)]), DEC_LOGITS_ALL)
    alloc.ensure(("cached", name), T)
    tbl = alloc.table_array([("cached", name)])
    first = s.prefill([0], [split], prompt[:split], tbl, DEC_LOGITS_ALL)
    second = s.prefill([split], [T - split], prompt[split:], tbl, DEC_LOGITS_ALL)
    torch.cuda.synchronize()
    cached = torch.cat([first, second]).cpu().numpy()
    for path, got in (("full", full.cpu().numpy()), ("cached", cached)):
        row = compare(got, ref, **gate(name))
        row.update(type="logit_parity", case=f"tiny_{name}", path=path)
        report(row)
        assert row["pass"], row


def test_kv_pool_holds_oracle_keys_at_paged_addresses(setup, prompt):
    name, shape, w, s, alloc = setup
    from decoder_forward_pass_amd.binding import DEC_LOGITS_NONE
    T = len(prompt)
    seq = ("pool", name)
    alloc.ensure(seq, T)
    tbl = alloc.table_array([seq])
    s.prefill([0], [T], prompt, tbl, DEC_LOGITS_NONE)
    torch.cuda.synchronize()
    pool = s.pool.cpu().numpy()
    pool = pool.view(np.float32 if shape.kv_dtype == "f32" else np.uint16)
    _, cache = oracle_full(w, prompt)
    table = alloc.tables[seq]
    worst = 0.0
    for layer in range(shape.n_layers):
        for is_v in (False, True):
            ref = (cache.V if is_v else cache.K)[layer]
            for pos in range(T):
                for h in range(shape.n_kv_heads):
                    off = paged.kv_element_offset(layer, is_v, pos, h, table, s.cfg.n_blocks, shape.n_kv_heads,
                                                  shape.block_tokens, shape.head_dim)
                    got = pool[off:off + shape.head_dim]
                    if shape.kv_dtype == "f16":
                        got = nx.f16_to_f32(got)
                    worst = max(worst, float(np.max(np.abs(got.astype(np.float64) - ref[pos, h]))))
    # float32 keys: rounding only; f16 keys: 2^-11 relative of values of magnitude <= ~4
    bound = 1e-5 if (shape.kv_dtype == "f32" and shape.weight_dtype == "f32") else 2e-2
    report({"type": "kv_pool", "case": f"tiny_{name}", "max_absolute_error": worst, "tolerance": bound})
    assert worst <= bound


def test_decode_steps_match_oracle(setup, prompt):
    name, shape, w, s, alloc = setup
    from decoder_forward_pass_amd.binding import DEC_LOGITS_ALL
    T, p0 = len(prompt), 5
    ref, _ = oracle_full(w, prompt)
    seq = ("decode", name)
    alloc.ensure(seq, T)
    tbl = alloc.table_array([seq])
    s.prefill([0], [p0], prompt[:p0], tbl, DEC_LOGITS_ALL)
    rows = []
    dev_tok = torch.empty(1, dtype=torch.int32, device="cuda")
    for pos in range(p0, T):
        if pos % 2:
            lg = s.decode_step([pos], tbl, tokens_host=prompt[pos:pos + 1])
        else:  # token ids read from device memory
            dev_tok.fill_(int(prompt[pos]))
            lg = s.decode_step([pos], tbl, tokens_device=dev_tok)
        rows.append(lg.cpu().numpy()[0])
    row = compare(np.array(rows), ref[p0:], **gate(name))
    row.update(type="logit_parity", case=f"tiny_{name}", path="decode")
    report(row)
    assert row["pass"], row


def test_batch_invariance_is_bit_exact(setup):
    name, shape, w, s, alloc = setup
    from decoder_forward_pass_amd.binding import DEC_LOGITS_ALL
    rng = np.random.default_rng(77)
    lens = [7, 19, 1]
    starts = [0, 0, 0]
    prompts = [rng.integers(0, shape.vocab, n).astype(np.int32) for n in lens]
    # alone
    alone = []
    for i, p in enumerate(prompts):
        seq = ("alone", name, i)
        alloc.ensure(seq, len(p))
        alone.append(s.prefill([0], [len(p)], p, alloc.table_array([seq]), DEC_LOGITS_ALL).clone())
    # together, in a different order
    order = [2, 0, 1]
    seqs = [("batch", name, i) for i in order]
    for i, sq in zip(order, seqs):
        alloc.ensure(sq, lens[i])
    tbl = alloc.table_array(seqs)
    both = s.prefill([starts[i] for i in order], [lens[i] for i in order],
                     np.concatenate([prompts[i] for i in order]), tbl, DEC_LOGITS_ALL)
    torch.cuda.synchronize()
    r = 0
    for i in order:
        assert torch.equal(both[r:r + lens[i]], alone[i]), f"sequence {i} differs when batched"
        r += lens[i]
    # decode: batch of 3 vs alone, bit for bit
    toks = rng.integers(0, shape.vocab, 3).astype(np.int32)
    for i in order:
        alloc.ensure(("alone", name, i), lens[i] + 1)
        alloc.ensure(("batch", name, i), lens[i] + 1)
    dec_b = s.decode_step([lens[i] for i in order], alloc.table_array(seqs), tokens_host=toks[order])
    for k, i in enumerate(order):
        one = s.decode_step([lens[i]], alloc.table_array([("alone", name, i)]), tokens_host=toks[i:i + 1])
        torch.cuda.synchronize()
        assert torch.equal(dec_b[k], one[0]), f"decode row {i} differs when batched"


def test_decode_at_position_zero(setup, prompt):
    # a sequence's first token through dec_decode_step: attention over the new key alone
    name, shape, w, s, alloc = setup
    seq = ("first", name)
    alloc.ensure(seq, 1)
    lg = s.decode_step([0], alloc.table_array([seq]), tokens_host=prompt[:1]).cpu().numpy()
    dec = om.OracleDecoder(w)
    ref = dec.forward([(prompt[:1], dec.new_cache())], logits="all")
    row = compare(lg, ref, **gate(name))
    row.update(type="logit_parity", case=f"tiny_{name}", path="decode_pos0")
    report(row)
    assert row["pass"], row


def test_context_filled_to_the_last_position(setup):
    # prefill positions 0 .. 254, then decode at 255 = max_context - 1, the last valid position
    name, shape, w, s, alloc = setup
    from decoder_forward_pass_amd.binding import DEC_LOGITS_LAST
    T = s.cfg.max_context
    toks = np.random.default_rng(78).integers(0, shape.vocab, T).astype(np.int32)
    seq = ("full_ctx", name)
    alloc.ensure(seq, T)
    tbl = alloc.table_array([seq])
    last = s.prefill([0], [T - 1], toks[:T - 1], tbl, DEC_LOGITS_LAST).cpu().numpy()
    lg = s.decode_step([T - 1], tbl, tokens_host=toks[T - 1:]).cpu().numpy()
    dec = om.OracleDecoder(w)
    ref = dec.forward([(toks, dec.new_cache(capacity=T))], logits="all")
    row = compare(np.concatenate([last, lg]), ref[T - 2:], **gate(name))
    row.update(type="logit_parity", case=f"tiny_{name}", path="context_full")
    report(row)
    assert row["pass"], row


def test_greedy_next_tokens_are_the_argmax(setup, prompt):
    name, shape, w, s, alloc = setup
    seq = ("greedy", name)
    alloc.ensure(seq, 4)
    from decoder_forward_pass_amd.binding import DEC_LOGITS_NONE
    tbl = alloc.table_array([seq])
    s.prefill([0], [3], prompt[:3], tbl, DEC_LOGITS_NONE)
    nxt = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    lg = s.decode_step([3], tbl, tokens_host=prompt[3:4], next_tokens=nxt)
    torch.cuda.synchronize()
    assert int(nxt[0]) == int(np.argmax(lg.cpu().numpy()[0]))


def test_dequant_hook_is_bit_exact(setup):
    name, shape, w, s, alloc = setup
    from decoder_forward_pass_amd import binding as B
    for idx in (0, 2, 9, 11, 13):
        e = B.dec_weight_entry(s.cfg, idx)
        nm = e.name.decode()
        src = w.embed if nm == "embed" else w.layers[e.layer][nm]
        ref = om.widen_matrix(src, shape.weight_dtype).astype(np.float32)
        got = s.dequant(idx).cpu().numpy()
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), nm


def test_rejected_call_leaves_pool_untouched(setup, prompt):
    name, shape, w, s, alloc = setup
    from decoder_forward_pass_amd import binding as B
    torch.cuda.synchronize()
    before = s.pool.clone()
    bad = prompt.copy()
    bad[3] = shape.vocab  # outside the vocabulary
    seq = ("bad", name)
    alloc.ensure(seq, len(bad))
    with pytest.raises(B.DecError) as e:
        s.prefill([0], [len(bad)], bad, alloc.table_array([seq]), B.DEC_LOGITS_ALL)
    assert e.value.code == B.DEC_E_TOKEN
    with pytest.raises(B.DecError) as e:  # position past the context
        s.prefill([s.cfg.max_context - 2], [4], prompt[:4], np.zeros((1, 16), np.int32), B.DEC_LOGITS_ALL)
    assert e.value.code == B.DEC_E_POSITION
    torch.cuda.synchronize()
    assert torch.equal(before, s.pool)


def test_long_prompt_tiles_cached_split_and_chunks(setup):
    """200 tokens: several 64-key tiles, a cached split at an unaligned position, and chunked
    prefill; chunked and cached logits equal the single-shot ones bit for bit."""
    name, shape, w, s, alloc = setup
    from decoder_forward_pass_amd.binding import DEC_LOGITS_ALL
    rng = np.random.default_rng(31)
    T = 200
    prompt = rng.integers(0, shape.vocab, T).astype(np.int32)
    ref, _ = oracle_full(w, prompt)
    alloc.ensure(("long", name), T)
    full = s.prefill([0], [T], prompt, alloc.table_array([("long", name)]), DEC_LOGITS_ALL).clone()
    row = compare(full.cpu().numpy(), ref, **gate(name))
    row.update(type="logit_parity", case=f"tiny_{name}_t200", path="full")
    report(row)
    assert row["pass"], row
    for chunk in (77, 64, 50):
        seq = ("long", name, chunk)
        alloc.ensure(seq, T)
        tbl = alloc.table_array([seq])
        parts = [s.prefill([c0], [min(chunk, T - c0)], prompt[c0:c0 + chunk], tbl, DEC_LOGITS_ALL).clone()
                 for c0 in range(0, T, chunk)]
        got = torch.cat(parts)
        torch.cuda.synchronize()
        same = int(torch.sum(torch.all(got == full, dim=1)))
        report({"type": "chunk_invariance", "case": f"tiny_{name}_t200", "chunk": chunk,
                "identical_rows": same, "rows": T,
                "max_absolute_error": float((got - full).abs().max())})
        assert torch.equal(got, full), f"chunk {chunk}: {same}/{T} rows identical"
