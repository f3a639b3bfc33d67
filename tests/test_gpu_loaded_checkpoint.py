"""A checkpoint loaded from disk drives the forward pass ("Candle model runner" 2.3 and 2.5; "A real
model in our own decoder", sections "A safetensors file is a JSON header and raw bytes" and the
Qwen3 settings).

Seeded weights (non-unit gains) are written as a Hugging Face-named Qwen3 model directory
(config.json + model.safetensors), read back through dec_config_from_json and
dec_load_safetensors, uploaded, and run: prefill and decode logits must match the oracle's on
the same arrays. Files: float32 and bf16 at the tiny shape, bf16 at the full 0.6B width with two
layers, and an int4 file (<name>.qweight / <name>.scales, quant = int4-g32-sym). The int4 runner
agrees with itself loaded either way (quantised at load from a float32 file, or from the int4
file: the same blob, the same logits bit for bit), and closely with its dequantised float32
twin (the int4 file loaded into a float32 blob): test int4_runner_matches_its_dequantized_model.
"""

import dataclasses
import json

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from gpu_util import compare, report
import oracle.model as om
from synthetic import MODELS, make_weights
from test_loader import hf_tensors, write_st

TINY = dataclasses.replace(MODELS["tiny_f32"], gains="random")
CASES = {
    "tiny_f32": TINY,
    "tiny_bf16": dataclasses.replace(TINY, name="tiny_bf16", weight_dtype="bf16", kv_dtype="f16"),
    "w1024_bf16_2layers": dataclasses.replace(MODELS["q06b_bf16"], name="w1024", n_layers=2),
}


def config_json(shape):
    return {"model_type": "qwen3", "hidden_act": "silu", "attention_bias": False, "attention_dropout": 0.0,
            "rope_scaling": None, "use_sliding_window": False, "tie_word_embeddings": True,
            "rms_norm_eps": shape.rms_eps, "vocab_size": shape.vocab, "max_position_embeddings": 256,
            "hidden_size": shape.d_model, "num_attention_heads": shape.n_heads,
            "num_hidden_layers": shape.n_layers, "num_key_value_heads": shape.n_kv_heads,
            "head_dim": shape.head_dim, "intermediate_size": shape.ff_hidden, "rope_theta": shape.rope_base}


def load_blob(tmp_path, shape, weights, file_dtype, blob_shape, meta=None):
    """Write the model directory, read it back through the library; (cfg, blob)."""
    from decoder_forward_pass_amd import binding as B
    from decoder_forward_pass_amd.session import make_config
    d = tmp_path / shape.name
    d.mkdir(exist_ok=True)
    (d / "config.json").write_text(json.dumps(config_json(shape)))
    write_st(d / "model.safetensors", hf_tensors(weights, bf16_bits=file_dtype == "bf16"), meta=meta)
    cfg = make_config(blob_shape, max_context=256, n_blocks=64, max_rows=128, max_seqs=4)
    text = (d / "config.json").read_bytes()
    B.dec_config_from_json(text, cfg)  # the shape fields come from the file
    assert (cfg.d_model, cfg.n_layers, cfg.vocab) == (shape.d_model, shape.n_layers, shape.vocab)
    return B.dec_load_safetensors(str(d / "model.safetensors"), cfg)


def run(shape, blob, prompts, steps=3):
    """Prefill (logits of every row) of the prompts, then `steps` decode steps with fixed ids."""
    from decoder_forward_pass_amd import binding as B
    from decoder_forward_pass_amd.session import BlockAllocator, Session
    s = Session(shape, None, max_context=256, n_blocks=64, max_rows=128, max_seqs=4, blob=blob)
    alloc = BlockAllocator(64, shape.block_tokens, seed=4)
    S = len(prompts)
    for i, p in enumerate(prompts):
        alloc.ensure(i, len(p) + steps)
    tbl = alloc.table_array(list(range(S)))
    lens = [len(p) for p in prompts]
    pre = s.prefill([0] * S, lens, np.concatenate(prompts), tbl, B.DEC_LOGITS_ALL).cpu().numpy()
    dec = []
    toks = np.arange(S, dtype=np.int32) * 7 + 3
    for t in range(steps):
        dec.append(s.decode_step(np.array(lens, np.int32) + t, tbl, tokens_host=toks + t).cpu().numpy())
    torch.cuda.synchronize()
    s.close()
    return pre, np.stack(dec), toks


def oracle(weights, prompts, toks, steps=3):
    dec = om.OracleDecoder(weights)
    pre, rows = [], []
    caches = [dec.new_cache() for _ in prompts]
    for p, c in zip(prompts, caches):
        pre.append(dec.forward([(p, c)], logits="all"))
    for t in range(steps):
        rows.append(np.concatenate([dec.forward([(np.array([toks[i] + t]), c)], logits="all")
                                    for i, c in enumerate(caches)]))
    return np.concatenate(pre), np.stack(rows)


def gate(shape):
    return dict(tol=1e-3) if shape.weight_dtype == "f32" else dict(rel_range=2e-2)


@pytest.mark.parametrize("name", list(CASES))
def test_loaded_checkpoint_matches_the_oracle(tmp_path, name):
    shape = CASES[name]
    w = make_weights(shape)
    blob = load_blob(tmp_path, shape, w, "bf16" if shape.weight_dtype == "bf16" else "f32", shape)
    rng = np.random.default_rng(12)
    prompts = [rng.integers(0, shape.vocab, n).astype(np.int32) for n in (9, 23)]
    pre, dec, toks = run(shape, blob, prompts)
    rp, rd = oracle(w, prompts, toks)
    for path, got, ref in (("prefill", pre, rp), ("decode", dec.reshape(-1, shape.vocab), rd.reshape(-1, shape.vocab))):
        row = compare(got, ref, **gate(shape))
        row.update(type="logit_parity", case=f"loaded_{name}", path=path)
        report(row)
        assert row["pass"], row


def test_int4_runner_matches_its_dequantized_model(tmp_path):
    import oracle.numerics as nx
    q_shape = dataclasses.replace(TINY, name="tiny_q4", weight_dtype="int4sym", kv_dtype="f16")
    f_shape = dataclasses.replace(q_shape, name="tiny_q4_f32src", weight_dtype="f32")
    wq = make_weights(q_shape)           # the int4 file's values and scales
    wf = make_weights(f_shape)           # the float32 weights they were chosen from
    blob_file = load_blob(tmp_path, q_shape, wq, None, q_shape, meta={"quant": "int4-g32-sym"})
    blob_load = load_blob(tmp_path, f_shape, wf, "f32", q_shape)  # quantised at load
    assert np.array_equal(blob_file, blob_load)
    twin_shape = dataclasses.replace(q_shape, name="tiny_q4_twin", weight_dtype="f32", kv_dtype="f32")
    blob_twin = load_blob(tmp_path, dataclasses.replace(q_shape, name="tiny_q4_b"), wq, None, twin_shape,
                          meta={"quant": "int4-g32-sym"})
    rng = np.random.default_rng(13)
    prompts = [rng.integers(0, q_shape.vocab, n).astype(np.int32) for n in (11, 30)]
    pre_f, dec_f, toks = run(q_shape, blob_file, prompts)
    pre_l, dec_l, _ = run(q_shape, blob_load, prompts)
    assert np.array_equal(pre_f.view(np.uint32), pre_l.view(np.uint32))
    assert np.array_equal(dec_f.view(np.uint32), dec_l.view(np.uint32))
    pre_t, dec_t, _ = run(twin_shape, blob_twin, prompts)
    # the twin: float32 weights q * s and a float32 KV pool; the int4 runner rounds its operands to
    # bf16 and keeps an f16 pool: within the bf16 / f16 gate of the twin's logits
    row = compare(np.concatenate([pre_f, dec_f.reshape(-1, q_shape.vocab)]),
                  np.concatenate([pre_t, dec_t.reshape(-1, q_shape.vocab)]).astype(np.float64), rel_range=2e-2)
    row.update(type="int4_vs_dequantized_twin", case="tiny_int4sym")
    report(row)
    assert row["pass"], row
    # and both against the oracle of the int4 values
    rp, rd = oracle(wq, prompts, toks)
    row = compare(pre_t, rp, tol=1e-3)
    row.update(type="logit_parity", case="loaded_int4_twin_f32", path="prefill")
    report(row)
    assert row["pass"], row
