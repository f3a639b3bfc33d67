"""Checkpoint loading on the host (dec_config_from_json, dec_load_safetensors): the Qwen3 config
whitelist of "A real model in our own decoder" (qwen_config) and the safetensors reader rules
of the same page (section "A safetensors file is a JSON header and raw bytes") and of "Candle
model runner" 2.3 (test safetensors_reader_rules: offsets from the data buffer, F16 and BF16
widening, gaps and trailing bytes refused; config_refuses_what_the_engine_cannot_run). Files are
synthetic: the tiny decoder's seeded weights written under Hugging Face's Qwen3 names."""

import dataclasses
import json
import struct

import numpy as np
import pytest

from decoder_forward_pass_amd import binding as B
from decoder_forward_pass_amd.blob import pack_blob
from decoder_forward_pass_amd.session import make_config
from synthetic import MODELS, make_weights

TINY = MODELS["tiny_f32"]
PER = ["input_layernorm", "self_attn.q_proj", "self_attn.k_proj", "self_attn.v_proj", "self_attn.q_norm",
       "self_attn.k_norm", "self_attn.o_proj", "post_attention_layernorm", "mlp.gate_proj", "mlp.up_proj",
       "mlp.down_proj"]
OURS = ["attn_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "ffn_norm", "w_gate", "w_up", "w_down"]


def hf_tensors(w, bf16_bits=False):
    """name -> (dtype, numpy array) in checkpoint form."""
    out = {}

    def mat(a):
        return ("BF16", np.asarray(a, np.uint16)) if bf16_bits else ("F32", np.asarray(a, np.float32))

    out["model.embed_tokens.weight"] = mat(w.embed)
    for l, layer in enumerate(w.layers):
        for hf, ours in zip(PER, OURS):
            a = layer[ours]
            out[f"model.layers.{l}.{hf}.weight"] = ("F32", a) if a.ndim == 1 else mat(a)
    out["model.norm.weight"] = ("F32", w.final_norm)
    return out


def write_st(path, tensors, header_text=None, extra=b"", meta=None):
    hdr, blobs, off = {}, [], 0
    if meta is not None:
        hdr["__metadata__"] = meta
    for name, (dt, a) in tensors.items():
        raw = np.ascontiguousarray(a).tobytes()
        hdr[name] = {"dtype": dt, "shape": list(a.shape), "data_offsets": [off, off + len(raw)]}
        blobs.append(raw)
        off += len(raw)
    text = header_text if header_text is not None else json.dumps(hdr).encode()
    with open(path, "wb") as f:
        f.write(struct.pack("<Q", len(text)) + text + b"".join(blobs) + extra)
    return hdr


def cfg_for(shape):
    return make_config(shape, max_context=64, n_blocks=4, max_rows=16, max_seqs=2)


def test_loads_f32_checkpoint_into_the_blob(tmp_path):
    w = make_weights(TINY)
    p = tmp_path / "model.safetensors"
    write_st(p, hf_tensors(w))
    cfg = cfg_for(TINY)
    assert np.array_equal(B.dec_load_safetensors(str(p), cfg), pack_blob(cfg, w))


def test_loads_bf16_checkpoint_and_widens_f16(tmp_path):
    shape = dataclasses.replace(TINY, weight_dtype="bf16")
    w = make_weights(shape)
    t = hf_tensors(w, bf16_bits=True)
    # a gain stored as F16 is widened exactly (0.5 and 1.5 are f16 values)
    g = np.where(np.arange(TINY.d_model) % 2 == 0, 0.5, 1.5).astype(np.float16)
    t["model.norm.weight"] = ("F16", g)
    p = tmp_path / "model.safetensors"
    write_st(p, t)
    cfg = cfg_for(shape)
    w.final_norm = g.astype(np.float32)
    assert np.array_equal(B.dec_load_safetensors(str(p), cfg), pack_blob(cfg, w))


def test_tied_lm_head_must_equal_the_embedding(tmp_path):
    w = make_weights(TINY)
    t = hf_tensors(w)
    t["lm_head.weight"] = ("F32", np.array(w.embed))
    p = tmp_path / "a.safetensors"
    write_st(p, t)
    B.dec_load_safetensors(str(p), cfg_for(TINY))
    e = np.array(w.embed)
    e[3, 5] += 1.0
    t["lm_head.weight"] = ("F32", e)
    write_st(p, t)
    with pytest.raises(B.DecError, match="tied weights differ"):
        B.dec_load_safetensors(str(p), cfg_for(TINY))


def _refused(tmp_path, match, **kw):
    w = make_weights(TINY)
    t = hf_tensors(w)
    mutate = kw.pop("mutate", None)
    if mutate:
        mutate(t)
    p = tmp_path / "bad.safetensors"
    write_st(p, t, **kw)
    with pytest.raises(B.DecError, match=match) as e:
        B.dec_load_safetensors(str(p), cfg_for(TINY))
    assert e.value.code == B.DEC_E_ARG


def test_reader_refusals(tmp_path):
    w = make_weights(TINY)
    good = json.dumps({"x": {"dtype": "F32", "shape": [1], "data_offsets": [0, 4]}})
    _refused(tmp_path, "payload", extra=b"\0")  # trailing bytes
    _refused(tmp_path, "must be an object", header_text=b"[1, 2]")
    _refused(tmp_path, "duplicate key", header_text=('{"a": 1, "a": 2}').encode())
    _refused(tmp_path, "metadata", meta={"format": 3})
    _refused(tmp_path, "unknown or unsupported dtype", mutate=lambda t: t.update(
        {"model.norm.weight": ("F64", np.asarray(w.final_norm, np.float64))}))
    _refused(tmp_path, "missing checkpoint tensor", mutate=lambda t: t.pop("model.layers.1.mlp.up_proj.weight"))
    _refused(tmp_path, "unexpected checkpoint tensor", mutate=lambda t: t.update(
        {"model.layers.0.self_attn.q_proj.bias": ("F32", np.zeros(4, np.float32))}))
    _refused(tmp_path, "shape mismatch", mutate=lambda t: t.update(
        {"model.layers.0.self_attn.k_proj.weight": ("F32", np.zeros((8, TINY.d_model), np.float32))}))
    p = tmp_path / "h.safetensors"
    with open(p, "wb") as f:  # header length beyond the file
        f.write(struct.pack("<Q", 1000) + good.encode())
    with pytest.raises(B.DecError, match="header length"):
        B.dec_load_safetensors(str(p), cfg_for(TINY))


def test_offsets_must_tile_the_data_buffer(tmp_path):
    w = make_weights(TINY)
    t = hf_tensors(w)
    p = tmp_path / "g.safetensors"
    hdr = write_st(p, t)
    data = open(p, "rb").read()
    n = struct.unpack("<Q", data[:8])[0]
    body = data[8 + n:]
    for how, m in (("gap", "gap"), ("overlap", "overlap"), ("count", "byte count")):
        h = json.loads(json.dumps(hdr))
        name = "model.norm.weight"
        s0, e0 = h[name]["data_offsets"]
        if how == "gap":  # shift the last tensor: a hole before it, past the payload end
            h[name]["data_offsets"] = [s0 + 4, e0 + 4]
        elif how == "overlap":
            h[name]["data_offsets"] = [s0 - 4, e0 - 4]
        else:
            h[name]["data_offsets"] = [s0, e0 - 4]
        text = json.dumps(h).encode()
        with open(p, "wb") as f:
            f.write(struct.pack("<Q", len(text)) + text + body)
        with pytest.raises(B.DecError, match=m):
            B.dec_load_safetensors(str(p), cfg_for(TINY))


QWEN = {"model_type": "qwen3", "hidden_act": "silu", "attention_bias": False, "attention_dropout": 0.0,
        "rope_scaling": None, "use_sliding_window": False, "tie_word_embeddings": True, "rms_norm_eps": 1e-6,
        "vocab_size": 151936, "max_position_embeddings": 40960, "hidden_size": 1024, "num_attention_heads": 16,
        "num_hidden_layers": 28, "num_key_value_heads": 8, "head_dim": 128, "intermediate_size": 3072,
        "rope_theta": 1000000}


def test_config_gives_the_0_6b_shape():
    cfg = B.dec_config()
    B.dec_config_from_json(json.dumps(QWEN).encode(), cfg)
    m = MODELS["q06b_bf16"]
    assert (cfg.n_layers, cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ff_hidden, cfg.vocab) == \
        (m.n_layers, m.d_model, m.n_heads, m.n_kv_heads, m.head_dim, m.ff_hidden, m.vocab)
    assert cfg.max_context == 40960 and cfg.rope_base == 1e6 and cfg.rope_split == cfg.qk_norm == 1


@pytest.mark.parametrize("key,value", [("rope_scaling", {"rope_type": "yarn", "factor": 4.0}),
                                       ("use_sliding_window", True), ("model_type", "llama"),
                                       ("tie_word_embeddings", False), ("attention_bias", True),
                                       ("rms_norm_eps", 1e-5), ("hidden_act", "gelu"), ("head_dim", 0),
                                       ("num_hidden_layers", None)])
def test_config_refuses_what_the_library_cannot_run(key, value):
    c = dict(QWEN)
    if value is None:
        c.pop(key)
    else:
        c[key] = value
    with pytest.raises(B.DecError) as e:
        B.dec_config_from_json(json.dumps(c).encode(), B.dec_config())
    assert e.value.code == B.DEC_E_UNSUPPORTED


def test_config_must_be_json():
    with pytest.raises(B.DecError) as e:
        B.dec_config_from_json(b'{"model_type": "qwen3",', B.dec_config())
    assert e.value.code == B.DEC_E_ARG
