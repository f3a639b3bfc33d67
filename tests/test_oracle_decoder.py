"""Decoder-level pins of the oracle and planted-mistake checks (CPU only).

* The numpy float64 decoder agrees with the independent loop-only decoder on
  the tiny model (brute force on tiny inputs).
* Full path == cached path == chunked path, and batched == alone, to 1e-12
  ("Proving it's the same model", section "Remove every source of noise
  first": the cached path must match; "Candle model runner" 2.4: batch and
  chunk invariance).
* Tied embedding, parameter count of the 0.6B shape.
* Mutants from "Candle model runner" section 5 (pitfalls) and a few more are
  planted in the oracle, one at a time, and each is caught by one of the pins.
"""

import numpy as np
import pytest

import oracle.model as om
from oracle.loops import LoopDecoder
from synthetic import MODELS, WORKLOADS, make_prompts, make_weights, param_count
from synthetic.generate import matrix_shapes
from conftest import golden_rows
import test_oracle_ops as ops


@pytest.fixture(scope="module")
def tiny_prompt():
    return make_prompts(WORKLOADS["tiny_f32_t16"])[0]


@pytest.fixture(scope="module")
def loop_logits(tiny_weights, tiny_prompt):
    logits, _ = LoopDecoder(tiny_weights).run(tiny_prompt)
    return np.array(logits)


def full_logits(weights, prompt, **kw):
    dec = om.OracleDecoder(weights, **kw)
    c = dec.new_cache()
    return dec.forward([(prompt, c)], logits="all")


def cached_logits(weights, prompt, split, **kw):
    dec = om.OracleDecoder(weights, **kw)
    c = dec.new_cache(capacity=4)  # small capacity also exercises cache growth
    a = dec.forward([(prompt[:split], c)], logits="all")
    b = dec.forward([(prompt[split:], c)], logits="all")
    return np.concatenate([a, b])


def chunked_logits(weights, prompt, chunk):
    dec = om.OracleDecoder(weights)
    c = dec.new_cache()
    parts = [dec.forward([(prompt[i:i + chunk], c)], logits="all") for i in range(0, len(prompt), chunk)]
    return np.concatenate(parts)


def check_numpy_matches_loops(weights, prompt, loop_logits) -> bool:
    return bool(np.max(np.abs(full_logits(weights, prompt) - loop_logits)) <= 1e-12)


def check_full_equals_cached(weights, prompt, split=8) -> bool:
    full = full_logits(weights, prompt)
    return bool(np.max(np.abs(full - cached_logits(weights, prompt, split))) <= 1e-12)


# ---- pins ---------------------------------------------------------------------------------

def test_logit_range_is_tens(tiny_weights, tiny_prompt):
    lg = full_logits(tiny_weights, tiny_prompt)
    rng = np.median(lg.max(axis=1) - lg.min(axis=1))
    assert 10 < rng < 60
    assert np.isfinite(lg).all()


def test_numpy_oracle_matches_loop_oracle(tiny_weights, tiny_prompt, loop_logits):
    assert check_numpy_matches_loops(tiny_weights, tiny_prompt, loop_logits)


def test_full_equals_cached_split_at_half(tiny_weights, tiny_prompt):
    split = WORKLOADS["tiny_f32_t16"].split
    assert split == max(1, len(tiny_prompt) // 2)
    assert check_full_equals_cached(tiny_weights, tiny_prompt, split)


@pytest.mark.parametrize("chunk", [1, 3, 5, 16])
def test_chunked_equals_single_shot(tiny_weights, tiny_prompt, chunk):
    full = full_logits(tiny_weights, tiny_prompt)
    assert np.max(np.abs(full - chunked_logits(tiny_weights, tiny_prompt, chunk))) <= 1e-12


def test_batched_equals_alone(tiny_weights):
    rng = np.random.default_rng(12)
    p1 = rng.integers(0, 512, 9).astype(np.int32)
    p2 = rng.integers(0, 512, 4).astype(np.int32)
    dec = om.OracleDecoder(tiny_weights)
    # sequence 2 already has 3 cached tokens, so the batch mixes a fresh and a cached sequence
    c1, c2 = dec.new_cache(), dec.new_cache()
    dec.forward([(p2[:3], c2)], logits="none")
    both = dec.forward([(p1, c1), (p2[3:], c2)], logits="all")
    a1 = dec.forward([(p1, dec.new_cache())], logits="all")
    c2b = dec.new_cache()
    dec.forward([(p2[:3], c2b)], logits="none")
    a2 = dec.forward([(p2[3:], c2b)], logits="all")
    assert np.max(np.abs(both - np.concatenate([a1, a2]))) <= 1e-12
    last = dec.forward([(p1[:2], dec.new_cache()), (p2, dec.new_cache())], logits="last")
    assert last.shape == (2, 512)


def test_decode_steps_equal_prefill(tiny_weights, tiny_prompt):
    # one token per step, each at its absolute position, equals one prefill
    dec = om.OracleDecoder(tiny_weights)
    c = dec.new_cache()
    steps = np.concatenate([dec.forward([(tiny_prompt[i:i + 1], c)], logits="all")
                            for i in range(len(tiny_prompt))])
    assert np.max(np.abs(steps - full_logits(tiny_weights, tiny_prompt))) <= 1e-12


def test_tied_embedding_is_the_lm_head(tiny_weights, tiny_prompt):
    # zeroing the embedding row of a token absent from the prompt zeroes that
    # token's logit at every position: the LM head is the embedding matrix
    v = next(t for t in range(512) if t not in set(tiny_prompt.tolist()))
    w = make_weights("tiny_f32")
    w.embed = w.embed.copy()
    w.embed[v] = 0.0
    lg = full_logits(w, tiny_prompt)
    assert np.all(lg[:, v] == 0.0)
    assert np.any(full_logits(tiny_weights, tiny_prompt)[:, v] != 0.0)


def test_param_count_of_the_06b_shape():
    (row,) = golden_rows("param_count.txt")
    name, want = row[0].split()
    assert param_count(MODELS["q06b_f32"]) == int(want)
    m = MODELS["q06b_f32"]
    shapes = matrix_shapes(m)
    per_layer = sum(a * b for a, b in shapes.values()) + 2 * m.d_model + 2 * m.head_dim
    assert m.vocab * m.d_model + m.n_layers * per_layer + m.d_model == int(want)
    assert param_count(MODELS["tiny_f32"]) == 156096


def test_greedy_ties_go_to_lowest_id():
    assert om.greedy(np.array([1.0, 3.0, 2.0, 3.0, -1.0])) == 1


def test_f16_kv_diagnostic_mode_stays_within_the_f16_bound(tiny_weights, tiny_prompt):
    a = full_logits(tiny_weights, tiny_prompt)
    b = full_logits(tiny_weights, tiny_prompt, kv_round="f16")
    rng = np.max(a, axis=1) - np.min(a, axis=1)
    assert 0 < np.max(np.abs(a - b)) <= 2e-2 * rng.min()


# ---- planted mistakes ------------------------------------------------------------------------

def _adjacent_pair_rope(x, pos, base):
    D = x.shape[-1]
    th = om.rope_angles(pos, D, base)[:, None, :]
    c, s = np.cos(th), np.sin(th)
    a, b = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = a * c - b * s
    y[..., 1::2] = b * c + a * s
    return y


def _reversed_freq_rope(x, pos, base):
    D = x.shape[-1]
    th = om.rope_angles(pos, D, base)[:, None, ::-1]
    c, s = np.cos(th), np.sin(th)
    x1, x2 = x[..., : D // 2], x[..., D // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def _eps_outside_sqrt(x, g, eps):
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * g


def _silu_on_up(gate, up):
    return om.silu(up) * gate


def _wrong_scale_attention(q, K, V, qpos, tile=256):
    # 1/sqrt(d_model / H) instead of 1/sqrt(head_dim): head_dim 32 -> 16 for the tiny model
    return _orig_attention(q * np.sqrt(2.0), K, V, qpos, tile)


_orig_attention = om.attention


def _q_offset_zero_attention(q, K, V, qpos, tile=256):
    return _orig_attention(q, K, V, qpos - qpos[0], tile)


def _relative_positions(start, n):
    return np.arange(n, dtype=np.int64)


def test_mutant_adjacent_pairing_is_caught(monkeypatch):
    assert not ops.check_rope_pairs_split_halves(_adjacent_pair_rope)


def test_mutant_reversed_frequency_order_is_caught():
    assert not ops.check_rope_angles(_reversed_freq_rope)


def test_mutant_eps_outside_root_is_caught():
    assert not ops.check_rmsnorm_constant_vector(_eps_outside_sqrt)


def test_mutant_silu_on_up_is_caught(tiny_weights, tiny_prompt, loop_logits, monkeypatch):
    assert not ops.check_swiglu_gates_first_argument(_silu_on_up)
    monkeypatch.setattr(om, "swiglu", _silu_on_up)
    assert not check_numpy_matches_loops(tiny_weights, tiny_prompt, loop_logits)


def test_mutant_wrong_attention_scale_is_caught(tiny_weights, tiny_prompt, loop_logits, monkeypatch):
    assert not ops.check_attention_scale(_wrong_scale_attention)
    monkeypatch.setattr(om, "attention", _wrong_scale_attention)
    assert not check_numpy_matches_loops(tiny_weights, tiny_prompt, loop_logits)


def test_mutant_positions_relative_to_the_step_is_caught(tiny_weights, tiny_prompt, monkeypatch):
    monkeypatch.setattr(om, "absolute_positions", _relative_positions)
    assert not check_full_equals_cached(tiny_weights, tiny_prompt)


def test_mutant_q_offset_zero_is_caught(tiny_weights, tiny_prompt, monkeypatch):
    assert not ops.check_attention_causal(_q_offset_zero_attention)
    monkeypatch.setattr(om, "attention", _q_offset_zero_attention)
    assert not check_full_equals_cached(tiny_weights, tiny_prompt)


def test_mutant_k_written_to_v_slab_is_caught(tiny_weights, tiny_prompt, loop_logits, monkeypatch):
    def write_k_twice(self, c, layer, start, k, v):
        n = k.shape[0]
        c.K[layer][start:start + n] = k
        c.V[layer][start:start + n] = k
    monkeypatch.setattr(om.OracleDecoder, "_write_cache", write_k_twice)
    assert not check_numpy_matches_loops(tiny_weights, tiny_prompt, loop_logits)


def test_mutant_skipped_final_norm_is_caught(tiny_weights, tiny_prompt, loop_logits, monkeypatch):
    monkeypatch.setattr(om.OracleDecoder, "_final_hidden", lambda self, x: x * self.final_norm)
    assert not check_numpy_matches_loops(tiny_weights, tiny_prompt, loop_logits)


@pytest.mark.slow
def test_06b_fp32_full_equals_cached():
    wl = WORKLOADS["q06b_f32_t188"]
    w = make_weights(wl.model)
    prompt = make_prompts(wl)[0]
    full = full_logits(w, prompt)
    cached = cached_logits(w, prompt, wl.split)
    assert np.max(np.abs(full - cached)) <= 1e-10
    lr = full.max(axis=1) - full.min(axis=1)
    assert 20 < np.median(lr) < 60
