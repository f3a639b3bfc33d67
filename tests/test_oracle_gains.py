"""Pins of where the oracles apply the five norm gains (CPU only).

The decoder has five gain vectors: the attention norm and the FFN norm of each layer
("Candle model runner" 2.4, RMSNorm equation: the normalised vector times w), the per-head
q and k norms applied before RoPE ("A real model in our own decoder", switch 5 qk_norm), and
the final norm in front of the tied LM head. With every gain at 1.0 a gain dropped, swapped
or applied after the rotation changes nothing, so these pins use non-unit gains and check
each placement against facts that do not repeat the oracle's formulas:

* Folding: RMSNorm(x) * g . W^T = RMSNorm(x) . (W diag g)^T. A model whose attention-norm
  gain is g equals, up to rounding, the model with gain 1 whose W_q, W_k, W_v columns are
  scaled by g; the same for the FFN-norm gain and W_gate, W_up. With gains that are powers of
  two both sides round identically.
* The final gain of channel c multiplies channel c of the normalised state only: doubling it
  adds to every logit row a multiple of column c of the tied embedding.
* The q/k step on a head whose channels are all equal returns exactly its gain at position 0
  (RoPE is the identity there, and a constant vector normalises to ones), and at any position
  each rotated pair keeps the length of its gain pair (a rotation keeps lengths). A rotation
  applied before the gains breaks the second fact whenever the gains of a pair differ.
* In the decoder, q / g_q and k / g_k at position 0 have unit RMS (the normalised head),
  for the gains read from the q_norm and k_norm entries.
* Both oracles (numpy float64 and the loop-only decoder) agree with random gains.

Mistakes planted one at a time in the numpy oracle (rotation before the norm, q and k gains
exchanged, attention and FFN gains exchanged, each gain dropped) are each caught.
"""

import dataclasses

import numpy as np
import pytest

import oracle.loops as ol
import oracle.model as om
from oracle.loops import LoopDecoder
from synthetic import MODELS, WORKLOADS, make_prompts, make_weights

TINY = dataclasses.replace(MODELS["tiny_f32"], gains="random")


@pytest.fixture(scope="module")
def gw():
    return make_weights(TINY)


@pytest.fixture(scope="module")
def prompt():
    return make_prompts(WORKLOADS["tiny_f32_t16"])[0]


def numpy_logits(w, prompt):
    dec = om.OracleDecoder(w)
    return dec.forward([(prompt, dec.new_cache())], logits="all")


def loop_logits(w, prompt):
    return np.array(LoopDecoder(w).run(prompt)[0])


FORWARDS = {"numpy": numpy_logits, "loops": loop_logits}


def pow2_gains(n, seed):
    """Gains in {1/4, 1/2, 2, 4}: scaling by them is exact in float32 and float64."""
    return np.random.default_rng(seed).choice(np.float32([0.25, 0.5, 2.0, 4.0]), size=n)


def copy_weights(w):
    return dataclasses.replace(w, layers=[{k: v.copy() for k, v in L.items()} for L in w.layers],
                               final_norm=w.final_norm.copy())


# ---- the checks (each returns True / False so that the mutant tests can use them) -----------

def check_attn_gain_folds(forward, w, prompt) -> bool:
    a, b = copy_weights(w), copy_weights(w)
    for li in range(len(w.layers)):
        g = pow2_gains(w.shape.d_model, 10 + li)
        a.layers[li]["attn_norm"] = g
        b.layers[li]["attn_norm"] = np.ones_like(g)
        for name in ("wq", "wk", "wv"):
            b.layers[li][name] = (b.layers[li][name] * g[None, :]).astype(np.float32)
    la, lb = forward(a, prompt), forward(b, prompt)
    return bool(np.max(np.abs(la - lb)) <= 1e-12 * np.max(np.abs(la)))


def check_ffn_gain_folds(forward, w, prompt) -> bool:
    a, b = copy_weights(w), copy_weights(w)
    for li in range(len(w.layers)):
        g = pow2_gains(w.shape.d_model, 20 + li)
        a.layers[li]["ffn_norm"] = g
        b.layers[li]["ffn_norm"] = np.ones_like(g)
        for name in ("w_gate", "w_up"):
            b.layers[li][name] = (b.layers[li][name] * g[None, :]).astype(np.float32)
    la, lb = forward(a, prompt), forward(b, prompt)
    return bool(np.max(np.abs(la - lb)) <= 1e-12 * np.max(np.abs(la)))


def check_final_gain_channel(forward, w, prompt, c=5) -> bool:
    base = forward(w, prompt)
    w2 = copy_weights(w)
    w2.final_norm[c] *= np.float32(2.0)
    diff = forward(w2, prompt) - base
    col = w.embed[:, c].astype(np.float64)
    alpha = diff @ col / (col @ col)
    resid = np.max(np.abs(diff - alpha[:, None] * col[None, :]))
    return bool(np.all(np.abs(alpha) > 1e-6) and resid <= 1e-10 * np.max(np.abs(diff)))


def _const_heads(n_pos, heads, D, seed):
    rng = np.random.default_rng(seed)
    c = rng.uniform(1.0, 3.0, size=(n_pos, heads)) * rng.choice([-1.0, 1.0], size=(n_pos, heads))
    return np.repeat(c[:, :, None], D, axis=2)


def check_qk_step(step, D=32, eps=1e-6, base=1e6) -> bool:
    """step(q [n,H,D], k [n,Hkv,D], g_q, g_k, pos) -> (q', k')."""
    rng = np.random.default_rng(3)
    gq, gk = rng.uniform(0.5, 1.5, D), rng.uniform(0.5, 1.5, D)
    pos = np.array([0, 5, 300, 7777])
    q, k = _const_heads(4, 4, D, 1), _const_heads(4, 2, D, 2)
    q2, k2 = step(q, k, gq, gk, pos)
    ok = True
    for x, y, g in ((q, q2, gq), (k, k2, gk)):
        sign = np.sign(x[:, :, :1])
        # position 0: the gain itself (eps shifts it by at most eps / 2 relative)
        ok &= np.allclose(y[0], sign[0] * g[None, :], rtol=1e-6, atol=0)
        # every position: each pair (j, j + D/2) has the length of the gain pair
        h = D // 2
        ylen = np.hypot(y[..., :h], y[..., h:])
        glen = np.hypot(g[:h], g[h:])
        ok &= np.allclose(ylen, np.broadcast_to(glen, ylen.shape), rtol=1e-6, atol=0)
    return bool(ok)


def numpy_qk_step(q, k, gq, gk, pos):
    return om.qk_norm_rope(q, k, gq, gk, pos, 1e-6, 1e6)


def loop_qk_step(q, k, gq, gk, pos):
    def heads(x, g):
        return np.array([[ol._qk_head(list(x[t, h]), list(g), int(pos[t]), 1e-6, 1e6) for h in range(x.shape[1])]
                         for t in range(x.shape[0])])
    return heads(q, gq), heads(k, gk)


def check_trace_unit_rms(trace_rows, w) -> bool:
    """(layer, q heads at position 0, k heads at position 0) -> q / g_q and k / g_k have RMS 1."""
    ok = True
    for li, q0, k0 in trace_rows:
        L = w.layers[li]
        for heads, g in ((q0, L["q_norm"]), (k0, L["k_norm"])):
            r = np.sqrt(np.mean((np.asarray(heads) / g.astype(np.float64)) ** 2, axis=-1))
            ok &= bool(np.all(np.abs(r - 1.0) <= 1e-4))
    return bool(ok)


def numpy_trace_rows(w, prompt):
    dec = om.OracleDecoder(w)
    dec.trace = []
    dec.forward([(prompt, dec.new_cache())], logits="none")
    return [(li, q[0], k[0]) for li, pos, q, k, v in dec.trace if pos[0] == 0]


def loop_trace_rows(w, prompt):
    tr = []
    LoopDecoder(w).run(prompt[:1], trace=tr)
    return [(li, qs, ks) for li, pos, qs, ks, vs in tr if pos == 0]


# ---- pins ------------------------------------------------------------------------------------

def test_generated_gains_are_distinct_and_not_one(gw):
    L = gw.layers[0]
    for name in ("attn_norm", "ffn_norm", "q_norm", "k_norm"):
        assert np.all((L[name] >= 0.5) & (L[name] <= 1.5)) and np.std(L[name]) > 0.1, name
    assert not np.array_equal(L["q_norm"], L["k_norm"])
    assert not np.array_equal(L["attn_norm"], L["ffn_norm"])
    assert not np.array_equal(gw.layers[0]["q_norm"], gw.layers[1]["q_norm"])
    unit = make_weights("tiny_f32")  # the configuration's own gains: 1.0, and the matrices are the same
    assert np.all(unit.layers[1]["k_norm"] == 1.0)
    assert np.array_equal(unit.layers[1]["w_up"], gw.layers[1]["w_up"])


@pytest.mark.parametrize("impl", list(FORWARDS))
def test_attention_gain_folds_into_qkv_columns(gw, prompt, impl):
    assert check_attn_gain_folds(FORWARDS[impl], gw, prompt)


@pytest.mark.parametrize("impl", list(FORWARDS))
def test_ffn_gain_folds_into_gate_and_up_columns(gw, prompt, impl):
    assert check_ffn_gain_folds(FORWARDS[impl], gw, prompt)


@pytest.mark.parametrize("impl", list(FORWARDS))
def test_final_gain_scales_its_own_channel_of_the_lm_head(gw, prompt, impl):
    assert check_final_gain_channel(FORWARDS[impl], gw, prompt)


@pytest.mark.parametrize("step", [numpy_qk_step, loop_qk_step])
def test_qk_step_norms_with_gain_then_rotates(step):
    assert check_qk_step(step)


def test_decoder_q_and_k_heads_carry_their_own_gains(gw, prompt):
    assert check_trace_unit_rms(numpy_trace_rows(gw, prompt), gw)
    assert check_trace_unit_rms(loop_trace_rows(gw, prompt), gw)
    # exchanging the two gains in the check itself fails it: the pin can tell q from k
    swapped = copy_weights(gw)
    for L in swapped.layers:
        L["q_norm"], L["k_norm"] = L["k_norm"], L["q_norm"]
    assert not check_trace_unit_rms(numpy_trace_rows(gw, prompt), swapped)


def test_numpy_oracle_matches_loop_oracle_with_random_gains(gw, prompt):
    assert np.max(np.abs(numpy_logits(gw, prompt) - loop_logits(gw, prompt))) <= 1e-12


# ---- planted mistakes --------------------------------------------------------------------------

_orig_qk = om.qk_norm_rope


def _rope_then_norm(q, k, gq, gk, pos, eps, base):
    return om.rms_norm(om.rope(q, pos, base), gq, eps), om.rms_norm(om.rope(k, pos, base), gk, eps)


def _qk_gains_exchanged(q, k, gq, gk, pos, eps, base):
    return _orig_qk(q, k, gk, gq, pos, eps, base)


def _q_gain_dropped(q, k, gq, gk, pos, eps, base):
    return _orig_qk(q, k, np.ones_like(gq), gk, pos, eps, base)


def _k_gain_dropped(q, k, gq, gk, pos, eps, base):
    return _orig_qk(q, k, gq, np.ones_like(gk), pos, eps, base)


def test_mutant_rope_before_qk_norm_is_caught(gw, prompt, monkeypatch):
    monkeypatch.setattr(om, "qk_norm_rope", _rope_then_norm)
    assert not check_qk_step(numpy_qk_step)
    assert np.max(np.abs(numpy_logits(gw, prompt) - loop_logits(gw, prompt))) > 1e-6


@pytest.mark.parametrize("mutant", [_qk_gains_exchanged, _q_gain_dropped, _k_gain_dropped])
def test_mutant_qk_gain_misplaced_is_caught(gw, prompt, monkeypatch, mutant):
    monkeypatch.setattr(om, "qk_norm_rope", mutant)
    assert not check_qk_step(numpy_qk_step)
    assert not check_trace_unit_rms(numpy_trace_rows(gw, prompt), gw)
    assert np.max(np.abs(numpy_logits(gw, prompt) - loop_logits(gw, prompt))) > 1e-6


def test_mutant_attention_and_ffn_gains_exchanged_is_caught(gw, prompt, monkeypatch):
    monkeypatch.setattr(om.OracleDecoder, "_attn_input",
                        lambda self, L, x: om.rms_norm(x, L["ffn_norm"], self.m.rms_eps))
    monkeypatch.setattr(om.OracleDecoder, "_ffn_input",
                        lambda self, L, x: om.rms_norm(x, L["attn_norm"], self.m.rms_eps))
    assert not check_attn_gain_folds(numpy_logits, gw, prompt)
    assert not check_ffn_gain_folds(numpy_logits, gw, prompt)


def test_mutant_attention_gain_dropped_is_caught(gw, prompt, monkeypatch):
    monkeypatch.setattr(om.OracleDecoder, "_attn_input",
                        lambda self, L, x: om.rms_norm(x, np.ones_like(L["attn_norm"]), self.m.rms_eps))
    assert not check_attn_gain_folds(numpy_logits, gw, prompt)


def test_mutant_ffn_gain_dropped_is_caught(gw, prompt, monkeypatch):
    monkeypatch.setattr(om.OracleDecoder, "_ffn_input",
                        lambda self, L, x: om.rms_norm(x, np.ones_like(L["ffn_norm"]), self.m.rms_eps))
    assert not check_ffn_gain_folds(numpy_logits, gw, prompt)


@pytest.mark.parametrize("kind", ["dropped", "reversed"])
def test_mutant_final_gain_misplaced_is_caught(gw, prompt, monkeypatch, kind):
    if kind == "dropped":
        f = lambda self, x: om.rms_norm(x, np.ones_like(self.final_norm), self.m.rms_eps)  # noqa: E731
    else:
        f = lambda self, x: om.rms_norm(x, self.final_norm[::-1], self.m.rms_eps)  # noqa: E731
    monkeypatch.setattr(om.OracleDecoder, "_final_hidden", f)
    assert not check_final_gain_channel(numpy_logits, gw, prompt)
