"""Seeded weights, prompts and context lengths.

Every value is drawn from numpy's PCG64 generator under a fixed seed.
Matrices are drawn N(0, init_std) in float32, one after another in this order:
the embedding, then for each layer W_q, W_k, W_v, W_o, W_gate, W_up, W_down.
Norm gains are constants (1.0 per layer; ``final_gain`` for the final norm) for
``gains="unit"``. For ``gains="random"`` they come from a second stream of
their own (so the matrices are the same either way): per layer attn_norm [d],
q_norm [D], k_norm [D], ffn_norm [d], then the final norm [d], each element
uniform in [0.5, 1.5] (the final norm's times ``final_gain``).

Storage formats of the drawn matrices (all stored [out, in], row-major, the
layout "Candle model runner" section 2.4 gives for the projections):

* ``f32``: the float32 draw itself.
* ``bf16``: the draw rounded to bfloat16 (round to nearest, ties to even),
  kept as uint16 bit patterns.
* ``uint4``: an asymmetric 4-bit code per element with a bfloat16 scale and a
  bfloat16 zero point per group of 32 consecutive input columns, chosen by
  ``quantize_uint4_g32``. The decoder reconstructs W = (q - zp) * scale
  ("Byte-identical: 1,000 tokens of proof", section "The bar we set"); this
  module only chooses the codes and never reconstructs weights.
* ``int4sym``: the symmetric int4 format of "Candle model runner" section 2.5
  with groups of 32 input columns: a signed 4-bit value per element and one
  f16 scale per group, chosen by ``quantize_int4_sym_g32`` (the stored-file
  form the runner loads; the decoder reconstructs W = q * scale).
"""

from __future__ import annotations

import dataclasses
from typing import NamedTuple

import numpy as np

from .configs import ModelShape, Workload, MODELS

GROUP = 32


class Q4(NamedTuple):
    q: np.ndarray  # uint8 [out, in], values 0..15 (one code per element, unpacked)
    scale: np.ndarray  # uint16 [out, in // 32], bfloat16 bit patterns
    zp: np.ndarray  # uint16 [out, in // 32], bfloat16 bit patterns


class Q4S(NamedTuple):
    q: np.ndarray  # int8 [out, in], values -8..7 (one per element, unpacked)
    scale: np.ndarray  # uint16 [out, in // 32], f16 bit patterns


def fp32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits.

    Used only to produce bf16 inputs. NaN and infinity never occur in drawn data.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = (b + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def _bf16_bits_value(bits: np.ndarray) -> np.ndarray:
    # The value a bf16 bit pattern stands for, needed by the code chooser to
    # divide by the scale it stores.
    return (bits.astype(np.uint32) << 16).view(np.float32)


def quantize_uint4_g32(w: np.ndarray) -> Q4:
    """Choose uint4 codes, bf16 scales and bf16 zero points per 32-column group.

    Per group: scale = bf16(max((max - min) / 15, 2**-24)),
    zp = bf16(clamp(-min / scale, 0, 15)), q = clamp(rint(w / scale + zp), 0, 15)
    with rint rounding half to even and ``scale``/``zp`` the stored bf16 values.
    """
    out, inp = w.shape
    assert inp % GROUP == 0
    g = w.reshape(out, inp // GROUP, GROUP).astype(np.float64)
    mn = g.min(axis=-1)
    mx = g.max(axis=-1)
    scale_bits = fp32_to_bf16_bits(np.maximum((mx - mn) / 15.0, 2.0 ** -24).astype(np.float32))
    scale = _bf16_bits_value(scale_bits).astype(np.float64)
    zp_bits = fp32_to_bf16_bits(np.clip(-mn / scale, 0.0, 15.0).astype(np.float32))
    zp = _bf16_bits_value(zp_bits).astype(np.float64)
    q = np.clip(np.rint(g / scale[..., None] + zp[..., None]), 0, 15).astype(np.uint8)
    return Q4(q.reshape(out, inp), scale_bits, zp_bits)


def quantize_int4_sym_g32(w: np.ndarray) -> Q4S:
    """Choose signed int4 values and f16 scales per 32-column group ("Candle model runner" 2.5).

    Per group, in float32 arithmetic: s = f16(max|W| / 7) (round to nearest even),
    q = clamp(rint(W / s), -8, 7) with rint rounding half to even and ``s`` the stored f16
    value. A group of zeros (s = 0, where W / s is undefined) stores q = 0.
    """
    out, inp = w.shape
    assert inp % GROUP == 0
    g = np.ascontiguousarray(w, dtype=np.float32).reshape(out, inp // GROUP, GROUP)
    s16 = (np.abs(g).max(axis=-1) / np.float32(7.0)).astype(np.float16)
    s = s16.astype(np.float32)[..., None]
    safe = np.where(s > 0, s, np.float32(1.0))
    r = np.where(s > 0, np.rint(g / safe), np.float32(0.0))
    q = np.clip(r, -8, 7).astype(np.int8)
    return Q4S(q.reshape(out, inp), s16.view(np.uint16))


MATRIX_NAMES = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")
GAIN_NAMES = ("attn_norm", "q_norm", "k_norm", "ffn_norm")


def matrix_shapes(m: ModelShape) -> dict:
    d, qw, kvw, ff = m.d_model, m.q_width, m.kv_width, m.ff_hidden
    return {
        "wq": (qw, d), "wk": (kvw, d), "wv": (kvw, d), "wo": (d, qw),
        "w_gate": (ff, d), "w_up": (ff, d), "w_down": (d, ff),
    }


@dataclasses.dataclass
class Weights:
    shape: ModelShape
    embed: object  # [V, d] in the model's storage format
    layers: list  # per layer: dict of matrices (storage format) and float32 gains
    final_norm: np.ndarray  # float32 [d]


def _store(m: ModelShape, w: np.ndarray):
    if m.weight_dtype == "f32":
        return w
    if m.weight_dtype == "bf16":
        return fp32_to_bf16_bits(w)
    if m.weight_dtype == "uint4":
        return quantize_uint4_g32(w)
    if m.weight_dtype == "int4sym":
        return quantize_int4_sym_g32(w)
    raise ValueError(m.weight_dtype)


def _draw(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    w = rng.standard_normal(shape, dtype=np.float32)
    w *= np.float32(std)
    return w


def make_weights(m: ModelShape | str, seed: int | None = None) -> Weights:
    """Draw all weights of a model. Deterministic in (shape, seed)."""
    if isinstance(m, str):
        m = MODELS[m]
    rng = np.random.Generator(np.random.PCG64(m.seed if seed is None else seed))
    # The embedding is drawn in row slabs so the uint4 chooser never holds a
    # float64 copy of the whole matrix.
    V, d = m.vocab, m.d_model
    if m.weight_dtype == "uint4":
        parts = []
        step = 16384
        for r0 in range(0, V, step):
            parts.append(quantize_uint4_g32(_draw(rng, (min(step, V - r0), d), m.init_std)))
        embed = Q4(np.concatenate([p.q for p in parts]), np.concatenate([p.scale for p in parts]),
                   np.concatenate([p.zp for p in parts]))
    elif m.weight_dtype == "int4sym":
        step = 16384
        parts = [quantize_int4_sym_g32(_draw(rng, (min(step, V - r0), d), m.init_std)) for r0 in range(0, V, step)]
        embed = Q4S(np.concatenate([p.q for p in parts]), np.concatenate([p.scale for p in parts]))
    else:
        embed = _store(m, _draw(rng, (V, d), m.init_std))
    shapes = matrix_shapes(m)
    layers = []
    for _ in range(m.n_layers):
        layer = {}
        for name in MATRIX_NAMES:
            layer[name] = _store(m, _draw(rng, shapes[name], m.init_std))
        layers.append(layer)
    gain = _gain_source(m, m.seed if seed is None else seed)
    for layer in layers:
        layer["attn_norm"] = gain(d)
        layer["q_norm"] = gain(m.head_dim)
        layer["k_norm"] = gain(m.head_dim)
        layer["ffn_norm"] = gain(d)
    final = (gain(d) * np.float32(m.final_gain)).astype(np.float32)
    return Weights(m, embed, layers, final)


def _gain_source(m: ModelShape, seed: int):
    """Gain vectors in draw order: all ones ("unit") or uniform in [0.5, 1.5] ("random")."""
    if m.gains == "unit":
        return lambda n: np.ones(n, np.float32)
    if m.gains != "random":
        raise ValueError(m.gains)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0x6A1])))
    return lambda n: rng.uniform(0.5, 1.5, size=n).astype(np.float32)


def _streams(wl: Workload):
    ss = np.random.SeedSequence(wl.seed)
    a, b = ss.spawn(2)
    return np.random.Generator(np.random.PCG64(a)), np.random.Generator(np.random.PCG64(b))


def make_context_lengths(wl: Workload) -> np.ndarray:
    """Per-sequence prompt lengths: fixed, or uniform integers in [ctx_lo, ctx_hi]."""
    if wl.prompt_len is not None:
        return np.full(wl.n_seqs, wl.prompt_len, np.int64)
    _, rng = _streams(wl)
    return rng.integers(wl.ctx_lo, wl.ctx_hi + 1, size=wl.n_seqs).astype(np.int64)


def make_prompts(wl: Workload, vocab: int | None = None) -> list:
    """Prompt token ids, uniform in [0, vocab), one int32 array per sequence."""
    if vocab is None:
        vocab = MODELS[wl.model].vocab
    rng, _ = _streams(wl)
    lens = make_context_lengths(wl)
    return [rng.integers(0, vocab, size=int(n)).astype(np.int32) for n in lens]
