"""Model shapes and workloads.

Shapes: the Qwen3-0.6B layout (28 layers, width 1,024, 16 query heads of
128 channels, 8 key/value heads, feed-forward width 3,072, vocabulary
151,936, tied embedding, RMSNorm epsilon 1e-6, RoPE base 1e6, split-halves
pairing, per-head q/k RMSNorm) as described on "A real model in our own
decoder" (section "Same design, bigger numbers, five switches", and the
``qwen_config`` whitelist), and a two-layer tiny decoder with the same
switches. The parameter count of the 0.6B shape is 596,049,920, the figure
printed on "Proving it's the same model" (opening paragraph) and "A real
model in our own decoder" (section "Everything arrives, nothing extra").

The final-norm gain ``final_gain`` scales the logits so that their range per
position is a few tens, the size "Proving it's the same model" reports for the
real checkpoint (section "Pick the tolerance before looking": median 29 and
42). Every matrix is drawn N(0, 0.02). The logit standard deviation is
final_gain * 0.02 * sqrt(d_model); the gain is chosen so that it equals 4.

Norm gains (``gains``): "unit" sets every per-layer gain to 1.0 and the final
gain to ``final_gain`` on every channel, as the two-layer configuration states;
"random" draws each gain vector per channel, uniform in [0.5, 1.5] (the final
one times ``final_gain``), so that a gain applied to the wrong tensor, to the
wrong channel or not at all changes the result. The 0.6B configurations leave
the gains open; they take "random", as a trained checkpoint's gains are not 1.
"""

from __future__ import annotations

import dataclasses
import math


@dataclasses.dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ff_hidden: int
    vocab: int
    rms_eps: float = 1e-6
    rope_base: float = 1e6
    weight_dtype: str = "f32"  # "f32" | "bf16" | "uint4" | "int4sym"
    kv_dtype: str = "f32"  # "f32" | "f16"
    block_tokens: int = 16
    init_std: float = 0.02
    final_gain: float = 1.0
    seed: int = 0
    gains: str = "unit"  # "unit" | "random" (per-channel gains, uniform in [0.5, 1.5])

    @property
    def q_width(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_width(self) -> int:
        return self.n_kv_heads * self.head_dim


def _logit_gain(d_model: int, std: float = 0.02, target_sigma: float = 4.0) -> float:
    return target_sigma / (std * math.sqrt(d_model))


_TINY = dict(n_layers=2, d_model=64, n_heads=4, n_kv_heads=2, head_dim=32, ff_hidden=192, vocab=512)
_Q06B = dict(n_layers=28, d_model=1024, n_heads=16, n_kv_heads=8, head_dim=128, ff_hidden=3072, vocab=151936)

MODELS = {
    "tiny_f32": ModelShape(name="tiny_f32", **_TINY, weight_dtype="f32", kv_dtype="f32",
                           final_gain=_logit_gain(64), seed=101),
    "q06b_f32": ModelShape(name="q06b_f32", **_Q06B, weight_dtype="f32", kv_dtype="f32",
                           final_gain=_logit_gain(1024), seed=202, gains="random"),
    "q06b_bf16": ModelShape(name="q06b_bf16", **_Q06B, weight_dtype="bf16", kv_dtype="f16",
                            final_gain=_logit_gain(1024), seed=303, gains="random"),
    "q06b_uint4": ModelShape(name="q06b_uint4", **_Q06B, weight_dtype="uint4", kv_dtype="f16",
                             final_gain=_logit_gain(1024), seed=505, gains="random"),
    "q06b_int4sym": ModelShape(name="q06b_int4sym", **_Q06B, weight_dtype="int4sym", kv_dtype="f16",
                               final_gain=_logit_gain(1024), seed=606, gains="random"),
}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    model: str
    n_seqs: int
    prompt_len: int | None  # fixed prompt length, or None for ragged contexts
    split: int | None = None  # cached-path split point (full vs cached)
    chunk: int | None = None  # chunked prefill chunk length
    decode_steps: int = 0
    ctx_lo: int | None = None  # ragged context lengths, inclusive bounds
    ctx_hi: int | None = None
    seed: int = 0


WORKLOADS = {
    # Two-layer fp32 decoder; 16 prompt tokens; full path vs cached path split at 8.
    "tiny_f32_t16": Workload("tiny_f32_t16", "tiny_f32", n_seqs=1, prompt_len=16, split=8, seed=11),
    # 0.6B-shaped fp32; 188 prompt tokens; full vs cached split at 94.
    "q06b_f32_t188": Workload("q06b_f32_t188", "q06b_f32", n_seqs=1, prompt_len=188, split=94, seed=22),
    # 0.6B bf16 weights, f16 KV; 32 x 1024 prefill then 256 greedy decode steps.
    "q06b_bf16_b32_p1024_d256": Workload("q06b_bf16_b32_p1024_d256", "q06b_bf16", n_seqs=32,
                                         prompt_len=1024, decode_steps=256, seed=33),
    # 0.6B bf16, 8 x 2048 prompts run in 512-token chunks vs one shot.
    "q06b_bf16_b8_p2048_c512": Workload("q06b_bf16_b8_p2048_c512", "q06b_bf16", n_seqs=8,
                                        prompt_len=2048, chunk=512, seed=44),
    # 0.6B uint4-g32 weights, f16 KV; batch 64 decode, contexts uniform in [512, 8192], 128 steps.
    "q06b_uint4_b64_ragged_d128": Workload("q06b_uint4_b64_ragged_d128", "q06b_uint4", n_seqs=64,
                                           prompt_len=None, decode_steps=128, ctx_lo=512,
                                           ctx_hi=8192, seed=55),
    # 0.6B symmetric int4-g32 weights, f16 KV; 16 x 1024 prefill (every projection on the large
    # tile product), then 32 greedy decode steps at batch 16.
    "q06b_int4sym_b16_p1024_d32": Workload("q06b_int4sym_b16_p1024_d32", "q06b_int4sym", n_seqs=16,
                                           prompt_len=1024, decode_steps=32, seed=66),
    # The headline prefill + decode shape (32 x 1024, 256 greedy steps) with symmetric int4-g32
    # weights: a benchmark workload for the 4-bit path.
    "q06b_int4sym_b32_p1024_d256": Workload("q06b_int4sym_b32_p1024_d256", "q06b_int4sym", n_seqs=32,
                                            prompt_len=1024, decode_steps=256, seed=33),
    # The same format on the ragged batch-64 decode workload of the uint4 weights.
    "q06b_int4sym_b64_ragged_d128": Workload("q06b_int4sym_b64_ragged_d128", "q06b_int4sym", n_seqs=64,
                                             prompt_len=None, decode_steps=128, ctx_lo=512,
                                             ctx_hi=8192, seed=55),
}


def param_count(m: ModelShape) -> int:
    """Unique parameters of the decoder: tied embedding, per-layer norms, projections, final norm."""
    d, qw, kvw, ff, D = m.d_model, m.q_width, m.kv_width, m.ff_hidden, m.head_dim
    per_layer = (d + qw * d + 2 * kvw * d + 2 * D + d * qw + d + 3 * ff * d)
    return m.vocab * d + m.n_layers * per_layer + d
