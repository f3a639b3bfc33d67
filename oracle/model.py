"""numpy float64 decoder forward pass -- test infrastructure (oracle).

The plain definition of what the GPU library computes, one step at a time,
in float64 on the exactly widened weights. Each step names the passage it
follows:

* embedding: x = E[id], the tied matrix ("Candle model runner" section 2.4,
  last paragraph; "A real model in our own decoder", "Same design..." and the
  tie in ``load_qwen``).
* RMSNorm: h = x / sqrt(mean(x^2) + eps) * w ("Candle model runner" 2.4,
  first equation), eps = rms_norm_eps = 1e-6 ("A real model..." ``qwen_config``).
* projections: q = h Wq^T, k = h Wk^T, v = h Wv^T with W stored [out, in]
  (2.4, first equation and symbol table); Wq is [H*D, d], wider than d
  ("A real model...", switch 1 head_dim).
* q/k norm: an RMSNorm over the D channels of each query head and each key
  head, before RoPE ("A real model...", switch 5 qk_norm). Reading: one gain
  vector of length D per layer for q and one for k, shared by the heads, and
  the same eps.
* RoPE at the absolute position pos(t) = p_s + i (2.4 symbol table), angle
  pos * base^(-2j/D) for pair j ("Byte-identical...", section "The rope table
  that was too accurate"), pairs (j, j + D/2) ("A real model...", section
  "Which channels rotate together": channel 0 with 64). Reading: the rotation
  y_j = x_j cos - x_{j+D/2} sin, y_{j+D/2} = x_{j+D/2} cos + x_j sin.
* the new keys and values are stored by absolute position; the cache holds
  every earlier position of the sequence (2.4, second paragraph).
* attention: o_t = sum_{j <= pos(t)} softmax_j(q_t . k_j / sqrt(D)) v_j over
  the sequence's own keys (2.4, second equation), D the head size. Grouped
  query heads: reading, query head h reads KV head h // (H / H_kv).
* x += o Wo^T; h2 = RMSNorm(x); x += (silu(h2 Wg^T) * (h2 Wu^T)) Wd^T with
  silu(z) = z / (1 + e^-z) on the gate only (2.4, second equation; pitfall
  "silu applied to the up projection").
* final RMSNorm, then logits = h_f E^T with the tied embedding (2.4, last
  paragraph; pitfall "Skipping the final norm"), for every position ("Proving
  it's the same model", section "Every logit, every position") or each
  sequence's last token (2.4).
* greedy choice: argmax with ties to the lowest id ("Candle model runner"
  section 2.6).

Sequences are independent: a batch is processed row by row for the row-wise
steps and sequence by sequence for attention.
"""

from __future__ import annotations

import numpy as np

from .numerics import bf16_to_f32, dequant_int4_sym_g32, dequant_uint4_g32, f16_to_f32, f32_to_f16


def widen_matrix(m, weight_dtype: str) -> np.ndarray:
    """The float64 value of a stored matrix (exact for every storage format)."""
    if weight_dtype == "f32":
        return np.asarray(m, dtype=np.float32).astype(np.float64)
    if weight_dtype == "bf16":
        return bf16_to_f32(m).astype(np.float64)
    if weight_dtype == "uint4":
        return dequant_uint4_g32(m.q, m.scale, m.zp).astype(np.float64)
    if weight_dtype == "int4sym":
        return dequant_int4_sym_g32(m.q, m.scale).astype(np.float64)
    raise ValueError(weight_dtype)


def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def rope_angles(pos: np.ndarray, head_dim: int, base: float) -> np.ndarray:
    j = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * j / head_dim)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]


def rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate [n, heads, D] by the angles of the absolute positions [n]; pairs (j, j + D/2)."""
    D = x.shape[-1]
    th = rope_angles(pos, D, base)[:, None, :]
    c, s = np.cos(th), np.sin(th)
    x1, x2 = x[..., : D // 2], x[..., D // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def qk_norm_rope(q: np.ndarray, k: np.ndarray, g_q: np.ndarray, g_k: np.ndarray, pos: np.ndarray, eps: float,
                 base: float):
    """The q/k step of the Qwen switches (switch 5): each query head [.., H, D] is RMS-normalised
    over its D channels with the gain g_q, each key head with g_k, and only then rotated by RoPE
    at the absolute positions ``pos``."""
    q = rms_norm(q, g_q, eps)
    k = rms_norm(k, g_k, eps)
    return rope(q, pos, base), rope(k, pos, base)


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def swiglu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    return silu(gate) * up


def absolute_positions(start: int, n: int) -> np.ndarray:
    return start + np.arange(n, dtype=np.int64)


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, qpos: np.ndarray,
              tile: int = 256) -> np.ndarray:
    """Causal grouped-query attention of one sequence.

    q: [n, H, D] at absolute positions qpos [n]; K, V: [ctx, H_kv, D] holding
    positions 0..ctx-1. Query t sees keys j <= qpos[t]. Queries are taken in
    tiles of ``tile`` rows only to bound memory.
    """
    n, H, D = q.shape
    Hkv = K.shape[1]
    group = H // Hkv
    scale = 1.0 / np.sqrt(D)
    out = np.empty_like(q)
    keys = np.arange(K.shape[0])
    for h in range(H):
        kvh = h // group
        for t0 in range(0, n, tile):
            t1 = min(n, t0 + tile)
            kend = min(K.shape[0], int(qpos[t0:t1].max()) + 1)  # keys past the tile's last query are never visible
            Kh, Vh = K[:kend, kvh, :], V[:kend, kvh, :]
            s = (q[t0:t1, h, :] @ Kh.T) * scale
            visible = keys[None, :kend] <= qpos[t0:t1, None]
            s = np.where(visible, s, -np.inf)
            s = s - s.max(axis=-1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=-1, keepdims=True)
            out[t0:t1, h, :] = p @ Vh
    return out


class SeqCache:
    """K and V of one sequence, per layer, indexed by absolute position (float64)."""

    def __init__(self, n_layers: int, n_kv_heads: int, head_dim: int, capacity: int = 256):
        self.length = 0
        self.K = [np.zeros((capacity, n_kv_heads, head_dim)) for _ in range(n_layers)]
        self.V = [np.zeros((capacity, n_kv_heads, head_dim)) for _ in range(n_layers)]

    def reserve(self, n: int) -> None:
        cap = self.K[0].shape[0]
        if n <= cap:
            return
        new = max(n, 2 * cap)
        for arrs in (self.K, self.V):
            for i, a in enumerate(arrs):
                b = np.zeros((new,) + a.shape[1:])
                b[:cap] = a
                arrs[i] = b


class OracleDecoder:
    """The decoder with float64 weights widened exactly from the stored formats.

    ``kv_round='f16'`` is a diagnostic mode: keys and values are stored as the
    f16 rounding of their float32 value, the cache format the GPU's f16 pool
    uses, so cache rounding can be told apart from kernel error.
    """

    def __init__(self, weights, kv_round: str | None = None):
        m = weights.shape
        # when a list: forward appends (layer, positions, q, k, v) of every layer, q and k after
        # the q/k norm and RoPE (for the tests' pins of the gains)
        self.trace = None
        self.m = m
        wd = m.weight_dtype
        self.E = widen_matrix(weights.embed, wd)
        self.layers = []
        for lw in weights.layers:
            self.layers.append({
                "attn_norm": lw["attn_norm"].astype(np.float64),
                "ffn_norm": lw["ffn_norm"].astype(np.float64),
                "q_norm": lw["q_norm"].astype(np.float64),
                "k_norm": lw["k_norm"].astype(np.float64),
                "wq": widen_matrix(lw["wq"], wd), "wk": widen_matrix(lw["wk"], wd),
                "wv": widen_matrix(lw["wv"], wd), "wo": widen_matrix(lw["wo"], wd),
                "w_gate": widen_matrix(lw["w_gate"], wd), "w_up": widen_matrix(lw["w_up"], wd),
                "w_down": widen_matrix(lw["w_down"], wd),
            })
        self.final_norm = weights.final_norm.astype(np.float64)
        self.kv_round = kv_round

    def new_cache(self, capacity: int = 256) -> SeqCache:
        return SeqCache(self.m.n_layers, self.m.n_kv_heads, self.m.head_dim, capacity)

    def _store_kv(self, a: np.ndarray) -> np.ndarray:
        if self.kv_round == "f16":
            return f16_to_f32(f32_to_f16(a.astype(np.float32))).astype(np.float64)
        return a

    def forward(self, seqs, logits: str = "all", rows=None) -> np.ndarray:
        """One step over a batch.

        seqs: list of (tokens, cache); each sequence's new tokens start at the
        absolute position cache.length, and the cache is extended in place.
        logits: "all" (every new row, batch order), "last" (each sequence's last
        new row) or "none". ``rows`` (indices into the batch's new rows)
        overrides ``logits``.
        Returns float64 logits [rows, vocab] (or None for "none").
        """
        m = self.m
        H, Hkv, D, eps = m.n_heads, m.n_kv_heads, m.head_dim, m.rms_eps
        tokens = [np.asarray(t, dtype=np.int64) for t, _ in seqs]
        caches = [c for _, c in seqs]
        counts = [len(t) for t in tokens]
        starts = [c.length for c in caches]
        offs = np.cumsum([0] + counts)
        ids = np.concatenate(tokens)
        pos = np.concatenate([absolute_positions(s, n) for s, n in zip(starts, counts)])
        for c, s, n in zip(caches, starts, counts):
            c.reserve(s + n)

        x = self.E[ids]
        for li, L in enumerate(self.layers):
            h = self._attn_input(L, x)
            q = (h @ L["wq"].T).reshape(-1, H, D)
            k = (h @ L["wk"].T).reshape(-1, Hkv, D)
            v = (h @ L["wv"].T).reshape(-1, Hkv, D)
            q, k = qk_norm_rope(q, k, L["q_norm"], L["k_norm"], pos, eps, m.rope_base)
            if self.trace is not None:
                self.trace.append((li, pos.copy(), q.copy(), k.copy(), v.copy()))
            o = np.empty_like(q)
            for si, c in enumerate(caches):
                a, b = offs[si], offs[si + 1]
                s0, n = starts[si], counts[si]
                self._write_cache(c, li, s0, k[a:b], v[a:b])
                o[a:b] = attention(q[a:b], c.K[li][:s0 + n], c.V[li][:s0 + n], pos[a:b])
            x = x + o.reshape(-1, H * D) @ L["wo"].T
            h2 = self._ffn_input(L, x)
            x = x + swiglu(h2 @ L["w_gate"].T, h2 @ L["w_up"].T) @ L["w_down"].T
        for c, s, n in zip(caches, starts, counts):
            c.length = s + n

        if rows is None:
            if logits == "none":
                return None
            rows = np.arange(len(ids)) if logits == "all" else offs[1:] - 1
        return self._final_hidden(x[np.asarray(rows)]) @ self.E.T

    def _write_cache(self, c: SeqCache, layer: int, start: int, k: np.ndarray, v: np.ndarray) -> None:
        n = k.shape[0]
        c.K[layer][start:start + n] = self._store_kv(k)
        c.V[layer][start:start + n] = self._store_kv(v)

    def _attn_input(self, L: dict, x: np.ndarray) -> np.ndarray:
        """The pre-attention RMSNorm, with the layer's attention-norm gain."""
        return rms_norm(x, L["attn_norm"], self.m.rms_eps)

    def _ffn_input(self, L: dict, x: np.ndarray) -> np.ndarray:
        """The post-attention RMSNorm in front of the SwiGLU block, with the layer's FFN-norm gain."""
        return rms_norm(x, L["ffn_norm"], self.m.rms_eps)

    def _final_hidden(self, x: np.ndarray) -> np.ndarray:
        return rms_norm(x, self.final_norm, self.m.rms_eps)


def greedy(logits_row: np.ndarray) -> int:
    """Argmax with ties to the lowest id (np.argmax returns the first maximum)."""
    return int(np.argmax(logits_row))
