"""Loop-only decoder for tiny shapes -- test infrastructure (oracle).

A second oracle written with Python floats and explicit loops, sharing no
helper with ``oracle.model``. It walks the prompt one token at a time,
each token attending to the keys stored for every position up to its own, so
it also checks that the batched formulation in ``oracle.model`` (all prompt
rows at once with a causal mask) is the same function. Same passages as
``oracle.model``: "Candle model runner" section 2.4 (RMSNorm, projections,
RoPE at pos(t), cache by position, attention, residuals, SwiGLU, final norm,
tied LM head), "A real model in our own decoder" (rectangular Q/O, q/k norm
before RoPE, split-halves pairing), "Byte-identical..." (RoPE angle).

Only float32-stored weights (the tiny model) are accepted.
"""

from __future__ import annotations

import math


def _vec(a):
    return [float(v) for v in a]


def _mat(a):
    return [[float(v) for v in row] for row in a]


def _matvec(W, x):
    # y_o = sum_i W[o][i] x[i]  (W stored [out, in])
    out = []
    for row in W:
        acc = 0.0
        for wi, xi in zip(row, x):
            acc += wi * xi
        out.append(acc)
    return out


def _rmsnorm(x, g, eps):
    ss = 0.0
    for v in x:
        ss += v * v
    r = 1.0 / math.sqrt(ss / len(x) + eps)
    return [v * r * gi for v, gi in zip(x, g)]


def _rotate(vec, pos, base):
    D = len(vec)
    half = D // 2
    out = list(vec)
    for j in range(half):
        ang = pos * math.pow(base, -2.0 * j / D)
        c, s = math.cos(ang), math.sin(ang)
        a, b = vec[j], vec[j + half]
        out[j] = a * c - b * s
        out[j + half] = b * c + a * s
    return out


def _qk_head(vec, g, pos, eps, base):
    # one query or key head: RMSNorm over its channels with its gain, then the rotation
    return _rotate(_rmsnorm(vec, g, eps), pos, base)


class LoopDecoder:
    def __init__(self, weights):
        m = weights.shape
        assert m.weight_dtype == "f32", "loop oracle takes float32 weights only"
        self.m = m
        self.E = _mat(weights.embed)
        self.L = []
        for lw in weights.layers:
            self.L.append({k: (_mat(v) if getattr(v, "ndim", 1) == 2 else _vec(v)) for k, v in lw.items()})
        self.gf = _vec(weights.final_norm)

    def new_cache(self):
        # per layer: dict position -> (k heads, v heads)
        return [dict() for _ in range(self.m.n_layers)]

    def step(self, token: int, pos: int, cache, trace=None):
        """One token at absolute position ``pos``; returns its logits (list). ``trace`` (a list, or
        None) receives (layer, pos, q heads, k heads, v heads) of every layer, q and k after the
        q/k norm and the rotation."""
        m = self.m
        H, Hkv, D, eps = m.n_heads, m.n_kv_heads, m.head_dim, m.rms_eps
        x = list(self.E[token])
        for li, L in enumerate(self.L):
            h = _rmsnorm(x, L["attn_norm"], eps)
            qf = _matvec(L["wq"], h)
            kf = _matvec(L["wk"], h)
            vf = _matvec(L["wv"], h)
            qs = [_qk_head(qf[i * D:(i + 1) * D], L["q_norm"], pos, eps, m.rope_base) for i in range(H)]
            ks = [_qk_head(kf[i * D:(i + 1) * D], L["k_norm"], pos, eps, m.rope_base) for i in range(Hkv)]
            vs = [vf[i * D:(i + 1) * D] for i in range(Hkv)]
            if trace is not None:
                trace.append((li, pos, qs, ks, vs))
            cache[li][pos] = (ks, vs)
            o = []
            for hq in range(H):
                kvh = hq * Hkv // H
                scores = []
                for j in range(pos + 1):
                    kj = cache[li][j][0][kvh]
                    dot = 0.0
                    for a, b in zip(qs[hq], kj):
                        dot += a * b
                    scores.append(dot / math.sqrt(D))
                mx = max(scores)
                w = [math.exp(s - mx) for s in scores]
                tot = sum(w)
                acc = [0.0] * D
                for j in range(pos + 1):
                    vj = cache[li][j][1][kvh]
                    p = w[j] / tot
                    for c in range(D):
                        acc[c] += p * vj[c]
                o.extend(acc)
            att = _matvec(L["wo"], o)
            x = [a + b for a, b in zip(x, att)]
            h2 = _rmsnorm(x, L["ffn_norm"], eps)
            g = _matvec(L["w_gate"], h2)
            u = _matvec(L["w_up"], h2)
            a = [(gi / (1.0 + math.exp(-gi))) * ui for gi, ui in zip(g, u)]
            dn = _matvec(L["w_down"], a)
            x = [p + q for p, q in zip(x, dn)]
        xf = _rmsnorm(x, self.gf, eps)
        return _matvec(self.E, xf)

    def run(self, tokens, start: int = 0, cache=None, trace=None):
        """Logits of every token of ``tokens`` placed at positions start, start+1, ..."""
        if cache is None:
            cache = self.new_cache()
        return [self.step(int(t), start + i, cache, trace) for i, t in enumerate(tokens)], cache
