"""Seeded token sampling -- test infrastructure (oracle).

Follows "Candle model runner (Llama + bigram, int4), Rust KV cache, sampler and
PCG32", section 2.6 "The sampler and PCG32", step by step, in float64:

1. widen the row's logits to float64;
2. repetition penalty r over the distinct ids of prompt and output: a positive
   logit is divided by r, any other multiplied by r;
3. presence a_p and frequency a_f penalties over the output only: an id that
   occurs c > 0 times in the output loses a_f * c + a_p;
4. the logprob of every id is log softmax of these values (before temperature);
5. temperature 0 is greedy: the largest value, ties to the lowest id, and no
   draw from the generator;
6. otherwise divide by the temperature T; keep the top k by (value descending,
   id ascending) (k = 0 keeps all); keep the nucleus, walking the kept ids in
   that order and stopping after the id whose cumulative probability reaches p
   (p = 1 keeps all); keep the ids whose probability is at least m times the
   largest (m = 0 keeps all); softmax over the kept ids in ascending id order;
   draw one uniform u and return the first id, in ascending id order, whose
   cumulative probability exceeds u.

Every sum is a left-to-right loop over ids in ascending order (the page requires
left-to-right sums; the order of the ids is our reading), except the nucleus
walk, whose order the page fixes. The probabilities of steps 6's top-p and min-p
are over the ids the top-k step kept.

The generator (same section): a request's stream(seed, purpose) is PCG32 seeded
with pcg32_srandom_r(child_seed(seed, purpose), purpose), where
child_seed(s, purpose) = mix64(s + purpose * 0x9E3779B97F4A7C15) and mix64 is the
splitmix64 finaliser (Steele, Lea and Flood, "Fast splittable pseudorandom number
generators", 2014); sampling uses purpose 4. PCG32 is O'Neill's XSH-RR 64/32
generator ("PCG: A family of simple fast space-efficient statistically good
algorithms for random number generation", 2014): state' = state * 6364136223846793005
+ inc, output = rotr32(((state ^ (state >> 18)) >> 27), state >> 59) of the old
state; pcg32_srandom_r sets inc = 2 * seq + 1, steps from state 0, adds the seed,
steps again. One uniform takes two outputs a, b: u = ((a >> 5) * 2^26 + (b >> 6)) * 2^-53.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

M64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15
PURPOSE_SAMPLE = 4


def mix64(z: int) -> int:
    z &= M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def child_seed(seed: int, purpose: int) -> int:
    return mix64((seed + purpose * GOLDEN_GAMMA) & M64)


class Pcg32:
    def __init__(self, initstate: int, initseq: int):
        self.state = 0
        self.inc = ((initseq << 1) | 1) & M64
        self.next_u32()
        self.state = (self.state + initstate) & M64
        self.next_u32()

    def next_u32(self) -> int:
        old = self.state
        self.state = (old * 6364136223846793005 + self.inc) & M64
        xorshifted = (((old >> 18) ^ old) >> 27) & 0xFFFFFFFF
        rot = old >> 59
        return ((xorshifted >> rot) | (xorshifted << ((-rot) & 31))) & 0xFFFFFFFF

    def uniform_f64(self) -> float:
        a = self.next_u32()
        b = self.next_u32()
        return ((a >> 5) * 67108864.0 + (b >> 6)) * (1.0 / 9007199254740992.0)


def stream(seed: int, purpose: int = PURPOSE_SAMPLE) -> Pcg32:
    return Pcg32(child_seed(seed, purpose), purpose)


@dataclasses.dataclass
class SamplingParams:
    temperature: float = 1.0
    top_k: int = 0
    top_p: float = 1.0
    min_p: float = 0.0
    repetition_penalty: float = 1.0
    presence_penalty: float = 0.0
    frequency_penalty: float = 0.0


def _lr_sum(x: np.ndarray) -> float:
    """Left-to-right float64 sum (numpy's cumulative sum adds in order)."""
    return float(np.cumsum(x, dtype=np.float64)[-1]) if x.size else 0.0


def penalised(logits, p: SamplingParams, prompt, output) -> np.ndarray:
    """Steps 1-3: the float64 values after the penalties."""
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    V = l.shape[0]
    seen = sorted({int(v) for v in list(prompt) + list(output) if 0 <= int(v) < V})
    for v in seen:
        l[v] = l[v] / p.repetition_penalty if l[v] > 0 else l[v] * p.repetition_penalty
    counts = {}
    for v in output:
        v = int(v)
        if 0 <= v < V:
            counts[v] = counts.get(v, 0) + 1
    for v in sorted(counts):
        l[v] -= p.frequency_penalty * counts[v] + p.presence_penalty
    return l


def sample(logits, p: SamplingParams, prompt, output, rng: Pcg32) -> tuple:
    """(token id, float64 logprob) for one row, advancing ``rng`` by one uniform unless greedy."""
    l = penalised(logits, p, prompt, output)
    V = l.shape[0]
    M = float(l.max())
    Z = _lr_sum(np.exp(l - M))
    logprob = (l - M) - math.log(Z)
    if p.temperature == 0:
        tok = int(np.argmax(l))  # first maximum: the lowest id
        return tok, float(logprob[tok])
    lt = l / p.temperature
    ids = np.arange(V)
    order = np.lexsort((ids, -lt))  # value descending, then id ascending
    kept = order[:p.top_k] if 0 < p.top_k < V else order
    kept_asc = np.sort(kept)
    mt = float(lt[order[0]])
    e = np.exp(lt - mt)
    Zk = _lr_sum(e[kept_asc])
    q = e / Zk
    keep = np.zeros(V, dtype=bool)
    if p.top_p < 1.0:
        c = 0.0
        for i in kept:
            c += q[i]
            keep[i] = True
            if c >= p.top_p:
                break
    else:
        keep[kept] = True
    if p.min_p > 0.0:
        qmax = q[order[0]]
        keep &= q >= p.min_p * qmax
    final = ids[keep]  # ascending
    Zf = _lr_sum(e[final])
    u = rng.uniform_f64()
    c = 0.0
    tok = int(final[-1])
    for i in final:
        c += e[i] / Zf
        if u < c:
            tok = int(i)
            break
    return tok, float(logprob[tok])
