"""Pins of the oracle's sampler and generator ("Candle model runner", sections 2.6 and 3)."""

import math

import numpy as np
import pytest

from conftest import golden_rows
from oracle import sampling as sm


def _example():
    (row,) = golden_rows("sampling_example.txt")
    logits = np.array([float(v) for v in row[0].split()], np.float32)
    p = sm.SamplingParams(temperature=float(row[1]), top_k=int(row[2]), top_p=float(row[3]))
    return row, logits, p


def test_worked_example_end_to_end():
    row, logits, p = _example()
    seed = int(row[4])
    assert sm.child_seed(seed, sm.PURPOSE_SAMPLE) == int(row[5], 16)
    assert round(sm.stream(seed).uniform_f64(), 5) == float(row[6])
    tok, lp = sm.sample(logits, p, [], [], sm.stream(seed))
    assert tok == int(row[9])
    assert round(lp, 5) == float(row[10])
    # the logprob is -ln Z with Z = e^-2 + 1 + e^-1 + 1 + e^-4 (section 3)
    assert lp == pytest.approx(-math.log(math.exp(-2) + 1 + math.exp(-1) + 1 + math.exp(-4)), abs=1e-15)


def test_worked_example_kept_sets():
    # top-k 3 keeps {1, 3, 2}; the nucleus keeps {1, 3}; with u below 0.5 the walk stops at id 1
    row, logits, p = _example()
    kept = [int(v) for v in row[7].split()]
    nucleus = [int(v) for v in row[8].split()]

    class Fixed:
        def __init__(self, u):
            self.u = u

        def uniform_f64(self):
            return self.u

    assert sm.sample(logits, p, [], [], Fixed(0.49))[0] == nucleus[0]
    assert sm.sample(logits, p, [], [], Fixed(0.51))[0] == nucleus[1]
    # with top-p off the walk covers all three kept ids in ascending id order: 1, 2, 3
    p3 = sm.SamplingParams(temperature=1.0, top_k=3)
    e = np.exp(np.array([3, 2, 3], np.float64) - 3)
    c = np.cumsum(e / e.sum())
    assert sorted(kept) == [1, 2, 3]
    assert sm.sample(logits, p3, [], [], Fixed(c[0] + 1e-9))[0] == 2
    assert sm.sample(logits, p3, [], [], Fixed(c[1] + 1e-9))[0] == 3


def test_pcg32_reference_outputs():
    # O'Neill's pcg32 demo (seed 42, sequence 54): the generator's published first outputs
    g = sm.Pcg32(42, 54)
    assert [g.next_u32() for _ in range(6)] == [0xA15C02B7, 0x7B47F409, 0xBA1D3330, 0x83D2F293, 0xBFA4784B,
                                               0xCBED606E]


def test_uniform_uses_both_outputs_in_order():
    a_gen, u_gen = sm.Pcg32(7, 3), sm.Pcg32(7, 3)
    a, b = a_gen.next_u32(), a_gen.next_u32()
    assert u_gen.uniform_f64() == ((a >> 5) * 2.0 ** 26 + (b >> 6)) * 2.0 ** -53
    # swapping the two shifts (a pitfall the page lists) gives another number
    assert u_gen.state == a_gen.state and ((b >> 5) * 2.0 ** 26 + (a >> 6)) * 2.0 ** -53 != ((a >> 5) * 2.0 ** 26 + (b >> 6)) * 2.0 ** -53


def test_greedy_takes_no_draw_and_sampling_takes_one():
    logits = np.array([0.5, 2.0, 2.0, -1.0], np.float32)
    g = sm.stream(5)
    before = (g.state, g.inc)
    tok, _ = sm.sample(logits, sm.SamplingParams(temperature=0.0), [], [], g)
    assert tok == 1 and (g.state, g.inc) == before  # ties go to the lowest id
    ref = sm.stream(5)
    ref.uniform_f64()
    sm.sample(logits, sm.SamplingParams(temperature=0.7), [], [], g)
    assert g.state == ref.state


def test_penalties_follow_their_definitions():
    logits = np.array([2.0, -2.0, 1.0, 3.0, 0.0], np.float32)
    p = sm.SamplingParams(repetition_penalty=2.0, presence_penalty=0.5, frequency_penalty=0.25)
    got = sm.penalised(logits, p, prompt=[0, 1, 1], output=[2, 2, 3])
    # prompt-only ids: repetition only (positive divided, negative multiplied)
    assert got[0] == 1.0 and got[1] == -4.0
    # output ids: repetition, then presence + frequency per occurrence
    assert got[2] == 0.5 - (0.25 * 2 + 0.5)
    assert got[3] == 1.5 - (0.25 * 1 + 0.5)
    assert got[4] == 0.0  # untouched
    # presence and frequency never touch prompt-only ids, however often they occur
    q = sm.SamplingParams(presence_penalty=1.0, frequency_penalty=1.0)
    assert np.array_equal(sm.penalised(logits, q, prompt=[0, 0, 0], output=[]), logits.astype(np.float64))


def test_nucleus_keeps_the_crossing_token():
    # four equal logits: every probability is exactly 1/4; top-p 0.5 is reached exactly by the
    # second id of the walk, which is kept, so ids 0 and 1 remain (each 1/2)
    logits = np.zeros(4, np.float32)
    p = sm.SamplingParams(temperature=1.0, top_p=0.5)

    class Fixed:
        def uniform_f64(self):
            return 0.75

    assert sm.sample(logits, p, [], [], Fixed())[0] == 1  # with only id 0 kept this would be 0


def test_walk_is_in_id_order_not_probability_order():
    # probabilities 0.1, 0.6, 0.3 (ids 0, 1, 2); u = 0.65: ascending ids give cumulative
    # 0.1, 0.7 -> id 1; walking by probability (1, 2, 0) would give 0.6, 0.9 -> id 2
    logits = np.log(np.array([0.1, 0.6, 0.3])).astype(np.float32)

    class Fixed:
        def uniform_f64(self):
            return 0.65

    assert sm.sample(logits, sm.SamplingParams(temperature=1.0), [], [], Fixed())[0] == 1


def test_min_p_drops_the_unlikely():
    logits = np.log(np.array([0.5, 0.3, 0.15, 0.05])).astype(np.float32)

    class Fixed:
        def uniform_f64(self):
            return 0.999

    # min-p 0.2: ids with q >= 0.1 stay (0, 1, 2); the last kept id is 2
    assert sm.sample(logits, sm.SamplingParams(temperature=1.0, min_p=0.2), [], [], Fixed())[0] == 2
    assert sm.sample(logits, sm.SamplingParams(temperature=1.0), [], [], Fixed())[0] == 3


def test_seeded_sampling_matches_the_distribution():
    logits = np.log(np.array([0.4, 0.3, 0.2, 0.1])).astype(np.float32)
    p = sm.SamplingParams(temperature=1.0)
    g = sm.stream(2024)
    counts = np.zeros(4)
    for _ in range(4000):
        counts[sm.sample(logits, p, [], [], g)[0]] += 1
    expect = 4000 * np.array([0.4, 0.3, 0.2, 0.1])
    chi2 = float(((counts - expect) ** 2 / expect).sum())
    assert chi2 < 16.27  # 3 degrees of freedom, 0.1% level
    g2 = sm.stream(2024)
    assert [sm.sample(logits, p, [], [], g2)[0] for _ in range(20)] == \
           [sm.sample(logits, p, [], [], g3)[0] for g3 in [sm.stream(2024)] for _ in range(20)]
