"""GPU parity of the seeded sampler (dec_sample) against the oracle's sampler ("Candle model
runner" section 2.6; worked example of section 3).

Each case runs rows of logits through dec_sample and the same rows through
oracle.sampling.sample with the same parameters, histories and streams. The chosen ids must be
equal, the generator states after the call equal (one uniform per sampled row, none for greedy),
and the float64 logprobs equal within 1e-9 (the device's sums over the vocabulary add in fixed
blocks; the oracle adds left to right). Cases: the page's worked example; greedy with penalties;
temperature alone over the whole vocabulary; top-k alone; top-k with the nucleus and min-p;
min-p alone; equal logits across the top-k cut (lowest ids first); several steps of one stream
with a growing history; the refusals.
"""

import dataclasses

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from gpu_util import report
from oracle import sampling as sm
from synthetic import MODELS, make_weights

V_SMALL = 512
V_FULL = 151936


def _session(vocab):
    from decoder_forward_pass_amd.session import Session
    shape = dataclasses.replace(MODELS["tiny_f32"], name=f"tiny_v{vocab}", vocab=vocab)
    return Session(shape, make_weights(shape), max_context=64, n_blocks=8, max_rows=64, max_seqs=16)


@pytest.fixture(scope="module")
def small():
    s = _session(V_SMALL)
    yield s
    s.close()


@pytest.fixture(scope="module")
def full():
    s = _session(V_FULL)
    yield s
    s.close()


def _params(**kw):
    from decoder_forward_pass_amd import binding as B
    p = sm.SamplingParams(**kw)
    c = B.dec_sampling()
    c.temperature, c.top_p, c.min_p = p.temperature, p.top_p, p.min_p
    c.repetition_penalty, c.presence_penalty, c.frequency_penalty = (p.repetition_penalty, p.presence_penalty,
                                                                      p.frequency_penalty)
    c.top_k = p.top_k
    return p, c


def _run(sess, logits, cases, seeds):
    """cases: list of (SamplingParams kwargs, prompt ids, output ids); returns per-row results."""
    from decoder_forward_pass_amd import binding as B
    n = len(cases)
    ids, hist, params, oparams = [], [], [], []
    for kw, prompt, output in cases:
        h = B.dec_history()
        h.prompt_offset, h.prompt_len = len(ids), len(prompt)
        ids.extend(prompt)
        h.output_offset, h.output_len = len(ids), len(output)
        ids.extend(output)
        hist.append(h)
        op, cp = _params(**kw)
        oparams.append(op)
        params.append(cp)
    rng = torch.tensor([list(B.dec_rng_stream(sd)) for sd in seeds], dtype=torch.uint64, device="cuda")
    dids = torch.tensor(ids, dtype=torch.int32, device="cuda") if ids else None
    lg = torch.tensor(logits, dtype=torch.float32, device="cuda")
    nxt, lp = sess.sample(lg, params, hist, dids, rng)
    torch.cuda.synchronize()
    got_ids, got_lp, got_rng = nxt.cpu().numpy(), lp.cpu().numpy(), rng.cpu().numpy().astype(object)
    out = []
    for i, (kw, prompt, output) in enumerate(cases):
        g = sm.stream(seeds[i])
        tok, lpv = sm.sample(logits[i], oparams[i], prompt, output, g)
        out.append(dict(case=kw, gpu=int(got_ids[i]), oracle=tok, lp_gpu=float(got_lp[i]), lp_oracle=lpv,
                        state_gpu=int(got_rng[i][0]) & (2 ** 64 - 1), state_oracle=g.state))
    return out


def _check(rows, name):
    worst = max(abs(r["lp_gpu"] - r["lp_oracle"]) for r in rows)
    ok = all(r["gpu"] == r["oracle"] and r["state_gpu"] == r["state_oracle"] for r in rows) and worst <= 1e-9
    report({"type": "sampling_parity", "case": name, "rows": len(rows), "ids_equal": sum(r["gpu"] == r["oracle"] for r in rows),
            "states_equal": sum(r["state_gpu"] == r["state_oracle"] for r in rows), "max_logprob_error": worst,
            "pass": ok})
    for r in rows:
        assert r["gpu"] == r["oracle"], r
        assert r["state_gpu"] == r["state_oracle"], r
        assert abs(r["lp_gpu"] - r["lp_oracle"]) <= 1e-9, r


def test_worked_example(small):
    row = np.full(V_SMALL, -np.inf, np.float32)
    row[:5] = [1, 3, 2, 3, -1]
    rows = _run(small, row[None, :], [(dict(temperature=1.0, top_k=3, top_p=0.8), [], [])], [0])
    assert rows[0]["gpu"] == 3 and round(rows[0]["lp_gpu"], 5) == -0.92487
    _check(rows, "worked_example")


CASES = [
    dict(temperature=0.0, repetition_penalty=1.3, presence_penalty=0.4, frequency_penalty=0.2),
    dict(temperature=0.8),
    dict(temperature=1.0, top_k=40),
    dict(temperature=1.0, top_k=50, top_p=0.9, min_p=0.05, repetition_penalty=1.2, frequency_penalty=0.3),
    dict(temperature=0.7, top_k=1000, top_p=0.95),
    dict(temperature=1.2, min_p=0.1),
    dict(temperature=0.9, top_k=7, min_p=0.02, presence_penalty=0.5),
    dict(temperature=1.5, top_k=300, top_p=0.5, repetition_penalty=0.8),
]


@pytest.mark.parametrize("which", ["small", "full"])
def test_parameter_grid_matches_oracle(which, request):
    sess = request.getfixturevalue(which)
    V = V_SMALL if which == "small" else V_FULL
    rng = np.random.default_rng(31 if which == "small" else 32)
    n = len(CASES)
    logits = (rng.standard_normal((n, V)) * 3.0).astype(np.float32)
    cases = []
    for i, kw in enumerate(CASES):
        prompt = rng.integers(0, V, 40).tolist()
        output = rng.integers(0, V, 12).tolist() + [int(np.argmax(logits[i]))] * 3
        cases.append((kw, prompt, output))
    _check(_run(sess, logits, cases, list(range(100, 100 + n))), f"grid_{which}")


# nucleus sampling over more ids than the ordered candidate path takes: top_k = 0 (all ids) or a
# top_k beyond 1,024, with peaked, flat and very flat distributions (nuclei of a few ids up to
# most of the vocabulary), with and without min-p and penalties
NUCLEUS = [
    dict(temperature=1.0, top_p=0.9),
    dict(temperature=0.6, top_p=0.5),
    dict(temperature=2.0, top_p=0.95),
    dict(temperature=8.0, top_p=0.99),
    dict(temperature=1.0, top_k=5000, top_p=0.8, min_p=0.01),
    dict(temperature=1.3, top_p=0.7, repetition_penalty=1.2, presence_penalty=0.3, frequency_penalty=0.2),
    dict(temperature=25.0, top_k=2000, top_p=0.6),
    dict(temperature=1.0, top_p=0.999999),
]


@pytest.mark.parametrize("which", ["small", "full"])
def test_nucleus_over_the_whole_vocabulary_matches_oracle(which, request):
    sess = request.getfixturevalue(which)
    V = V_SMALL if which == "small" else V_FULL
    rng = np.random.default_rng(41 if which == "small" else 42)
    n = len(NUCLEUS)
    logits = (rng.standard_normal((n, V)) * 3.0).astype(np.float32)
    cases = []
    for i, kw in enumerate(NUCLEUS):
        prompt = rng.integers(0, V, 30).tolist()
        output = rng.integers(0, V, 10).tolist()
        cases.append((kw, prompt, output))
    _check(_run(sess, logits, cases, list(range(300, 300 + n))), f"nucleus_{which}")


def test_nucleus_cut_inside_equal_values(full):
    # integer logits: long runs of equal values; the nucleus cut falls inside one of them, whose
    # ids are then taken in id order
    rng = np.random.default_rng(43)
    logits = rng.integers(-4, 3, size=(4, V_FULL)).astype(np.float32)
    cases = [(dict(temperature=1.0, top_p=p), [], []) for p in (0.3, 0.5, 0.77, 0.9)]
    _check(_run(full, logits, cases, [21, 22, 23, 24]), "nucleus_ties")


def test_nucleus_is_the_same_on_every_run(full):
    # the same inputs, three times: the same ids and generator states (fixed-order sums)
    rng = np.random.default_rng(44)
    logits = (rng.standard_normal((6, V_FULL)) * 1.5).astype(np.float32)
    cases = [(dict(temperature=1.5, top_p=0.93), [], [])] * 6
    runs = [_run(full, logits, cases, list(range(60, 66))) for _ in range(3)]
    for r in runs[1:]:
        assert [x["gpu"] for x in r] == [x["gpu"] for x in runs[0]]
        assert [x["state_gpu"] for x in r] == [x["state_gpu"] for x in runs[0]]
    _check(runs[0], "nucleus_repeat")


def test_equal_logits_across_the_top_k_cut(small):
    # integer-valued logits: many equal values, the cut of top_k falls inside a run of equals
    rng = np.random.default_rng(33)
    logits = rng.integers(-3, 4, size=(4, V_SMALL)).astype(np.float32)
    cases = [(dict(temperature=1.0, top_k=k, top_p=p), [], []) for k, p in ((7, 1.0), (70, 1.0), (7, 0.6), (100, 0.9))]
    _check(_run(small, logits, cases, [7, 8, 9, 10]), "ties_at_cut")


def test_stream_over_steps_with_growing_history(full):
    from decoder_forward_pass_amd import binding as B
    rng_np = np.random.default_rng(34)
    S, steps = 4, 6
    kw = dict(temperature=0.9, top_k=64, top_p=0.92, repetition_penalty=1.15, frequency_penalty=0.1)
    op, cp = _params(**kw)
    prompts = [rng_np.integers(0, V_FULL, 20).tolist() for _ in range(S)]
    outputs = [[] for _ in range(S)]
    gens = [sm.stream(500 + i) for i in range(S)]
    rng = torch.tensor([list(B.dec_rng_stream(500 + i)) for i in range(S)], dtype=torch.uint64, device="cuda")
    mism = 0
    for t in range(steps):
        logits = (rng_np.standard_normal((S, V_FULL)) * 2.5).astype(np.float32)
        ids, hist = [], []
        for i in range(S):
            h = B.dec_history()
            h.prompt_offset, h.prompt_len = len(ids), len(prompts[i])
            ids.extend(prompts[i])
            h.output_offset, h.output_len = len(ids), len(outputs[i])
            ids.extend(outputs[i])
            hist.append(h)
        nxt, lp = full.sample(torch.tensor(logits, device="cuda"), [cp] * S, hist,
                              torch.tensor(ids, dtype=torch.int32, device="cuda"), rng)
        got = nxt.cpu().numpy()
        for i in range(S):
            tok, _ = sm.sample(logits[i], op, prompts[i], outputs[i], gens[i])
            mism += int(tok != int(got[i]))
            outputs[i].append(tok)  # both sides continue from the oracle's token
    states = rng.cpu().numpy().astype(object)
    report({"type": "sampling_parity", "case": "stream_steps", "rows": S * steps, "ids_equal": S * steps - mism,
            "pass": mism == 0})
    assert mism == 0
    for i in range(S):
        assert int(states[i][0]) & (2 ** 64 - 1) == gens[i].state


def test_refusals(full):
    from decoder_forward_pass_amd import binding as B
    lg = torch.zeros((1, V_FULL), dtype=torch.float32, device="cuda")
    rng = torch.tensor([list(B.dec_rng_stream(1))], dtype=torch.uint64, device="cuda")
    h = B.dec_history()
    for kw, code in ((dict(temperature=1.0, top_p=0.0), B.DEC_E_ARG),
                     (dict(temperature=-1.0), B.DEC_E_ARG),
                     (dict(temperature=1.0, repetition_penalty=0.0), B.DEC_E_ARG)):
        _, cp = _params(**kw)
        with pytest.raises(B.DecError) as e:
            full.sample(lg, [cp], [h], None, rng)
        assert e.value.code == code, kw
    bad = B.dec_history()
    bad.prompt_offset, bad.prompt_len = 0, 5  # no ids given
    _, cp = _params(temperature=1.0)
    with pytest.raises(B.DecError) as e:
        full.sample(lg, [cp], [bad], None, rng)
    assert e.value.code == B.DEC_E_ARG
