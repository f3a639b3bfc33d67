"""GPU parity at full size for uint4-g32 weights (W = (q - zp) * scale, "Byte-identical...",
"The bar we set") with an f16 KV cache: 64 sequences with seeded ragged contexts uniform in
[512, 8192], prefilled through the library, then 128 greedy decode steps at batch 64 with the
next token ids passed on the device.

Dequantisation is checked bit for bit against the oracle's float32 evaluation of the same
formula on whole matrices. The oracle follows the shortest and the longest sequence one by one
(prefill, then every decode step with the GPU's tokens), comparing the last prompt logits and
a fixed set of decode steps; gate 2e-2 of each row's oracle logit range. The shortest sequence
is also run alone: its decode logits must equal the batch's bit for bit (the batched calls of
thousands of rows widen each layer's 4-bit matrices to bf16 before the products; the lone call
of a few hundred rows dequantises inside the products, so this also checks that both give the
same operands).
"""

import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from gpu_util import compare, report
import oracle.model as om
from synthetic import MODELS, WORKLOADS, make_context_lengths, make_prompts, make_weights

REL = 2e-2
CHECK_STEPS = (0, 1, 64, 127)
MAX_ROWS = 32768


@pytest.fixture(scope="module")
def weights():
    wl = WORKLOADS["q06b_uint4_b64_ragged_d128"]
    return make_weights(MODELS[wl.model])


@pytest.fixture(scope="module")
def run(weights):
    from decoder_forward_pass_amd import binding as B
    from decoder_forward_pass_amd.session import BlockAllocator, Session
    wl = WORKLOADS["q06b_uint4_b64_ragged_d128"]
    shape = MODELS[wl.model]
    w = weights
    prompts = make_prompts(wl)
    lens = make_context_lengths(wl)
    S, steps = wl.n_seqs, wl.decode_steps
    ctx = int(lens.max()) + steps
    short, long_ = int(np.argmin(lens)), int(np.argmax(lens))
    n_blocks = sum(math.ceil((int(L) + steps) / shape.block_tokens) for L in lens)
    n_blocks += math.ceil((int(lens[short]) + steps) / shape.block_tokens)
    s = Session(shape, w, max_context=ctx, n_blocks=n_blocks, max_rows=MAX_ROWS, max_seqs=S)
    alloc = BlockAllocator(n_blocks, shape.block_tokens, seed=6)
    for i in range(S):
        alloc.ensure(i, int(lens[i]) + steps)
    alloc.ensure("alone", int(lens[short]) + steps)
    hist = torch.zeros((steps + 1, S), dtype=torch.int32, device="cuda")
    last = torch.empty((S, shape.vocab), dtype=torch.float32, device="cuda")
    # prefill in calls of consecutive sequences, each at most MAX_ROWS tokens
    i = 0
    while i < S:
        j, rows = i, 0
        while j < S and rows + int(lens[j]) <= MAX_ROWS:
            rows += int(lens[j])
            j += 1
        print(f"[c5] prefill sequences {i}..{j - 1} ({rows} tokens)", flush=True)
        s.prefill([0] * (j - i), lens[i:j], np.concatenate(prompts[i:j]), alloc.table_array(list(range(i, j))),
                  B.DEC_LOGITS_LAST, logits=last[i:j], next_tokens=hist[0, i:j])
        i = j
    tbl = alloc.table_array(list(range(S)))
    tbl_alone = alloc.table_array(["alone"])
    s.prefill([0], [int(lens[short])], prompts[short], tbl_alone, B.DEC_LOGITS_NONE)
    keep = {}
    logits = torch.empty((S, shape.vocab), dtype=torch.float32, device="cuda")
    pos = lens.astype(np.int32)
    print(f"[c5] decode {steps} steps", flush=True)
    for t in range(steps):
        s.decode_step(pos + t, tbl, tokens_device=hist[t], logits=logits, next_tokens=hist[t + 1])
        if t in CHECK_STEPS:
            keep[t] = logits[[short, long_]].cpu().numpy()
    hist_cpu = hist.cpu().numpy()
    la = torch.empty((1, shape.vocab), dtype=torch.float32, device="cuda")
    alone = {}
    for t in range(steps):
        s.decode_step([int(pos[short]) + t], tbl_alone, tokens_host=hist_cpu[t, short:short + 1], logits=la)
        if t in CHECK_STEPS:
            alone[t] = la.cpu().numpy()[0]
    deq = {idx: s.dequant(idx).cpu().numpy() for idx in (0, 2, 7, 11, 1 + 27 * 11 + 9)}
    out = dict(last=last[[short, long_]].cpu().numpy(), hist=hist_cpu, keep=keep, alone=alone, deq=deq,
               short=short, long=long_, lens=lens)
    torch.cuda.synchronize()
    s.close()
    yield wl, shape, w, prompts, out


def test_dequant_is_bit_exact_on_whole_matrices(run):
    wl, shape, w, prompts, out = run
    from decoder_forward_pass_amd.session import make_config
    from decoder_forward_pass_amd import binding as B
    cfg = make_config(shape, max_context=64, n_blocks=1, max_rows=1, max_seqs=1)
    for idx, got in out["deq"].items():
        e = B.dec_weight_entry(cfg, idx)
        nm = e.name.decode()
        src = w.embed if nm == "embed" else w.layers[e.layer][nm]
        ref = om.widen_matrix(src, "uint4").astype(np.float32)
        assert got.shape == ref.shape
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), nm


def test_decode_batch_invariance_bit_exact(run):
    wl, shape, w, prompts, out = run
    for t in CHECK_STEPS:
        assert np.array_equal(out["keep"][t][0].view(np.uint32), out["alone"][t].view(np.uint32)), t


@pytest.mark.parametrize("which", ["short", "long"])
def test_ragged_decode_matches_oracle(run, which):
    wl, shape, w, prompts, out = run
    seq = out[which]
    k = 0 if which == "short" else 1
    L = int(out["lens"][seq])
    dec = om.OracleDecoder(w)
    c = dec.new_cache(capacity=L + wl.decode_steps)
    print(f"[c5] oracle prefill seq {seq} ({L} tokens)", flush=True)
    ref_last = dec.forward([(prompts[seq], c)], logits="last")[0]
    rows_gpu, rows_ref = [out["last"][k]], [ref_last]
    hist = out["hist"]
    flips = bad = 0

    def choice(ref_row, tok):
        nonlocal flips, bad
        top = int(np.argmax(ref_row))
        if top != tok:
            flips += 1
            if ref_row[top] - ref_row[tok] > REL * (ref_row.max() - ref_row.min()):
                bad += 1

    choice(ref_last, int(hist[0, seq]))
    for t in range(wl.decode_steps):
        tok = np.array([hist[t, seq]])
        r = dec.forward([(tok, c)], logits="all")[0]
        choice(r, int(hist[t + 1, seq]))  # every step's greedy choice
        if t in CHECK_STEPS:
            rows_gpu.append(out["keep"][t][k])
            rows_ref.append(r)
    row = compare(np.array(rows_gpu), np.array(rows_ref), rel_range=REL)
    row.update(type="logit_parity", case=wl.name, path=f"{which}_seq{seq}_ctx{L}", greedy_flips=flips,
               greedy_steps_checked=wl.decode_steps + 1,
               greedy_flips_outside_gate=bad)
    report(row)
    assert row["pass"], row
    assert bad == 0
