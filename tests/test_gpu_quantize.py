"""GPU: symmetric int4-g32 quantisation at load (dec_quantize_int4_sym; "Candle model runner"
2.5, the runner's quantise-at-load route) against the oracle's quantiser, bit for bit: values
and f16 scale bits of random matrices (groups of zeros, exact ties for rint, a wide range of
magnitudes) and of every matrix of the tiny decoder."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from oracle import numerics as nx
from synthetic import MODELS, make_weights


def gpu_quantize(w):
    from decoder_forward_pass_amd import binding as B
    rows, cols = w.shape
    wd = torch.tensor(w, dtype=torch.float32, device="cuda")
    q = torch.zeros((rows, cols // 2), dtype=torch.uint8, device="cuda")
    s = torch.zeros((rows, cols // 32), dtype=torch.int16, device="cuda")
    B.dec_quantize_int4_sym(torch.cuda.current_stream().cuda_stream, wd.data_ptr(), rows, cols, q.data_ptr(),
                            s.data_ptr())
    torch.cuda.synchronize()
    packed = q.cpu().numpy()
    lo = (packed & 15).astype(np.int16)
    hi = (packed >> 4).astype(np.int16)
    vals = np.empty((rows, cols), np.int16)
    vals[:, 0::2] = np.where(lo > 7, lo - 16, lo)
    vals[:, 1::2] = np.where(hi > 7, hi - 16, hi)
    return vals.astype(np.int8), s.cpu().numpy().view(np.uint16)


def test_random_matrices_match_the_oracle():
    rng = np.random.default_rng(41)
    w = (rng.standard_normal((96, 512)) * rng.uniform(1e-5, 50.0, size=(96, 1))).astype(np.float32)
    w[3, 64:96] = 0.0                                    # a group of zeros
    w[7, :32] = np.float32(0.25) * rng.integers(-7, 8, 32).astype(np.float32)  # exact multiples
    w[8, :32] = np.float32(1.75) * (np.arange(32) % 2 * 2 - 1)  # equal magnitudes
    w[9, :32] = 0.0  # s = f16(3.5 / 7) = 0.5 exactly: quotients 2.5, -1.5, 0.5 are rint ties
    w[9, :4] = [3.5, 1.25, -0.75, 0.25]
    q, s = gpu_quantize(w)
    rq, rs = nx.quantize_int4_sym_g32(w)
    assert np.array_equal(s, rs)
    assert np.array_equal(q, rq)


def test_tiny_decoder_matrices_match_the_oracle():
    w = make_weights(MODELS["tiny_f32"])
    mats = [w.embed] + [layer[n] for layer in w.layers for n in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")]
    for m in mats:
        q, s = gpu_quantize(np.asarray(m, np.float32))
        rq, rs = nx.quantize_int4_sym_g32(m)
        assert np.array_equal(s, rs) and np.array_equal(q, rq)


def test_refuses_misshaped_input():
    from decoder_forward_pass_amd import binding as B
    w = torch.zeros((4, 48), dtype=torch.float32, device="cuda")
    q = torch.zeros((4, 24), dtype=torch.uint8, device="cuda")
    s = torch.zeros((4, 2), dtype=torch.int16, device="cuda")
    with pytest.raises(B.DecError) as e:
        B.dec_quantize_int4_sym(0, w.data_ptr(), 4, 48, q.data_ptr(), s.data_ptr())
    assert e.value.code == B.DEC_E_ARG
