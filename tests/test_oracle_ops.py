"""Pins of the oracle's per-step operations (CPU only).

Each check compares the oracle with something fixed by the pages or by
mathematics -- closed forms, special values, invariants -- never with a
retyped copy of the oracle's own formula. The ``check_*`` helpers return
True/False so the mutant tests can show that a planted mistake fails them.
"""

import math

import numpy as np
import pytest
from scipy.special import expit

import oracle.model as om


# ---- RoPE -------------------------------------------------------------------------------

def check_rope_identity_at_zero(rope=om.rope) -> bool:
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 2, 32))
    return np.array_equal(rope(x, np.zeros(3, np.int64), 1e6), x)


def check_rope_pairs_split_halves(rope=om.rope, D=128) -> bool:
    """A one-hot in channel j (first half) moves only into channels j and j + D/2."""
    ok = True
    for j in (0, 1, 5, D // 2 - 1):
        x = np.zeros((1, 1, D))
        x[0, 0, j] = 1.0
        y = rope(x, np.array([7]), 1e6)[0, 0]
        nz = set(np.flatnonzero(np.abs(y) > 1e-15).tolist())
        ok &= nz <= {j, j + D // 2} and abs(np.hypot(y[j], y[j + D // 2]) - 1) < 1e-14
    return bool(ok)


def check_rope_angles(rope=om.rope, D=128) -> bool:
    """Pair 0 turns by exactly pos radians; pair D/4 by pos * base^(-1/2) = pos/1000 for base 1e6."""
    ok = True
    for j, pos, angle in ((0, 3, 3.0), (0, 1000, 1000.0), (D // 4, 1000, 1.0), (D // 4, 2500, 2.5)):
        x = np.zeros((1, 1, D))
        x[0, 0, j] = 1.0
        y = rope(x, np.array([pos]), 1e6)[0, 0]
        ok &= abs(y[j] - math.cos(angle)) < 1e-12 and abs(y[j + D // 2] - math.sin(angle)) < 1e-12
    return bool(ok)


def check_rope_relative(rope=om.rope, D=32) -> bool:
    """q.k after rotation depends only on the position difference."""
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, D))
    base = None
    for shift in (0, 1, 17, 4000):
        a = rope(q, np.array([25 + shift]), 1e6)[0, 0]
        b = rope(k, np.array([11 + shift]), 1e6)[0, 0]
        d = float(a @ b)
        if base is None:
            base = d
        elif abs(d - base) > 1e-12:
            return False
    return True


def test_rope_identity_at_zero():
    assert check_rope_identity_at_zero()


@pytest.mark.parametrize("D", [32, 128])
def test_rope_pairs_split_halves(D):
    assert check_rope_pairs_split_halves(D=D)


@pytest.mark.parametrize("D", [32, 128])
def test_rope_angle_special_values(D):
    assert check_rope_angles(D=D)


def test_rope_relative_position():
    assert check_rope_relative()


def test_rope_large_positions_stay_finite_and_norm_preserving():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 3, 128))
    y = om.rope(x, np.array([0, 1, 8191, 8319]), 1e6)
    xa = np.hypot(x[..., :64], x[..., 64:])
    ya = np.hypot(y[..., :64], y[..., 64:])
    assert np.allclose(xa, ya, atol=1e-13, rtol=0)


# ---- RMSNorm ----------------------------------------------------------------------------

def check_rmsnorm_constant_vector(rms=om.rms_norm) -> bool:
    ok = True
    for c in (1e-3, 0.5, 3.0, -2.0):
        x = np.full((1, 64), c)
        y = rms(x, np.ones(64), 1e-6)
        ok &= np.allclose(y, c / math.sqrt(c * c + 1e-6), atol=0, rtol=1e-14)
    return bool(ok)


def test_rmsnorm_constant_vector():
    assert check_rmsnorm_constant_vector()


def test_rmsnorm_unit_rms_scale_invariance_and_gain():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 1024)) * 3
    y = om.rms_norm(x, np.ones(1024), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, atol=1e-14)
    assert np.allclose(om.rms_norm(7.5 * x, np.ones(1024), 0.0), y, atol=1e-14)
    g = rng.uniform(0.5, 2.0, 1024)
    assert np.allclose(om.rms_norm(x, g, 0.0), y * g, atol=1e-14)


# ---- activation -------------------------------------------------------------------------

def test_silu_matches_logistic():
    z = np.linspace(-30, 30, 2001)
    assert np.allclose(om.silu(z), z * expit(z), atol=1e-14, rtol=1e-13)
    assert om.silu(np.array([0.0]))[0] == 0.0


def check_swiglu_gates_first_argument(swiglu=om.swiglu) -> bool:
    g = np.array([-3.0, 0.0, 2.0])
    u = np.array([5.0, 5.0, 5.0])
    return bool(np.allclose(swiglu(g, u), g * expit(g) * u, atol=1e-14))


def test_swiglu_gates_first_argument():
    assert check_swiglu_gates_first_argument()


# ---- attention --------------------------------------------------------------------------

def test_attention_single_key_returns_its_value():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 4, 32))
    K = rng.standard_normal((1, 2, 32))
    V = rng.standard_normal((1, 2, 32))
    o = om.attention(q, K, V, np.array([0]))
    # GQA reading: query head h reads KV head h // (H / H_kv)
    for h in range(4):
        assert np.allclose(o[0, h], V[0, h // 2], atol=0)


def test_attention_equal_keys_average_visible_values():
    rng = np.random.default_rng(6)
    n, D = 6, 32
    K = np.tile(rng.standard_normal((1, 1, D)), (n, 1, 1))
    V = rng.standard_normal((n, 1, D))
    q = rng.standard_normal((n, 1, D))
    o = om.attention(q, K, V, np.arange(n))
    for t in range(n):
        assert np.allclose(o[t, 0], V[: t + 1, 0].mean(axis=0), atol=1e-14)


def check_attention_scale(attn=om.attention, D=32) -> bool:
    """Two keys with scores s and 0 weight their values by logistic(s / sqrt(D))."""
    a, b = 1.7, 2.3
    q = np.zeros((1, 1, D)); q[0, 0, 0] = a
    K = np.zeros((2, 1, D)); K[0, 0, 0] = b
    V = np.zeros((2, 1, D)); V[0, 0, 1] = 1.0; V[1, 0, 2] = 1.0
    o = attn(q, K, V, np.array([1]))[0, 0]
    w = expit(a * b / math.sqrt(D))
    return bool(abs(o[1] - w) < 1e-14 and abs(o[2] - (1 - w)) < 1e-14)


def test_attention_scale_is_one_over_sqrt_head_dim():
    assert check_attention_scale(D=32) and check_attention_scale(D=128)


def check_attention_causal(attn=om.attention) -> bool:
    """Query at position t is unaffected by keys/values at positions > t (absolute)."""
    rng = np.random.default_rng(8)
    ctx, D = 10, 32
    q = rng.standard_normal((3, 2, D))
    K = rng.standard_normal((ctx, 1, D))
    V = rng.standard_normal((ctx, 1, D))
    qpos = np.array([7, 8, 9])  # a cached step: queries at absolute positions 7..9
    o1 = attn(q, K, V, qpos)
    K2, V2 = K.copy(), V.copy()
    K2[8:] += 5.0
    V2[8:] -= 3.0
    o2 = attn(q, K2, V2, qpos)
    o_full = attn(q, K, V, np.array([9, 9, 9]))
    return bool(np.array_equal(o1[0], o2[0]) and not np.allclose(o1[0], o_full[0]))


def test_attention_is_causal_on_absolute_positions():
    assert check_attention_causal()


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(9)
    n, H, Hkv, D = 5, 4, 2, 32
    q = rng.standard_normal((n, H, D))
    K = rng.standard_normal((n, Hkv, D))
    V = rng.standard_normal((n, Hkv, D))
    pos = np.arange(n)
    o = om.attention(q, K, V, pos)
    Kr = np.repeat(K, H // Hkv, axis=1)
    Vr = np.repeat(V, H // Hkv, axis=1)
    o_mha = om.attention(q, Kr, Vr, pos)
    assert np.array_equal(o, o_mha)
