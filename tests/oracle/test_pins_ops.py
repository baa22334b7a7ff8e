"""Pins of the oracle's elementary operations against closed forms,
invariants and brute force (no GPU)."""

import itertools
import math

import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(123)


def test_rmsnorm_unit_rms_and_scale_invariance():
    x = RNG.standard_normal((5, 37))
    g = np.ones(37)
    y = oracle.rmsnorm(x, g, 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-12)
    np.testing.assert_allclose(oracle.rmsnorm(7.5 * x, g, 0.0), y, rtol=1e-12)
    # the gain scales each feature independently
    g2 = RNG.uniform(0.5, 2.0, 37)
    np.testing.assert_allclose(oracle.rmsnorm(x, g2, 0.0), y * g2, rtol=1e-12)
    # eps enters under the root: a constant row c gives c / sqrt(c^2 + eps)
    row = np.full((1, 8), 0.5)
    np.testing.assert_allclose(oracle.rmsnorm(row, np.ones(8), 0.75), 0.5 / 1.0, rtol=1e-12)


def test_silu_special_values():
    assert oracle.silu(np.float64(0.0)) == 0.0
    np.testing.assert_allclose(oracle.silu(np.float64(40.0)), 40.0, rtol=1e-15)
    assert abs(oracle.silu(np.float64(-40.0))) < 1e-15
    x = RNG.standard_normal(50)
    # silu(x) - silu(-x) = x  (sigmoid(x) + sigmoid(-x) = 1)
    np.testing.assert_allclose(oracle.silu(x) - oracle.silu(-x), x, atol=1e-14)


def test_rope_identity_at_zero_and_norm_preserving():
    x = RNG.standard_normal((6, 3, 16))
    np.testing.assert_array_equal(oracle.rope(x, np.zeros(6, np.int32), 1e4), x)
    pos = np.array([1, 5, 17, 300, 4095, 3510], np.int32)
    y = oracle.rope(x, pos, 1e6)
    pair_norm = lambda z: z[..., :8] ** 2 + z[..., 8:] ** 2
    np.testing.assert_allclose(pair_norm(y), pair_norm(x), rtol=1e-12)


def test_rope_relative_position():
    q = RNG.standard_normal((1, 1, 32))
    k = RNG.standard_normal((1, 1, 32))
    dots = []
    for m, n in [(10, 3), (107, 100), (4007, 4000)]:
        qm = oracle.rope(q, np.array([m]), 5e5)
        kn = oracle.rope(k, np.array([n]), 5e5)
        dots.append(float((qm * kn).sum()))
    np.testing.assert_allclose(dots, dots[0], rtol=1e-9)


def test_rope_pairs_rotate_half_and_frequency():
    # the first pair (i=0) rotates by exactly pos radians; the pair couples
    # element i with element i + hd/2
    x = np.zeros((1, 1, 8))
    x[0, 0, 0] = 1.0
    y = oracle.rope(x, np.array([2]), 1e4)
    np.testing.assert_allclose(y[0, 0, [0, 4]], [math.cos(2.0), math.sin(2.0)], atol=1e-15)
    # pair i rotates by pos * theta^(-2i/hd)
    x = np.zeros((1, 1, 8))
    x[0, 0, 3] = 1.0
    y = oracle.rope(x, np.array([7]), 100.0)
    ang = 7 * 100.0 ** (-2 * 3 / 8)
    np.testing.assert_allclose(y[0, 0, [3, 7]], [math.cos(ang), math.sin(ang)], atol=1e-14)


def _attend_brute(q, K, V, ctx):
    """Explicit loops: row j, head h, keys 0..ctx+j."""
    n, Hq, hd = q.shape
    Hkv = K.shape[1]
    out = np.zeros_like(q)
    for j in range(n):
        for h in range(Hq):
            g = h * Hkv // Hq
            lim = ctx + j + 1
            s = [sum(q[j, h, e] * K[p, g, e] for e in range(hd)) / math.sqrt(hd)
                 for p in range(lim)]
            mx = max(s)
            w = [math.exp(v - mx) for v in s]
            tot = sum(w)
            for e in range(hd):
                out[j, h, e] = sum(w[p] * V[p, g, e] for p in range(lim)) / tot
    return out


@pytest.mark.parametrize("n,ctx,Hq,Hkv", [(3, 0, 4, 2), (1, 6, 4, 2), (4, 5, 4, 1), (2, 2, 2, 2)])
def test_attention_matches_brute_force(n, ctx, Hq, Hkv):
    hd = 8
    q = RNG.standard_normal((n, Hq, hd))
    K = RNG.standard_normal((ctx + n, Hkv, hd))
    V = RNG.standard_normal((ctx + n, Hkv, hd))
    np.testing.assert_allclose(oracle.attend_item(q, K, V, ctx), _attend_brute(q, K, V, ctx),
                               rtol=1e-12, atol=1e-12)


def test_attention_single_key_and_identical_keys():
    q = RNG.standard_normal((1, 4, 16))
    K = RNG.standard_normal((1, 2, 16))
    V = RNG.standard_normal((1, 2, 16))
    o = oracle.attend_item(q, K, V, 0)
    # one visible key: output is that key's value, GQA head h -> h // 2
    for h in range(4):
        np.testing.assert_allclose(o[0, h], V[0, h // 2], rtol=1e-14)
    # identical keys: uniform weights, output is the mean of the values
    Kc = np.repeat(K, 9, axis=0)
    Vr = RNG.standard_normal((9, 2, 16))
    o = oracle.attend_item(q, Kc, Vr, 8)
    for h in range(4):
        np.testing.assert_allclose(o[0, h], Vr[:, h // 2].mean(axis=0), rtol=1e-12)


def test_attention_is_causal():
    q = RNG.standard_normal((5, 2, 8))
    K = RNG.standard_normal((7, 1, 8))
    V = RNG.standard_normal((7, 1, 8))
    base = oracle.attend_item(q, K, V, 2)
    K2, V2 = K.copy(), V.copy()
    K2[6] += 3.0
    V2[6] -= 2.0
    mod = oracle.attend_item(q, K2, V2, 2)
    np.testing.assert_array_equal(mod[:4], base[:4])
    assert not np.allclose(mod[4], base[4])
