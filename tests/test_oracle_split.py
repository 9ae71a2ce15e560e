"""Pins of the oracle's key-split functions (partial_attention, combine).

The combine formula is pinned against the definition of attention itself:
attention over a union of disjoint key ranges must equal the combination of
the attentions over the ranges (the block-combine identity of the streaming
softmax, Hopper tag page contents 3.2.1 / 10.2.1).  A wrong weight, a sign, a
missing max shift or a transposed LSE index fails these checks.
"""
import math

import numpy as np
import pytest

from oracle.attention import attention, combine, partial_attention


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bounds", [[0, 37], [0, 5, 37], [0, 16, 17, 30, 37], [0, 0, 20, 37, 37]])
def test_combine_of_partials_is_full_attention(causal, bounds):
    B, Sq, Sk, Hq, Hkv, d = 2, 29, 37, 4, 2, 8
    q, k, v = _rand((B, Sq, Hq, d), 1), _rand((B, Sk, Hkv, d), 2), _rand((B, Sk, Hkv, d), 3)
    scale = 0.4
    parts = [partial_attention(q, k, v, scale, causal, lo, hi) for lo, hi in zip(bounds[:-1], bounds[1:])]
    o, lse = combine(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    o_ref, lse_ref = attention(q, k, v, scale, causal)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_partial_over_everything_is_attention():
    q, k, v = _rand((1, 9, 2, 4), 4), _rand((1, 11, 2, 4), 5), _rand((1, 11, 2, 4), 6)
    for causal in (False, True):
        o, l = partial_attention(q, k, v, 0.7, causal, 0, 11)
        o_ref, l_ref = attention(q, k, v, 0.7, causal)
        np.testing.assert_allclose(o, o_ref, atol=1e-13)
        np.testing.assert_allclose(l, l_ref, atol=1e-13)


def test_partial_causal_uses_absolute_positions():
    # keys [5, 9) under a causal mask: query i sees keys 5..min(i, 8); rows 0..4 see none
    q, k, v = _rand((1, 8, 1, 4), 7), _rand((1, 12, 1, 4), 8), _rand((1, 12, 1, 4), 9)
    o, l = partial_attention(q, k, v, 1.0, True, 5, 9)
    assert np.all(np.isneginf(l[0, 0, :5])) and np.all(o[0, :5] == 0)
    for i in range(5, 8):
        keys = np.arange(5, min(i, 8) + 1)
        s = q[0, i, 0] @ k[0, keys, 0].T
        assert math.isclose(l[0, 0, i], float(np.log(np.exp(s).sum())), abs_tol=1e-12)
        w = np.exp(s - s.max()); w /= w.sum()
        np.testing.assert_allclose(o[0, i, 0], w @ v[0, keys, 0], atol=1e-12)


def test_combine_two_parts_closed_form():
    # O = w1 O1 + w2 O2 with w_p = e^{L_p} / (e^{L1} + e^{L2}); LSE = log(e^{L1} + e^{L2})
    o1, o2 = _rand((1, 1, 1, 3), 10), _rand((1, 1, 1, 3), 11)
    l1, l2 = 2.5, -1.0
    o, lse = combine(np.stack([o1, o2]), np.array([[[[l1]]], [[[l2]]]]))
    w1 = math.exp(l1) / (math.exp(l1) + math.exp(l2))
    np.testing.assert_allclose(o, w1 * o1 + (1 - w1) * o2, atol=1e-15)
    assert math.isclose(lse[0, 0, 0], math.log(math.exp(l1) + math.exp(l2)), abs_tol=1e-15)


def test_combine_single_part_order_and_empty_parts():
    o1, o2, o3 = _rand((1, 2, 1, 3), 12), _rand((1, 2, 1, 3), 13), _rand((1, 2, 1, 3), 14)
    l1, l2 = np.array([[[0.3, -2.0]]]), np.array([[[1.1, 0.5]]])
    o, lse = combine(o1[None], l1[None])
    np.testing.assert_allclose(o, o1, atol=1e-15)
    np.testing.assert_allclose(lse, l1, atol=1e-15)
    a = combine(np.stack([o1, o2]), np.stack([l1, l2]))
    b = combine(np.stack([o2, o1]), np.stack([l2, l1]))
    np.testing.assert_allclose(a[0], b[0], atol=1e-15)
    np.testing.assert_allclose(a[1], b[1], atol=1e-15)
    # an empty part (-inf) changes nothing, whatever its O holds
    empty = np.full_like(l1, -np.inf)
    c = combine(np.stack([o1, o2, np.full_like(o3, 7.0)]), np.stack([l1, l2, empty]))
    np.testing.assert_allclose(c[0], a[0], atol=1e-15)
    np.testing.assert_allclose(c[1], a[1], atol=1e-15)
    # all parts empty: O = 0, LSE = -inf
    d = combine(np.stack([o1, o2]), np.stack([empty, empty]))
    assert np.all(d[0] == 0) and np.all(np.isneginf(d[1]))
