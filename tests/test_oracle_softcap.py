"""Pins of the oracle's softcapped scores (no GPU): a scalar brute force
written with math.tanh / math.exp / math.fsum on tiny shapes, the limit of a
very large cap (plain attention), zero queries (tanh 0 = 0), and the bound
|capped score| < cap on the LSE."""
import math

import numpy as np
import pytest

from oracle import attention as A


def brute(q, k, v, scale, causal, cap):
    Sq, Sk, d = q.shape[0], k.shape[0], v.shape[1]
    O = np.zeros((Sq, d))
    L = np.zeros(Sq)
    for i in range(Sq):
        s = []
        for j in range(Sk):
            if causal and j > i:
                continue
            x = scale * math.fsum(q[i, t] * k[j, t] for t in range(q.shape[1]))
            s.append((j, cap * math.tanh(x / cap)))
        m = max(x for _, x in s)
        w = [(j, math.exp(x - m)) for j, x in s]
        l = math.fsum(x for _, x in w)
        for t in range(d):
            O[i, t] = math.fsum(x * v[j, t] for j, x in w) / l
        L[i] = m + math.log(l)
    return O, L


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("cap", [0.5, 3.0, 30.0])
def test_brute_force(causal, cap):
    rng = np.random.default_rng(41)
    q, k, v = rng.standard_normal((6, 4)) * 3, rng.standard_normal((9, 4)) * 3, rng.standard_normal((9, 5))
    o, l = A.head_attention(q, k, v, 0.8, causal, softcap=cap)
    ob, lb = brute(q, k, v, 0.8, causal, cap)
    np.testing.assert_allclose(o, ob, atol=1e-12)
    np.testing.assert_allclose(l, lb, atol=1e-12)


def test_large_cap_is_plain_attention():
    rng = np.random.default_rng(42)
    q, k, v = rng.standard_normal((1, 20, 2, 8)), rng.standard_normal((1, 30, 2, 8)), rng.standard_normal((1, 30, 2, 8))
    o1, l1 = A.attention(q, k, v, 0.35, True, softcap=1e7)
    o2, l2 = A.attention(q, k, v, 0.35, True)
    np.testing.assert_allclose(o1, o2, atol=1e-9)
    np.testing.assert_allclose(l1, l2, atol=1e-9)


def test_zero_q_and_lse_bound():
    rng = np.random.default_rng(43)
    k, v = rng.standard_normal((1, 25, 1, 8)) * 5, rng.standard_normal((1, 25, 1, 8))
    o, l = A.attention(np.zeros((1, 25, 1, 8)), k, v, 0.5, True, softcap=2.0)
    np.testing.assert_allclose(l[0, 0], np.log(np.arange(1, 26)), atol=1e-13)
    q = rng.standard_normal((1, 25, 1, 8)) * 50
    _, l = A.attention(q, k, v, 0.5, False, softcap=2.0)
    assert np.all(l < np.log(25) + 2.0) and np.all(l > np.log(25) - 2.0)
