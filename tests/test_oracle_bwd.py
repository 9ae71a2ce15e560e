"""Pins of the oracle's attention backward (no GPU).

The gradients are checked against things other than their own formula:
central finite differences of the oracle's forward (itself pinned in
test_oracle.py), torch's scaled_dot_product_attention differentiated by
autograd in float64 on the CPU, and identities the definition implies (shift
invariances, a single key, causal row 0, GQA as a sum of MHA heads, varlen as
independent sequences).
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def loss(q, k, v, do, dlse, scale, causal):
    o, l = A.attention(q, k, v, scale, causal)
    val = float((o * do).sum())
    if dlse is not None:
        val += float((l * dlse).sum())
    return val


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("with_dlse", [False, True])
def test_finite_differences(causal, with_dlse):
    # L = <dO, O> + <dlse, LSE>: its gradient is exactly what the backward returns
    B, Sq, Sk, Hq, Hkv, d = 1, 5, 7, 4, 2, 3
    q, k, v = rand((B, Sq, Hq, d), 1), rand((B, Sk, Hkv, d), 2), rand((B, Sk, Hkv, d), 3)
    do = rand((B, Sq, Hq, d), 4)
    dlse = rand((B, Hq, Sq), 5) if with_dlse else None
    scale = 0.7
    dq, dk, dv = A.attention_backward(q, k, v, do, scale, causal, dlse)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = loss(args["q"], args["k"], args["v"], do, dlse, scale, causal)
            args[name] = xm
            lm = loss(args["q"], args["k"], args["v"], do, dlse, scale, causal)
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g, num, atol=1e-7, rtol=1e-6, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_autograd(causal):
    B, Sq, Sk, Hq, Hkv, d = 2, 9, 13, 6, 2, 8
    g = torch.Generator().manual_seed(6)
    q = torch.randn(B, Sq, Hq, d, generator=g, dtype=torch.float64)
    k = torch.randn(B, Sk, Hkv, d, generator=g, dtype=torch.float64)
    v = torch.randn(B, Sk, Hkv, d, generator=g, dtype=torch.float64)
    do = torch.randn(B, Sq, Hq, d, generator=g, dtype=torch.float64)
    qt, kt, vt = (x.transpose(1, 2).clone().requires_grad_(True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=0.3,
                                                         enable_gqa=True)
    o.backward(do.transpose(1, 2))
    dq, dk, dv = A.attention_backward(q, k, v, do, 0.3, causal)
    np.testing.assert_allclose(dq, qt.grad.transpose(1, 2).numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad.transpose(1, 2).numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, vt.grad.transpose(1, 2).numpy(), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_shift_invariances(causal):
    # O is unchanged by k_j -> k_j + u (softmax shift) so sum_j dK_j = 0;
    # V -> V + 1 b^T shifts every seen row of O by b, so sum_j dV_j = sum_i dO_i
    B, Sq, Sk, Hq, Hkv, d = 2, 11, 11, 4, 4, 5
    q, k, v = rand((B, Sq, Hq, d), 7), rand((B, Sk, Hkv, d), 8), rand((B, Sk, Hkv, d), 9)
    do = rand((B, Sq, Hq, d), 10)
    dq, dk, dv = A.attention_backward(q, k, v, do, 0.5, causal)
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=1), do.sum(axis=1), atol=1e-12)


def test_single_key_and_causal_row_zero():
    # one key: P = 1, so dS = 0 -> dQ = dK = 0 and dV = sum of dO
    q, k, v = rand((1, 6, 2, 4), 11), rand((1, 1, 2, 4), 12), rand((1, 1, 2, 4), 13)
    do = rand((1, 6, 2, 4), 14)
    dq, dk, dv = A.attention_backward(q, k, v, do, 0.9, False)
    assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14
    np.testing.assert_allclose(dv[0, 0], do[0].sum(axis=0), atol=1e-14)
    # causal: query 0 sees key 0 only, so its dQ is 0 whatever the keys
    q, k, v = rand((1, 6, 2, 4), 15), rand((1, 6, 2, 4), 16), rand((1, 6, 2, 4), 17)
    dq, _, _ = A.attention_backward(q, k, v, rand((1, 6, 2, 4), 18), 0.9, True)
    assert np.abs(dq[0, 0]).max() < 1e-14 and np.abs(dq[0, 1]).max() > 1e-3


def test_gqa_is_sum_of_mha():
    B, S, Hq, Hkv, d = 1, 8, 6, 2, 4
    q, k, v = rand((B, S, Hq, d), 19), rand((B, S, Hkv, d), 20), rand((B, S, Hkv, d), 21)
    do = rand((B, S, Hq, d), 22)
    dq, dk, dv = A.attention_backward(q, k, v, do, 0.4, True)
    kr, vr = np.repeat(k, Hq // Hkv, axis=2), np.repeat(v, Hq // Hkv, axis=2)
    dq2, dk2, dv2 = A.attention_backward(q, kr, vr, do, 0.4, True)
    np.testing.assert_allclose(dq, dq2, atol=1e-13)
    np.testing.assert_allclose(dk, dk2.reshape(B, S, Hkv, Hq // Hkv, d).sum(axis=3), atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(B, S, Hkv, Hq // Hkv, d).sum(axis=3), atol=1e-13)


def test_varlen_is_independent_sequences():
    lens = [3, 0, 5, 1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H, d = int(cu[-1]), 2, 4
    q, k, v, do = rand((T, H, d), 23), rand((T, H, d), 24), rand((T, H, d), 25), rand((T, H, d), 26)
    dq, dk, dv = A.attention_backward(q, k, v, do, 0.6, True, cu_seqlens=cu)
    for s in range(len(lens)):
        a, b = cu[s], cu[s + 1]
        if b == a:
            continue
        g = A.attention_backward(q[None, a:b], k[None, a:b], v[None, a:b], do[None, a:b], 0.6, True)
        np.testing.assert_allclose(dq[a:b], g[0][0], atol=1e-14)
        np.testing.assert_allclose(dk[a:b], g[1][0], atol=1e-14)
        np.testing.assert_allclose(dv[a:b], g[2][0], atol=1e-14)


def test_row_chunking_does_not_change_the_result():
    q, k, v, do = rand((40, 8), 27), rand((33, 8), 28), rand((33, 8), 29), rand((40, 8), 30)
    a = A.head_backward(q, k, v, do, 0.35, True)
    b = A.head_backward(q, k, v, do, 0.35, True, row_chunk=7)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, atol=1e-13)


def test_backward_flop_count():
    assert A.attention_backward_flops(8, 8, 4, False) == 2.5 * 4 * 4 * 64
    assert A.attention_backward_flops(8, 8, 4, True) == 2.5 * 4 * 4 * 36
