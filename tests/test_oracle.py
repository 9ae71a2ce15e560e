"""Pins for the fp64 attention oracle: closed forms, invariants, library
routines and brute force.  Each is chosen so that a plausible mistake in the
oracle (a dropped term, a wrong sign or index, a transposed operand, a wrong
mask direction, a wrong GQA map) fails at least one of them."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A

RNG = np.random.default_rng(1234)


def rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


# ---------------------------------------------------------------- normalisation
@pytest.mark.parametrize("causal", [False, True])
def test_prob_rows_sum_to_one(causal):
    q, k = rand(37, 16), rand(53, 16)
    p, m, l = A.head_probs(q, k, 0.25, causal)
    assert np.all(p >= 0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)
    if causal:
        i, j = np.nonzero(p)
        assert np.all(j <= i)


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("causal", [False, True])
def test_zero_q_gives_log_n_and_mean_v(causal):
    B, S, H, d = 2, 45, 3, 8
    q = np.zeros((B, S, H, d))
    k, v = rand(B, S, H, d), rand(B, S, H, d)
    O, L = A.attention(q, k, v, 0.3, causal)
    for i in range(S):
        n = i + 1 if causal else S
        np.testing.assert_allclose(L[:, :, i], math.log(n), atol=1e-12)
        np.testing.assert_allclose(O[:, i], v[:, :n].mean(axis=1), atol=1e-12)


def test_identical_v_rows():
    B, S, H, d = 1, 33, 2, 16
    q, k = rand(B, S, H, d), rand(B, S, H, d)
    row = rand(d)
    v = np.broadcast_to(row, (B, S, H, d)).copy()
    for causal in (False, True):
        O, _ = A.attention(q, k, v, 0.7, causal)
        np.testing.assert_allclose(O, np.broadcast_to(row, O.shape), atol=1e-12)


def test_single_key():
    q, k, v = rand(1, 9, 2, 8), rand(1, 1, 2, 8), rand(1, 1, 2, 8)
    scale = 0.41
    O, L = A.attention(q, k, v, scale, False)
    np.testing.assert_allclose(O, np.broadcast_to(v, O.shape), atol=1e-12)
    expect = scale * np.einsum("bshd,bhd->bhs", q, k[:, 0])
    np.testing.assert_allclose(L, expect, atol=1e-12)


def test_two_keys_closed_form():
    q, k, v = rand(1, 6, 1, 4), rand(1, 2, 1, 4), rand(1, 2, 1, 4)
    scale = 0.9
    O, L = A.attention(q, k, v, scale, False)
    for i in range(6):
        s0 = scale * float(q[0, i, 0] @ k[0, 0, 0])
        s1 = scale * float(q[0, i, 0] @ k[0, 1, 0])
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        np.testing.assert_allclose(O[0, i, 0], w0 * v[0, 0, 0] + (1 - w0) * v[0, 1, 0], atol=1e-12)
        lse = max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1)))
        assert abs(L[0, 0, i] - lse) < 1e-12


def test_two_keys_hand_example():
    # q=(1,0), k0=(2,0), k1=(0,0), scale 1/2: scores 1 and 0, weight on key 0 is e/(1+e)
    q = np.array([[[[1.0, 0.0]]]])
    k = np.array([[[[2.0, 0.0]], [[0.0, 0.0]]]])
    v = np.array([[[[1.0, 2.0]], [[3.0, -1.0]]]])
    O, L = A.attention(q, k, v, 0.5, False)
    w = math.e / (1 + math.e)
    np.testing.assert_allclose(O[0, 0, 0], [w * 1 + (1 - w) * 3, w * 2 - (1 - w)], atol=1e-15)
    assert abs(L[0, 0, 0] - (1.0 + math.log(1 + math.exp(-1.0)))) < 1e-15


# ---------------------------------------------------------------- invariances
def test_key_shift_invariance():
    B, S, H, d = 1, 29, 2, 8
    q, k, v = rand(B, S, H, d), rand(B, S, H, d), rand(B, S, H, d)
    u = rand(d)
    scale = 0.5
    O1, L1 = A.attention(q, k, v, scale, True)
    O2, L2 = A.attention(q, k + u, v, scale, True)
    np.testing.assert_allclose(O1, O2, atol=1e-10)
    shift = scale * np.einsum("bshd,d->bhs", q, u)
    np.testing.assert_allclose(L2 - L1, shift, atol=1e-10)


def test_value_affine_equivariance():
    B, S, H, d = 1, 31, 2, 8
    q, k, v = rand(B, S, H, d), rand(B, S, H, d), rand(B, S, H, d)
    a, bvec = 2.5, rand(d)
    O1, _ = A.attention(q, k, v, 0.3, True)
    O2, _ = A.attention(q, k, a * v + bvec, 0.3, True)
    np.testing.assert_allclose(O2, a * O1 + bvec, atol=1e-10)


def test_key_permutation_invariance_noncausal():
    B, S, H, d = 1, 40, 2, 8
    q, k, v = rand(B, S, H, d), rand(B, S, H, d), rand(B, S, H, d)
    perm = RNG.permutation(S)
    O1, L1 = A.attention(q, k, v, 0.3, False)
    O2, L2 = A.attention(q, k[:, perm], v[:, perm], 0.3, False)
    np.testing.assert_allclose(O1, O2, atol=1e-10)
    np.testing.assert_allclose(L1, L2, atol=1e-10)


def test_causal_row_equals_prefix_attention():
    B, S, H, d = 1, 24, 1, 8
    q, k, v = rand(B, S, H, d), rand(B, S, H, d), rand(B, S, H, d)
    Oc, Lc = A.attention(q, k, v, 0.3, True)
    for i in (0, 5, 23):
        On, Ln = A.attention(q[:, i:i + 1], k[:, :i + 1], v[:, :i + 1], 0.3, False)
        np.testing.assert_allclose(Oc[:, i], On[:, 0], atol=1e-12)
        np.testing.assert_allclose(Lc[:, :, i], Ln[:, :, 0], atol=1e-12)
    On, Ln = A.attention(q, k, v, 0.3, False)
    np.testing.assert_allclose(Oc[:, -1], On[:, -1], atol=1e-12)


# ---------------------------------------------------------------- library routines
@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_fp64(causal):
    B, S, H, d = 2, 70, 3, 32
    q, k, v = rand(B, S, H, d), rand(B, S, H, d), rand(B, S, H, d)
    scale = 1 / math.sqrt(d)
    O, L = A.attention(q, k, v, scale, causal)
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    np.testing.assert_allclose(O, ref.permute(0, 2, 1, 3).numpy(), atol=1e-12)
    s = torch.einsum("bhqd,bhkd->bhqk", tq, tk) * scale
    if causal:
        s = s.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(L, torch.logsumexp(s, dim=-1).numpy(), atol=1e-12)


def test_gqa_equals_repeated_kv():
    B, S, Hq, Hkv, d = 1, 20, 8, 2, 8
    q, k, v = rand(B, S, Hq, d), rand(B, S, Hkv, d), rand(B, S, Hkv, d)
    O1, L1 = A.attention(q, k, v, 0.4, True)
    kr, vr = np.repeat(k, Hq // Hkv, axis=2), np.repeat(v, Hq // Hkv, axis=2)
    O2, L2 = A.attention(q, kr, vr, 0.4, True)
    np.testing.assert_allclose(O1, O2, atol=1e-14)
    np.testing.assert_allclose(L1, L2, atol=1e-14)
    # head 0..3 use kv head 0, heads 4..7 use kv head 1 (not h % Hkv)
    O3, _ = A.attention(q[:, :, 1:2], k[:, :, 0:1], v[:, :, 0:1], 0.4, True)
    np.testing.assert_allclose(O1[:, :, 1], O3[:, :, 0], atol=1e-14)


def test_varlen_equals_per_sequence():
    lengths = [5, 0, 17, 1, 9]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T, H, d = int(cu[-1]), 2, 8
    q, k, v = rand(T, H, d), rand(T, H, d), rand(T, H, d)
    for causal in (False, True):
        O, L = A.attention(q, k, v, 0.5, causal, cu_seqlens=cu)
        for s in range(len(lengths)):
            a, b = cu[s], cu[s + 1]
            if a == b:
                continue
            Os, Ls = A.attention(q[None, a:b], k[None, a:b], v[None, a:b], 0.5, causal)
            np.testing.assert_allclose(O[a:b], Os[0], atol=1e-14)
            np.testing.assert_allclose(L[:, a:b], Ls[0], atol=1e-14)


def test_empty_keys_give_zero_and_minus_inf():
    q, k, v = rand(1, 4, 1, 8), np.zeros((1, 0, 1, 8)), np.zeros((1, 0, 1, 8))
    O, L = A.attention(q, k, v, 0.5, False)
    assert np.all(O == 0) and np.all(np.isneginf(L))


def test_row_subset_matches_full():
    B, S, H, d = 2, 50, 4, 8
    q, k, v = rand(B, S, H, d), rand(B, S, 2, d), rand(B, S, 2, d)
    Of, Lf = A.attention(q, k, v, 0.3, True)
    rows = np.array([0, 7, 49])
    Op, Lp = A.attention(q, k, v, 0.3, True, heads=[1, 3], rows=rows, batches=[1])
    np.testing.assert_allclose(Op[1][rows][:, [1, 3]], Of[1][rows][:, [1, 3]], atol=1e-14)
    np.testing.assert_allclose(Lp[1][[1, 3]][:, rows], Lf[1][[1, 3]][:, rows], atol=1e-14)


# ---------------------------------------------------------------- brute force
def brute_force(q, k, v, scale, causal, group):
    """Scalar loops with math.exp and math.fsum, tiny shapes only."""
    B, Sq, Hq, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Sk = len(k[0])
    O = [[[[0.0] * d for _ in range(Hq)] for _ in range(Sq)] for _ in range(B)]
    L = [[[0.0] * Sq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            hk = h // group
            for i in range(Sq):
                s = []
                for j in range(Sk):
                    if causal and j > i:
                        continue
                    s.append((j, scale * math.fsum(q[b][i][h][t] * k[b][j][hk][t] for t in range(d))))
                mx = max(x for _, x in s)
                w = [(j, math.exp(x - mx)) for j, x in s]
                tot = math.fsum(x for _, x in w)
                L[b][h][i] = mx + math.log(tot)
                for t in range(d):
                    O[b][i][h][t] = math.fsum(x * v[b][j][hk][t] for j, x in w) / tot
    return O, L


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 5, 7, 2, 2, 4), (2, 17, 17, 2, 1, 8), (1, 9, 13, 4, 2, 3)])
def test_brute_force(causal, shape):
    B, Sq, Sk, Hq, Hkv, d = shape
    q, k, v = rand(B, Sq, Hq, d), rand(B, Sk, Hkv, d), rand(B, Sk, Hkv, d)
    O, L = A.attention(q, k, v, 0.37, causal)
    Ob, Lb = brute_force(q.tolist(), k.tolist(), v.tolist(), 0.37, causal, Hq // Hkv)
    np.testing.assert_allclose(O, np.array(Ob), atol=1e-12)
    np.testing.assert_allclose(L, np.array(Lb), atol=1e-12)


def test_flop_count():
    assert A.attention_flops(4, 4, 2, False) == 4 * 2 * 16
    assert A.attention_flops(4, 4, 2, True) == 4 * 2 * 10
    assert A.attention_flops(8192, 8192, 128, True, B=2, H=32) == 4 * 128 * 64 * 8192 * 8193 // 2
    assert A.attention_flops(0, 0, 64, True, H=16, lengths=[3, 2]) == 4 * 64 * 16 * (6 + 3)


def test_row_chunking_does_not_change_the_result():
    # the forward oracle cuts a head's rows into chunks (1024 by default) to
    # bound memory; chunks of 7 (ragged last chunk), 1024 (two chunks) and one
    # chunk for all rows must give the same result, causal and not, also for
    # a row subset that straddles chunk boundaries
    q, k, v = rand(1100, 8), rand(1100, 8), rand(1100, 8)
    for causal in (False, True):
        Oc, Lc = A.head_attention(q, k, v, 0.4, causal, row_chunk=1100)
        for chunk in (7, 1024):
            O, L = A.head_attention(q, k, v, 0.4, causal, row_chunk=chunk)
            np.testing.assert_allclose(O, Oc, rtol=1e-13, atol=1e-14)
            np.testing.assert_allclose(L, Lc, rtol=1e-13, atol=1e-14)
        rows = np.array([0, 6, 7, 8, 1023, 1024, 1099])
        O, L = A.head_attention(q, k, v, 0.4, causal, rows=rows, row_chunk=7)
        np.testing.assert_allclose(O, Oc[rows], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(L, Lc[rows], rtol=1e-13, atol=1e-14)
    # and through the dense entry, whose heads are longer than one chunk
    qd, kd, vd = rand(1, 1100, 2, 8), rand(1, 1100, 1, 8), rand(1, 1100, 1, 8)
    Od, Ld = A.attention(qd, kd, vd, 0.4, True)
    for h in range(2):
        Oh, Lh = A.head_attention(qd[0, :, h], kd[0, :, 0], vd[0, :, 0], 0.4, True, row_chunk=1100)
        np.testing.assert_allclose(Od[0, :, h], Oh, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(Ld[0, h], Lh, rtol=1e-13, atol=1e-14)
