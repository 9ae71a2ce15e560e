"""GPU parity at the largest sizes the library accepts: a query tensor and a
key/value tensor just under the 2^31-element limit of the in-kernel 32-bit
offsets (the next size up is rejected with ATTN_ERR_SIZE, checked in
test_boundary.py).  The other side is kept small so that the work stays
short; the oracle computes sampled rows.

Inputs are drawn on the GPU with a seeded torch generator (4 GiB per tensor
is too much to draw on the host here); the oracle reads the sampled rows of
the same tensors copied back.  Tolerances as for every bf16 forward:
O max-abs <= 1e-2, relative RMS <= 5e-3, LSE abs <= 1e-3.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A

pytestmark = pytest.mark.gpu

O_MAXABS, O_RELRMS, LSE_ABS = 1e-2, 5e-3, 1e-3


@pytest.fixture(scope="module")
def ea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_75_amd as m
    m.library()
    return m


def compare(o, lse, o_ref, l_ref, tag):
    o = o.float().double().numpy()
    l = lse.double().numpy()
    diff = np.abs(o - o_ref)
    maxabs = float(diff.max())
    relrms = float(np.sqrt((diff ** 2).sum() / (o_ref ** 2).sum()))
    lmax = float(np.abs(l - l_ref).max())
    print(f"[parity] {tag} O max-abs {maxabs:.3e} rel-RMS {relrms:.3e} LSE max-abs {lmax:.3e}", flush=True)
    assert maxabs <= O_MAXABS and relrms <= O_RELRMS and lmax <= LSE_ABS, tag


def randn(shape, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)


def test_query_tensor_at_the_limit(ea):
    # q, o: 131071 x 128 heads x 128 = 2^31 - 16384 elements (4 GiB each)
    Sq, H, d, Sk = 131071, 128, 128, 64
    assert Sq * H * d < 2 ** 31
    print(f"[case] limit: q [1, {Sq}, {H}, {d}], k/v [1, {Sk}, {H}, {d}]", flush=True)
    q = randn((1, Sq, H, d), 61)
    k = randn((1, Sk, H, d), 62)
    v = randn((1, Sk, H, d), 63)
    for causal in (False, True):
        o, lse = ea.fwd(q, k, v, causal=causal)
        torch.cuda.synchronize()
        rows = np.array([0, 1, 63, 64, 65, 4095, 65536, Sq - 257, Sq - 2, Sq - 1])
        heads = [0, 77, H - 1]
        qs = q[:, rows][:, :, heads].cpu()
        o_ref, l_ref = A.attention(qs, k[:, :, heads].cpu(), v[:, :, heads].cpu(), 1 / math.sqrt(d), False)
        if causal:
            # row i sees keys 0 .. min(i, Sk - 1): the sampled rows compared one by one
            for j, r in enumerate(rows):
                n = min(int(r), Sk - 1) + 1
                orj, lrj = A.attention(qs[:, j:j + 1], k[:, :n, heads].cpu(), v[:, :n, heads].cpu(),
                                       1 / math.sqrt(d), False)
                o_ref[:, j:j + 1], l_ref[:, :, j:j + 1] = orj, lrj
        compare(o[:, rows][:, :, heads].cpu(), lse[:, heads][:, :, rows].cpu(), o_ref, l_ref,
                f"q at limit c{int(causal)}")
        del o, lse
    torch.cuda.empty_cache()


def test_key_tensor_at_the_limit(ea):
    # k, v: 1048575 keys x 16 KV heads x 128 = 2^31 - 2048 elements (4 GiB each);
    # decode-like: 4 query rows per head, GQA 4:1, plain and split-KV
    Sk, Hkv, Hq, d, Sq = 1048575, 16, 64, 128, 4
    assert Sk * Hkv * d < 2 ** 31
    print(f"[case] limit: k/v [1, {Sk}, {Hkv}, {d}], q [1, {Sq}, {Hq}, {d}]", flush=True)
    k = randn((1, Sk, Hkv, d), 64)
    v = randn((1, Sk, Hkv, d), 65)
    q = randn((1, Sq, Hq, d), 66)
    heads = [0, 37, Hq - 1]
    kvh = sorted(set(h // (Hq // Hkv) for h in heads))
    kc, vc = k[:, :, kvh].cpu(), v[:, :, kvh].cpu()
    qc = q[:, :, heads].cpu()
    # map the sampled query heads onto the copied KV heads
    o_ref = np.zeros((1, Sq, len(heads), d))
    l_ref = np.zeros((1, len(heads), Sq))
    for j, h in enumerate(heads):
        hk = kvh.index(h // (Hq // Hkv))
        oo, ll = A.attention(qc[:, :, j:j + 1], kc[:, :, hk:hk + 1], vc[:, :, hk:hk + 1], 1 / math.sqrt(d), False)
        o_ref[:, :, j:j + 1], l_ref[:, j:j + 1] = oo, ll
    for name, run in (("plain", lambda: ea.fwd(q, k, v)), ("split", lambda: ea.fwd_splitkv(q, k, v))):
        o, lse = run()
        torch.cuda.synchronize()
        compare(o[:, :, heads].cpu(), lse[:, heads].cpu(), o_ref, l_ref, f"k at limit {name}")
        del o, lse
    torch.cuda.empty_cache()
