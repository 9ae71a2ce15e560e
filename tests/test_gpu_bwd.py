"""GPU parity of the attention backward (attn_bwd, through the C ABI) against
the fp64 oracle's gradients on the same seeded inputs.

The kernel's inputs o and lse are the oracle forward's (o rounded to the
kernel dtype), so every expected value comes from the oracle; one test feeds
the GPU forward's own o and lse instead (end to end).

Tolerance (no figure for gradients is printed on the pages; derived from the
arithmetic): the kernel rounds P and dS to the 16-bit operand type before
their GEMMs and rounds dQ, dK, dV on output, three independent relative
errors of at most 2^-9 (bf16) each, RMS about 2^-9 / sqrt(3) = 1.1e-3, so
about 2e-3 together; fp32 accumulation adds little.  Gate: relative RMS
<= 1e-2 per gradient (5x that estimate), and every element within
3e-2 * max|reference| of it.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A

pytestmark = pytest.mark.gpu

REL_RMS, REL_MAX = 1e-2, 3e-2


@pytest.fixture(scope="module")
def ea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_75_amd as m
    m.library()
    return m


def grad_inputs(B, Sq, Sk, Hq, Hkv, d, dtype, seed, causal, with_dlse=False):
    q, k, v = W.make_dense(B, Sq, Sk, Hq, Hkv, d, dtype, seed=seed)
    g = torch.Generator().manual_seed(seed + 1000)
    do = torch.randn(B, Sq, Hq, d, generator=g).to(q.dtype)
    dlse = torch.randn(B, Hq, Sq, generator=g) if with_dlse else None
    o_ref, l_ref = A.attention(q, k, v, 1 / math.sqrt(d), causal)
    o = torch.from_numpy(o_ref).to(q.dtype)
    lse = torch.from_numpy(l_ref).float()
    return q, k, v, do, dlse, o, lse


def compare(name, got, ref, tag):
    x = got.detach().float().cpu().double().numpy()
    assert np.isfinite(x).all(), (tag, name)
    err = np.abs(x - ref)
    den = float(np.sqrt((ref ** 2).sum()))
    scale = float(np.abs(ref).max())
    rel = float(np.sqrt((err ** 2).sum())) / den if den > 0 else float(err.max())
    mx = float(err.max()) / scale if scale > 0 else float(err.max())
    print(f"[parity] {tag} {name} rel-RMS {rel:.3e} max/maxref {mx:.3e}", flush=True)
    assert rel <= REL_RMS, (tag, name, rel)
    assert mx <= REL_MAX, (tag, name, mx)


def run_case(ea, shape, d, dtype, causal, seed, with_dlse=False):
    B, Sq, Sk, Hq, Hkv = shape
    q, k, v, do, dlse, o, lse = grad_inputs(B, Sq, Sk, Hq, Hkv, d, dtype, seed, causal, with_dlse)
    dev = [t.cuda() for t in (q, k, v, o, lse, do)]
    dq, dk, dv = ea.bwd(*dev, causal=causal, dlse=None if dlse is None else dlse.cuda())
    torch.cuda.synchronize()
    rq, rk, rv = A.attention_backward(q, k, v, do, 1 / math.sqrt(d), causal, dlse)
    tag = f"bwd {dtype} d{d} c{int(causal)} {shape}{' dlse' if with_dlse else ''}"
    compare("dq", dq, rq, tag)
    compare("dk", dk, rk, tag)
    compare("dv", dv, rv, tag)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 128, 128, 2, 2), (2, 200, 333, 4, 2), (1, 77, 65, 8, 1),
                                   (1, 300, 129, 2, 1), (1, 129, 300, 4, 4)])
def test_bwd_small_full(ea, dtype, d, causal, shape):
    print(f"[case] bwd dtype={dtype} d={d} causal={causal} shape={shape}", flush=True)
    run_case(ea, shape, d, dtype, causal, seed=(shape[1] * 7 + shape[2] + d) % 10000)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_with_lse_gradient(ea, causal):
    print(f"[case] bwd dlse causal={causal}", flush=True)
    run_case(ea, (2, 150, 150, 4, 2), 128, "bf16", causal, seed=31, with_dlse=True)


def test_bwd_degenerate(ea):
    # one key: dQ = dK = 0 and dV = sum over queries of dO
    B, Sq, Sk, Hq, Hkv, d = 1, 50, 1, 2, 1, 64
    q, k, v, do, _, o, lse = grad_inputs(B, Sq, Sk, Hq, Hkv, d, "bf16", 32, False)
    dq, dk, dv = ea.bwd(*(t.cuda() for t in (q, k, v, o, lse, do)))
    torch.cuda.synchronize()
    # (P = exp(s - LSE) is 1 up to fp32 rounding, so dS = P (dP - delta) is a
    # rounding residue, not an exact 0)
    print(f"[parity] single key max|dq| {dq.abs().max().item():.3e} max|dk| {dk.abs().max().item():.3e}",
          flush=True)
    assert dq.abs().max().item() < 2e-3 and dk.abs().max().item() < 2e-3
    ref = do.double().sum(dim=(1, 2))                   # [B, d] summed over queries and the group
    np.testing.assert_allclose(dv[:, 0, 0].float().cpu().double().numpy(), ref.numpy(), rtol=1e-2, atol=1e-2)
    # causal with more keys than queries: keys past the last query get zero gradients
    B, Sq, Sk, Hq, Hkv, d = 1, 40, 300, 2, 2, 128
    q, k, v, do, _, o, lse = grad_inputs(B, Sq, Sk, Hq, Hkv, d, "bf16", 33, True)
    dq, dk, dv = ea.bwd(*(t.cuda() for t in (q, k, v, o, lse, do)), causal=True)
    torch.cuda.synchronize()
    assert torch.all(dk[:, 40:] == 0) and torch.all(dv[:, 40:] == 0)
    rq, rk, rv = A.attention_backward(q, k, v, do, 1 / math.sqrt(d), True)
    compare("dq", dq, rq, "causal Sk>Sq")
    compare("dk", dk, rk, "causal Sk>Sq")
    compare("dv", dv, rv, "causal Sk>Sq")


def test_bwd_end_to_end_with_gpu_forward(ea):
    # o and lse from the library's own forward
    B, S, Hq, Hkv, d = 2, 500, 8, 2, 128
    q, k, v = W.make_dense(B, S, S, Hq, Hkv, d, "bf16", seed=34)
    do = torch.randn(B, S, Hq, d, generator=torch.Generator().manual_seed(35)).to(torch.bfloat16)
    qc, kc, vc, gc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = ea.fwd(qc, kc, vc, causal=True)
    dq, dk, dv = ea.bwd(qc, kc, vc, o, lse, gc, causal=True)
    torch.cuda.synchronize()
    rq, rk, rv = A.attention_backward(q, k, v, do, 1 / math.sqrt(d), True)
    compare("dq", dq, rq, "end to end")
    compare("dk", dk, rk, "end to end")
    compare("dv", dv, rv, "end to end")


def test_bwd_deterministic(ea):
    B, S, Hq, Hkv, d = 1, 700, 4, 1, 128
    q, k, v, do, _, o, lse = grad_inputs(B, S, S, Hq, Hkv, d, "bf16", 36, True)
    dev = [t.cuda() for t in (q, k, v, o, lse, do)]
    a = ea.bwd(*dev, causal=True)
    b = ea.bwd(*dev, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("name", ["c2", "c3"])
def test_bwd_full_size_sampled(ea, name):
    # the full workload on the GPU (o, lse from the library's forward); the
    # oracle computes the gradients of one whole KV group (every query head
    # that reads that KV head, all rows and keys) of the last batch
    w = W.CONFIGS[name]
    inp = W.make_inputs(w)
    q, k, v = inp["q"], inp["k"], inp["v"]
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(w.seed_base + 7)).to(q.dtype)
    qc, kc, vc, gc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    print(f"[case] bwd full size {name}", flush=True)
    o, lse = ea.fwd(qc, kc, vc, causal=w.causal)
    dq, dk, dv = ea.bwd(qc, kc, vc, o, lse, gc, causal=w.causal)
    torch.cuda.synchronize()
    b, hkv = w.B - 1, w.Hkv - 1
    g = w.Hq // w.Hkv
    hs = list(range(hkv * g, (hkv + 1) * g))
    sl = lambda t, heads: t[b:b + 1, :, heads]
    rq, rk, rv = A.attention_backward(sl(q, hs), sl(k, [hkv]), sl(v, [hkv]), sl(do, hs), w.scale, w.causal)
    compare("dq", sl(dq, hs), rq, f"full {name}")
    compare("dk", sl(dk, [hkv]), rk, f"full {name}")
    compare("dv", sl(dv, [hkv]), rv, f"full {name}")


def varlen_inputs(lens, Hq, Hkv, d, dtype, seed, causal):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v = W.make_dense(1, T, T, Hq, Hkv, d, dtype, seed=seed)
    q, k, v = q[0], k[0], v[0]
    g = torch.Generator().manual_seed(seed + 1000)
    do = torch.randn(T, Hq, d, generator=g).to(q.dtype)
    o_ref, l_ref = A.attention(q, k, v, 1 / math.sqrt(d), causal, cu_seqlens=cu)
    return cu, q, k, v, do, torch.from_numpy(o_ref).to(q.dtype), torch.from_numpy(l_ref).float()


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lens", [[100, 0, 300, 1, 129], [256], [33, 500, 64]])
def test_bwd_varlen(ea, dtype, d, causal, lens):
    print(f"[case] bwd varlen dtype={dtype} d={d} causal={causal} lens={lens}", flush=True)
    cu, q, k, v, do, o, lse = varlen_inputs(lens, 4, 2, d, dtype, sum(lens) + d, causal)
    dev = [t.cuda() for t in (q, k, v, o, lse, do)]
    dq, dk, dv = ea.bwd(*dev, causal=causal, cu_seqlens=torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    rq, rk, rv = A.attention_backward(q, k, v, do, 1 / math.sqrt(d), causal, cu_seqlens=cu)
    tag = f"bwd varlen {dtype} d{d} c{int(causal)} {lens}"
    compare("dq", dq, rq, tag)
    compare("dk", dk, rk, tag)
    compare("dv", dv, rv, tag)


@pytest.mark.parametrize("case", ["many_sequences", "long_sequence"])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_varlen_block_order_fallbacks(ea, case, causal):
    # Both backward kernels rank (sequence, block) entries longest first for
    # at most 64 sequences of at most 64 blocks and walk the batch in order
    # beyond that; both sides of the limit, every gradient element compared.
    if case == "many_sequences":
        lens = [int(x) for x in np.random.default_rng(4).integers(0, 200, 70)]
        Hq, Hkv = 2, 1
    else:
        lens = [8321, 300, 5, 129]               # 66 blocks of 128 in the first
        Hq, Hkv = 1, 1
    print(f"[case] bwd varlen {case} causal={causal} B={len(lens)}", flush=True)
    cu, q, k, v, do, o, lse = varlen_inputs(lens, Hq, Hkv, 64, "fp16", 77, causal)
    dev = [t.cuda() for t in (q, k, v, o, lse, do)]
    dq, dk, dv = ea.bwd(*dev, causal=causal, cu_seqlens=torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    rq, rk, rv = A.attention_backward(q, k, v, do, 1 / 8, causal, cu_seqlens=cu)
    tag = f"bwd varlen {case} c{int(causal)}"
    compare("dq", dq, rq, tag)
    compare("dk", dk, rk, tag)
    compare("dv", dv, rv, tag)


def test_bwd_varlen_c4_sampled_heads(ea):
    # c4's packed batch (10 sequences, fp16, d = 64, causal): the GPU computes
    # every head, the oracle heads 0 and 15 over all sequences
    w = W.CONFIGS["c4"]
    inp = W.make_inputs(w)
    cu = inp["cu_seqlens"]
    q, k, v = inp["q"], inp["k"], inp["v"]
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(47)).to(q.dtype)
    cuc = torch.from_numpy(cu).cuda()
    qc, kc, vc, gc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    print("[case] bwd varlen c4", flush=True)
    o, lse = ea.fwd(qc, kc, vc, causal=True, cu_seqlens=cuc)
    dq, dk, dv = ea.bwd(qc, kc, vc, o, lse, gc, causal=True, cu_seqlens=cuc)
    torch.cuda.synchronize()
    for h in (0, 15):
        sl = lambda t: t[:, h:h + 1]
        rq, rk, rv = A.attention_backward(sl(q), sl(k), sl(v), sl(do), w.scale, True, cu_seqlens=cu)
        compare("dq", sl(dq), rq, f"c4 head {h}")
        compare("dk", sl(dk), rk, f"c4 head {h}")
        compare("dv", sl(dv), rv, f"c4 head {h}")


@pytest.mark.parametrize("dtype,d", [("fp16", 64), ("bf16", 128)])
def test_bwd_varlen_very_negative_lse(ea, dtype, d):
    # The first token of each sequence after the first has q = -4 k, so its
    # (causal) row sees only itself with a score near -4 sqrt(d): its LSE is
    # far below zero.  The dK/dV kernel's last step of the sequence before it
    # holds rows past that sequence's end, whose statistics slots hold the
    # next rows' pairs; those rows must get P = 0 (an exp2 of minus such an
    # LSE overflows the 16-bit P), and every gradient must match the oracle.
    lens = [100, 37, 300, 45]
    Hq, Hkv = 4, 2
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v = W.make_dense(1, T, T, Hq, Hkv, d, dtype, seed=91)
    q, k, v = q[0].float(), k[0].float(), v[0].float()
    for t0 in cu[1:-1]:
        for h in range(Hq):
            q[t0, h] = -4.0 * k[t0, h // (Hq // Hkv)]
    dt = W.TORCH_DTYPES[dtype]
    q, k, v = q.to(dt), k.to(dt), v.to(dt)
    g = torch.Generator().manual_seed(92)
    do = torch.randn(T, Hq, d, generator=g).to(dt)
    scale = 1 / math.sqrt(d)
    o_ref, l_ref = A.attention(q, k, v, scale, True, cu_seqlens=cu)
    lows = [float(l_ref[h, t0]) for t0 in cu[1:-1] for h in range(Hq)]
    print(f"[case] bwd varlen negative LSE {dtype} d={d}: first-token LSE {min(lows):.1f} .. {max(lows):.1f}",
          flush=True)
    assert max(lows) < -12.0
    o = torch.from_numpy(o_ref).to(dt)
    lse = torch.from_numpy(l_ref).float()
    dev = [t.cuda() for t in (q, k, v, o, lse, do)]
    dq, dk, dv = ea.bwd(*dev, causal=True, cu_seqlens=torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    rq, rk, rv = A.attention_backward(q, k, v, do, scale, True, cu_seqlens=cu)
    tag = f"bwd varlen negative LSE {dtype} d{d}"
    compare("dq", dq, rq, tag)
    compare("dk", dk, rk, tag)
    compare("dv", dv, rv, tag)
