"""GPU parity of split-KV (flash-decoding), the combine kernel and PackGQA, through the
C ABI, against the fp64 oracle on the same seeded inputs.

attn_fwd_splitkv must give the attention over all keys (the oracle's
``attention``) within the bf16/fp16 tolerances, for every number of key
ranges, causal or not, with GQA, ragged key counts, few query rows and ranges
that some query blocks never see.  attn_combine is checked on its own against
the oracle's ``combine`` of oracle partials, including partials with
LSE = -inf and rows whose partials are all -inf.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
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


def compare(o_gpu, lse_gpu, o_ref, lse_ref, tag):
    o = o_gpu.detach().float().cpu().double().numpy()
    l = lse_gpu.detach().cpu().double().numpy()
    assert not np.isnan(o).any(), tag
    diff = np.abs(o - o_ref)
    maxabs = float(diff.max())
    den = float((o_ref ** 2).sum())
    relrms = float(np.sqrt((diff ** 2).sum() / den)) if den > 0 else float(np.sqrt((diff ** 2).sum()))
    both_inf = np.isneginf(l) & np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(l), np.isneginf(lse_ref)), tag
    with np.errstate(invalid="ignore"):
        ldiff = np.where(both_inf, 0.0, np.abs(l - lse_ref))
    lmax = float(ldiff.max())
    print(f"[parity] {tag} O max-abs {maxabs:.3e} rel-RMS {relrms:.3e} LSE max-abs {lmax:.3e}", flush=True)
    assert maxabs <= O_MAXABS, (tag, maxabs)
    assert relrms <= O_RELRMS, (tag, relrms)
    assert lmax <= LSE_ABS, (tag, lmax)


def splitkv(ea, q, k, v, causal, n, scale=None, pack=None):
    o, lse = ea.fwd_splitkv(q.cuda(), k.cuda(), v.cuda(), causal=causal, num_splits=n, scale=scale,
                            pack_gqa=pack)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [2, 3, 7, 0])
@pytest.mark.parametrize("pack", [None, False])
@pytest.mark.parametrize("shape", [(2, 1, 1000, 8, 2), (1, 3, 777, 4, 4), (1, 130, 4100, 4, 1)])
def test_splitkv_small_full(ea, dtype, d, causal, n, pack, shape):
    B, Sq, Sk, Hq, Hkv = shape
    plan = ea.split_plan(B, Hq, Hkv, Sq, Sk, d=d, num_splits=n, pack_gqa=pack)
    print(f"[case] splitkv dtype={dtype} d={d} causal={causal} n={n} pack={pack} shape={shape} plan={plan}",
          flush=True)
    q, k, v = W.make_dense(B, Sq, Sk, Hq, Hkv, d, dtype, seed=(Sq * 31 + Sk + d) % 10000)
    o, lse = splitkv(ea, q, k, v, causal, n, pack=pack)
    o_ref, l_ref = A.attention(q, k, v, 1 / math.sqrt(d), causal)
    compare(o, lse, o_ref, l_ref, f"splitkv {dtype} d{d} c{int(causal)} n{n} pack{pack} {shape}")


# ---------------------------------------------------------------- PackGQA
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 1, 1000, 8, 2), (1, 3, 777, 8, 1), (1, 30, 500, 16, 4),
                                   (3, 5, 130, 32, 2), (1, 1, 300, 128, 1)])
def test_packgqa_plain_forward(ea, dtype, d, causal, shape):
    # few query positions with GQA: attn_fwd packs the group's heads into one
    # tile on its own (checked with the plan)
    B, Sq, Sk, Hq, Hkv = shape
    assert ea.split_plan(B, Hq, Hkv, Sq, Sk, d=d, num_splits=1)[2], shape
    print(f"[case] packgqa fwd dtype={dtype} d={d} causal={causal} shape={shape}", flush=True)
    q, k, v = W.make_dense(B, Sq, Sk, Hq, Hkv, d, dtype, seed=(Sq * 7 + Sk + Hq) % 10000)
    o, lse = ea.fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal)
    torch.cuda.synchronize()
    o_ref, l_ref = A.attention(q, k, v, 1 / math.sqrt(d), causal)
    compare(o, lse, o_ref, l_ref, f"packgqa fwd {dtype} d{d} c{int(causal)} {shape}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 4])
@pytest.mark.parametrize("shape", [(1, 300, 300, 8, 2), (2, 257, 600, 16, 2), (1, 1000, 1000, 4, 1)])
def test_packgqa_forced_many_tiles(ea, d, causal, n, shape):
    # packing forced on shapes with many packed tiles: causal masks across
    # tiles whose rows mix positions and heads, ragged last tile, with and
    # without split-KV
    B, Sq, Sk, Hq, Hkv = shape
    plan = ea.split_plan(B, Hq, Hkv, Sq, Sk, d=d, num_splits=n, pack_gqa=True)
    assert plan[2]
    print(f"[case] packgqa forced d={d} causal={causal} n={n} shape={shape} plan={plan}", flush=True)
    q, k, v = W.make_dense(B, Sq, Sk, Hq, Hkv, d, "bf16", seed=(Sq + Sk + d + n) % 10000)
    o, lse = splitkv(ea, q, k, v, causal, n, pack=True)
    o_ref, l_ref = A.attention(q, k, v, 1 / math.sqrt(d), causal)
    compare(o, lse, o_ref, l_ref, f"packgqa forced d{d} c{int(causal)} n{n} {shape}")


def test_packgqa_identical_v_rows_exact(ea):
    # identical V rows in every KV head: O = v of the query's KV head exactly,
    # with the group's heads packed into one tile
    q, k, v = W.make_dense(2, 2, 700, 16, 2, 128, "bf16", seed=21)
    v = v[:, :1].expand(2, 700, 2, 128).contiguous()
    for causal in (False, True):
        o, _ = ea.fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal)
        torch.cuda.synchronize()
        want = v[:, :1].repeat_interleave(8, dim=2).expand(2, 2, 16, 128)
        assert torch.equal(o.cpu(), want)


@pytest.mark.parametrize("n", [2, 5, 16])
def test_splitkv_causal_ranges_beyond_the_block(ea, n):
    # Sq == Sk causal: early query blocks see no key of the late ranges, so
    # their partials are all -inf and the combine must skip them
    B, S, Hq, Hkv, d = 1, 1000, 4, 2, 128
    q, k, v = W.make_dense(B, S, S, Hq, Hkv, d, "bf16", seed=11)
    print(f"[case] splitkv causal square n={n}", flush=True)
    o, lse = splitkv(ea, q, k, v, True, n)
    o_ref, l_ref = A.attention(q, k, v, 1 / math.sqrt(d), True)
    compare(o, lse, o_ref, l_ref, f"splitkv causal square n{n}")


def test_splitkv_decode_shape(ea):
    # one query row per sequence, GQA 4:1, long keys: the shape split-KV is for
    B, Sq, Sk, Hq, Hkv, d = 4, 1, 16384, 32, 8, 128
    q, k, v = W.make_dense(B, Sq, Sk, Hq, Hkv, d, "bf16", seed=12)
    for causal in (False, True):
        for pack in (None, False):
            print(f"[case] splitkv decode causal={causal} plan={ea.split_plan(B, Hq, Hkv, Sq, Sk, d=d, pack_gqa=pack)}",
                  flush=True)
            o, lse = splitkv(ea, q, k, v, causal, 0, pack=pack)
            o_ref, l_ref = A.attention(q, k, v, 1 / math.sqrt(d), causal)
            compare(o, lse, o_ref, l_ref, f"splitkv decode c{int(causal)} pack{pack}")


def test_fwd_splits_the_decode_shape(ea):
    # attn_fwd on a decode shape (the plain launch would hold 32 workgroups,
    # 16384 keys) follows attn_fwd_splitkv's own plan: the same kernels, so
    # the same bits; a shape with a full grid keeps the plain kernel
    B, Sq, Sk, Hq, Hkv, d = 4, 1, 16384, 32, 8, 128
    q, k, v = W.make_dense(B, Sq, Sk, Hq, Hkv, d, "bf16", seed=16)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    o1, l1 = ea.fwd(qc, kc, vc)
    o2, l2 = ea.fwd_splitkv(qc, kc, vc, num_splits=0)
    torch.cuda.synchronize()
    assert ea.split_plan(B, Hq, Hkv, Sq, Sk, d=d)[0] > 1
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o_ref, l_ref = A.attention(q, k, v, 1 / math.sqrt(d), False)
    compare(o1, l1, o_ref, l_ref, "attn_fwd decode shape")


def test_splitkv_one_range_is_the_plain_forward(ea):
    q, k, v = W.make_dense(1, 300, 300, 2, 2, 64, "fp16", seed=13)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    o1, l1 = ea.fwd_splitkv(qc, kc, vc, causal=True, num_splits=1, pack_gqa=False)
    o2, l2 = ea.fwd(qc, kc, vc, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_splitkv_identical_rows_and_zero_q(ea):
    # identical V rows: every partial is v, so O = v exactly after rounding
    q, k, v = W.make_dense(1, 5, 2000, 2, 1, 128, "bf16", seed=14)
    v = v[:, :1].expand(1, 2000, 1, 128).contiguous()
    o, _ = splitkv(ea, q, k, v, False, 6)
    assert torch.equal(o.cpu(), v[:, :1].expand(1, 5, 2, 128))
    # zero Q: LSE = log Sk whatever the ranges
    q = torch.zeros(1, 5, 2, 128, dtype=torch.bfloat16)
    _, lse = splitkv(ea, q, k, v, False, 6)
    np.testing.assert_allclose(lse.cpu().numpy(), np.full((1, 2, 5), math.log(2000)), atol=1e-5)


def test_splitkv_deterministic(ea):
    q, k, v = W.make_dense(2, 3, 5000, 8, 2, 128, "bf16", seed=15)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    o1, l1 = ea.fwd_splitkv(qc, kc, vc, num_splits=9)
    o2, l2 = ea.fwd_splitkv(qc, kc, vc, num_splits=9)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---------------------------------------------------------------- combine alone
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("d", [64, 128])
def test_combine_oracle_partials(ea, dtype, d):
    # partials of the oracle over uneven key ranges, merged on the GPU, must
    # give the oracle's attention over all keys (and the oracle's combine)
    B, Sq, Sk, Hq, Hkv = 2, 70, 900, 4, 2
    name = "bf16" if dtype == torch.bfloat16 else "fp16"
    q, k, v = W.make_dense(B, Sq, Sk, Hq, Hkv, d, name, seed=16 + d)
    bounds = [0, 10, 300, 301, 650, 900]
    for causal in (False, True):
        parts = [A.partial_attention(q, k, v, 1 / math.sqrt(d), causal, lo, hi)
                 for lo, hi in zip(bounds[:-1], bounds[1:])]
        op = torch.tensor(np.stack([p[0] for p in parts]), dtype=torch.float32)
        lp = torch.tensor(np.stack([p[1] for p in parts]), dtype=torch.float32)
        print(f"[case] combine oracle partials d={d} causal={causal} -inf parts "
              f"{int(np.isneginf(lp.numpy()).sum())}", flush=True)
        o, lse = ea.combine(op.cuda(), lp.cuda(), dtype=dtype)
        torch.cuda.synchronize()
        o_ref, l_ref = A.attention(q, k, v, 1 / math.sqrt(d), causal)
        compare(o, lse, o_ref, l_ref, f"combine d{d} c{int(causal)}")
        o_c, l_c = A.combine(op.double().numpy(), lp.double().numpy())
        compare(o, lse, o_c, l_c, f"combine vs oracle combine d{d} c{int(causal)}")


def test_combine_random_partials_with_empty_rows(ea):
    g = torch.Generator().manual_seed(17)
    P, B, Sq, Hq, d = 7, 2, 33, 3, 128
    op = torch.randn(P, B, Sq, Hq, d, generator=g) * 0.5   # |O| < 4: bf16 half-ulp below 1e-2
    lp = torch.randn(P, B, Hq, Sq, generator=g) * 30.0
    drop = torch.rand(P, B, Hq, Sq, generator=g) < 0.3
    lp[drop] = -math.inf
    lp[:, 1, 2, 5] = -math.inf          # a row no partial saw
    lp[:, 0, 0, 7] = -math.inf
    lp[3, 0, 0, 7] = 12.5               # a row only one partial saw
    op[torch.isneginf(lp).permute(0, 1, 3, 2)] = float("nan")   # partials with LSE -inf are never read
    o, lse = ea.combine(op.cuda(), lp.cuda(), dtype=torch.bfloat16)
    torch.cuda.synchronize()
    o_ref, l_ref = A.combine(op.double().numpy(), lp.double().numpy())
    compare(o, lse, o_ref, l_ref, "combine random")
    # many partials (the most attn_combine takes), d = 64, fp16
    P2 = 256
    op2 = torch.randn(P2, 1, 5, 2, 64, generator=g) * 0.5
    lp2 = torch.randn(P2, 1, 2, 5, generator=g) * 3.0
    lp2[:200, 0, 1, 3] = -math.inf
    o2, l2 = ea.combine(op2.cuda(), lp2.cuda(), dtype=torch.float16)
    torch.cuda.synchronize()
    o2_ref, l2_ref = A.combine(op2.double().numpy(), lp2.double().numpy())
    compare(o2, l2, o2_ref, l2_ref, "combine 256 partials")
    assert torch.all(o[1, 5, 2] == 0) and math.isinf(lse[1, 2, 5].item())
    assert torch.equal(o[0, 7, 0].cpu(), op[3, 0, 7, 0].to(torch.bfloat16))
