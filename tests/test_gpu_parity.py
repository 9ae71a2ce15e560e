"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.

Tolerances (bf16/fp16): O max-abs <= 1e-2 and relative RMS <= 5e-3, LSE
abs <= 1e-3.  Small shapes are compared element by element in full; the
full-size workloads are compared on sampled (batch, head, row) sets that the
oracle computes row by row, chosen to cover the first and last query blocks,
ragged tails, every KV group and both lane halves of the tiles.
"""
import math

import numpy as np
import pytest
import torch

import rounding_bounds as RB
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


def compare(o_gpu, lse_gpu, o_ref, lse_ref, tag=""):
    o = o_gpu.detach().float().cpu().double().numpy()
    l = lse_gpu.detach().cpu().double().numpy()
    mask = ~np.isnan(o_ref)
    assert mask.any()
    diff = np.abs(o[mask] - o_ref[mask])
    maxabs = float(diff.max())
    relrms = float(np.sqrt((diff ** 2).sum() / (o_ref[mask] ** 2).sum()))
    lm = ~np.isnan(lse_ref)
    both_inf = np.isneginf(l[lm]) & np.isneginf(lse_ref[lm])
    ldiff = np.where(both_inf, 0.0, np.abs(l[lm] - lse_ref[lm]))
    lmax = float(ldiff.max())
    print(f"[parity] {tag} O max-abs {maxabs:.3e} rel-RMS {relrms:.3e} LSE max-abs {lmax:.3e}", flush=True)
    assert maxabs <= O_MAXABS, (tag, maxabs)
    assert relrms <= O_RELRMS, (tag, relrms)
    assert lmax <= LSE_ABS, (tag, lmax)


def check_bound(o_gpu, q, k, v, scale, causal, kind, rows, tag):
    """Every element of o_gpu (rows `rows` of a dense output) within the
    rounding bound of tests/rounding_bounds.py."""
    bound, o_ref = RB.rounding_bound(q, k, v, scale, causal, kind, rows)
    og = o_gpu.detach().float().cpu().double().numpy()
    err = np.abs(og - o_ref)
    ratio = float((err / bound).max())
    print(f"[bound] {tag}: max error / derived bound {ratio:.3f} (max-abs {err.max():.3e})", flush=True)
    assert ratio <= 1.0, (tag, ratio)


def run_dense(ea, q, k, v, causal, scale=None):
    o, lse = ea.fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


# ---------------------------------------------------------------- small full comparisons
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 333, 333, 4, 2), (1, 128, 128, 2, 2), (1, 77, 200, 3, 1),
                                   (1, 300, 65, 8, 2)])
def test_small_full(ea, dtype, d, causal, shape):
    B, Sq, Sk, Hq, Hkv = shape
    print(f"[case] small dtype={dtype} d={d} causal={causal} shape={shape}", flush=True)
    q, k, v = W.make_dense(B, Sq, Sk, Hq, Hkv, d, dtype, seed=hash((B, Sq, Sk, d)) % 10000)
    scale = 1 / math.sqrt(d)
    o, lse = run_dense(ea, q, k, v, causal)
    o_ref, l_ref = A.attention(q, k, v, scale, causal)
    compare(o, lse, o_ref, l_ref, f"small {dtype} d{d} c{int(causal)} {shape}")


@pytest.mark.parametrize("d", [64, 128])
def test_degenerate_shapes(ea, d):
    for (B, Sq, Sk, Hq, Hkv, causal) in [(1, 1, 1, 1, 1, False), (1, 1, 500, 2, 1, False),
                                         (1, 1, 500, 2, 1, True), (2, 130, 1, 2, 2, False),
                                         (1, 64, 64, 1, 1, True), (1, 129, 129, 4, 4, True)]:
        print(f"[case] degenerate d={d} {(B, Sq, Sk, Hq, Hkv, causal)}", flush=True)
        q, k, v = W.make_dense(B, Sq, Sk, Hq, Hkv, d, "bf16", seed=7)
        o, lse = run_dense(ea, q, k, v, causal)
        o_ref, l_ref = A.attention(q, k, v, 1 / math.sqrt(d), causal)
        compare(o, lse, o_ref, l_ref, f"degenerate {(B, Sq, Sk, Hq, Hkv, causal)}")


def test_single_key_and_identical_rows_exact(ea):
    # single key: O = V0 exactly after rounding; identical V rows: O = v exactly
    q, k, v = W.make_dense(1, 200, 1, 2, 2, 128, "bf16", seed=3)
    o, lse = run_dense(ea, q, k, v, False)
    assert torch.equal(o.cpu(), v.expand(1, 200, 2, 128))
    q, k, v = W.make_dense(1, 300, 300, 2, 1, 64, "bf16", seed=4)
    v = v[:, :1].expand(1, 300, 1, 64).contiguous()
    for causal in (False, True):
        o, _ = run_dense(ea, q, k, v, causal)
        assert torch.equal(o.cpu(), v[:, :1].expand(1, 300, 2, 64))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("path", ["wide", "wide_h4", "packgqa", "splitkv"])
def test_identical_v_rows(ea, dtype, causal, path):
    # identical V rows: the exact output is that row.  The kernels divide
    # sum_j Pt_j v by l = sum_j P_j (P rounded to the operand type only for
    # the product, l over the fp32 values), so O = v (sum Pt / sum P) before
    # the output rounding: the derived rounding bound, which for identical
    # rows is (u_P + eps) |v| + u_O |O| (plus the fp16 subnormal term).
    # wide: the one-wave-per-SIMD d = 128 kernel, one head per tile; wide_h4:
    # the same kernel with four query heads of a KV head per workgroup;
    # packgqa: rows of all heads of a KV group in one 128-row tile (4-wave
    # kernel); splitkv: key ranges and their combine.
    Hq, Hkv = (2, 2) if path == "wide" else (8, 2)
    Sq, Sk = (300, 700) if path in ("packgqa", "splitkv") else (700, 700)
    q, k, v = W.make_dense(1, Sq, Sk, Hq, Hkv, 128, dtype, seed=14)
    v = v[:, :1].expand(1, Sk, Hkv, 128).contiguous()
    scale = 1 / math.sqrt(128)
    print(f"[case] identical V rows {dtype} causal={causal} path={path}", flush=True)
    if path == "packgqa":
        o, lse = ea.fwd_splitkv(q.cuda(), k.cuda(), v.cuda(), causal=causal, num_splits=1, pack_gqa=True)
    elif path == "splitkv":
        o, lse = ea.fwd_splitkv(q.cuda(), k.cuda(), v.cuda(), causal=causal, num_splits=4, pack_gqa=False)
    else:
        o, lse = ea.fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal)
    torch.cuda.synchronize()
    want = v[:, :1].repeat_interleave(Hq // Hkv, dim=2).expand(1, Sq, Hq, 128)
    exact = float((o.cpu() == want).float().mean())
    print(f"[exact] identical V rows {dtype} c{int(causal)} {path}: {exact * 100:.2f}% of elements equal v", flush=True)
    check_bound(o, q, k, v, scale, causal, dtype, None, f"identical V rows {dtype} c{int(causal)} {path}")


def test_zero_q_gives_log_n(ea):
    q = torch.zeros(1, 300, 2, 128, dtype=torch.bfloat16)
    _, k, v = W.make_dense(1, 300, 300, 2, 2, 128, "bf16", seed=5)
    for causal in (False, True):
        o, lse = run_dense(ea, q, k, v, causal)
        n = np.arange(1, 301) if causal else np.full(300, 300)
        np.testing.assert_allclose(lse.cpu().numpy()[0], np.log(n)[None, :].repeat(2, 0), atol=1e-5)
        vm = v.double()
        ref = (vm.cumsum(1) / torch.arange(1, 301).view(1, -1, 1, 1)) if causal else vm.mean(1, keepdim=True)
        np.testing.assert_allclose(o.cpu().double().numpy(), ref.expand(1, 300, 2, 128).numpy(), atol=1e-2)


def test_scale_other_than_default(ea):
    q, k, v = W.make_dense(1, 200, 200, 2, 2, 64, "fp16", seed=8)
    o, lse = run_dense(ea, q, k, v, True, scale=0.3)
    o_ref, l_ref = A.attention(q, k, v, 0.3, True)
    compare(o, lse, o_ref, l_ref, "scale 0.3")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_running_max_moves(ea, dtype, causal, d):
    # channel 0 holds q = 1 and k = alpha * (128 * (j // 128)): every row's
    # scores step up by `step` log2 units at each 128-key boundary, so the
    # running max has to move again and again, by more than any lazy
    # threshold, while a row still averages the many keys of its last step.
    # Causal rows within 32 keys past a step boundary see only a few keys of
    # their top step: there the output is a mix of a handful of V rows and
    # the rounding of P to the operand type is not averaged away, so those
    # rows are gated by the bound derived from that rounding
    # (tests/rounding_bounds.py), the others by the standard gate; the LSE
    # gate holds for every row.
    B, S, Hq, Hkv = 1, 1100, 8, 2       # a group of 4: at d = 128 the head-packed wide kernel
    q, k, v = W.make_dense(B, S, S, Hq, Hkv, d, dtype, seed=12)
    scale = 1 / math.sqrt(d)
    rows = np.arange(S)
    few = rows[rows % 128 < 32] if causal else rows[:0]
    many = np.setdiff1d(rows, few)
    for step in (20.0, 60.0):
        alpha = step / (scale * math.log2(math.e) * 128)
        q2, k2 = q.clone(), k.clone()
        q2[..., 0] = 1.0
        k2[..., 0] = (alpha * 128 * (torch.arange(S, dtype=torch.float64) // 128)).view(1, S, 1).to(k.dtype)
        print(f"[case] running max moves {dtype} d={d} causal={causal} step={step}", flush=True)
        o, lse = run_dense(ea, q2, k2, v, causal)
        o_ref, l_ref = A.attention(q2, k2, v, scale, causal)
        compare(o[:, many], lse[:, :, many], o_ref[:, many], l_ref[:, :, many],
                f"max moves {dtype} d{d} c{int(causal)} step {step}")
        if len(few):
            check_bound(o[:, few], q2, k2, v, scale, causal, dtype, few,
                        f"max moves {dtype} d{d} c{int(causal)} step {step} few-key rows")
            lg = lse.cpu().double().numpy()[:, :, few]
            assert float(np.abs(lg - l_ref[:, :, few]).max()) <= LSE_ABS


def test_deterministic(ea):
    q, k, v = W.make_dense(2, 1000, 1000, 4, 2, 128, "bf16", seed=9)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    o1, l1 = ea.fwd(qc, kc, vc, causal=True)
    o2, l2 = ea.fwd(qc, kc, vc, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---------------------------------------------------------------- varlen
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_varlen_small(ea, dtype, d):
    lengths = [5, 0, 130, 1, 257, 64, 200]
    print(f"[case] varlen small {dtype} d={d}", flush=True)
    q, k, v, cu = W.make_varlen(lengths, 4, 2, d, dtype, seed=11)
    for causal in (False, True):
        o, lse = ea.fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal,
                        cu_seqlens=torch.from_numpy(cu).cuda())
        torch.cuda.synchronize()
        o_ref, l_ref = A.attention(q, k, v, 1 / math.sqrt(d), causal, cu_seqlens=cu)
        compare(o, lse, o_ref, l_ref, f"varlen {dtype} d{d} c{int(causal)}")


@pytest.mark.parametrize("case", ["many_sequences", "long_sequence"])
def test_varlen_block_order_fallbacks(ea, case):
    # The kernel ranks (sequence, block) entries longest first when there are
    # at most 64 sequences of at most 64 blocks; beyond that it walks the
    # batch in order.  Both sides of that limit, every row compared.
    if case == "many_sequences":
        lengths = [int(x) for x in np.random.default_rng(3).integers(0, 300, 70)]
        Hq, Hkv, d = 2, 1, 64
    else:
        lengths = [8321, 300, 5, 129]          # 66 blocks of 128 rows in the first
        Hq, Hkv, d = 1, 1, 64
    print(f"[case] varlen {case} B={len(lengths)} T={sum(lengths)}", flush=True)
    q, k, v, cu = W.make_varlen(lengths, Hq, Hkv, d, "fp16", seed=17)
    for causal in (False, True):
        o, lse = ea.fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal,
                        cu_seqlens=torch.from_numpy(cu).cuda())
        torch.cuda.synchronize()
        o_ref, l_ref = A.attention(q, k, v, 1 / math.sqrt(d), causal, cu_seqlens=cu)
        compare(o, lse, o_ref, l_ref, f"varlen {case} c{int(causal)}")


# ---------------------------------------------------------------- the five workloads
def sampled_rows(S, n=40, seed=0):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, S // 2, S - 129, S - 65, S - 33, S - 2, S - 1]
    rows = set(r for r in fixed if 0 <= r < S) | set(rng.integers(0, S, n).tolist())
    return np.array(sorted(rows))


def test_c1(ea):
    w = W.CONFIGS["c1"]
    inp = W.make_inputs(w)
    o, lse = run_dense(ea, inp["q"], inp["k"], inp["v"], w.causal)
    o_ref, l_ref = A.attention(inp["q"], inp["k"], inp["v"], w.scale, w.causal)
    compare(o, lse, o_ref, l_ref, "c1 full")


@pytest.mark.parametrize("name", ["c2", "c3"])
def test_dense_workload_sampled(ea, name):
    w = W.CONFIGS[name]
    print(f"[case] {name} full size, sampled rows", flush=True)
    inp = W.make_inputs(w)
    o, lse = run_dense(ea, inp["q"], inp["k"], inp["v"], w.causal)
    rows = sampled_rows(w.Sq)
    group = w.Hq // w.Hkv
    heads = sorted(set([0, w.Hq - 1] + [g * group + (g % group) for g in range(w.Hkv)]))
    for b in range(w.B):
        o_ref, l_ref = A.attention(inp["q"], inp["k"], inp["v"], w.scale, w.causal,
                                   heads=heads, rows=rows, batches=[b])
        compare(o[b:b + 1], lse[b:b + 1], o_ref[b:b + 1], l_ref[b:b + 1], f"{name} b{b} sampled")


def test_c2_full_heads(ea):
    # c2: every row of three heads compared in full
    w = W.CONFIGS["c2"]
    inp = W.make_inputs(w)
    o, lse = run_dense(ea, inp["q"], inp["k"], inp["v"], w.causal)
    for b, h in [(0, 0), (3, 15), (1, 7)]:
        o_ref, l_ref = A.attention(inp["q"], inp["k"], inp["v"], w.scale, w.causal, heads=[h], batches=[b])
        compare(o[b:b + 1, :, h:h + 1], lse[b:b + 1, h:h + 1], o_ref[b:b + 1, :, h:h + 1],
                l_ref[b:b + 1, h:h + 1], f"c2 b{b} h{h} full")


@pytest.mark.parametrize("shape,causal", [
    ((1, 2560, 2560, 32, 8), True),    # 8 KV groups x 40 blocks = 320 tiles, XCD affinity
    ((1, 2560, 2560, 32, 8), False),   # the same, full attention (groups one after another)
    ((3, 3200, 3200, 8, 2), True),     # 6 KV groups (no even XCD split) x 50 blocks = 300 tiles
    ((1, 2500, 2500, 32, 8), True),    # ragged last block (2500 = 39 x 64 + 4)
    ((2, 1600, 1600, 64, 8), True),    # group 8: two head quadruples per KV head, 800 tiles
    ((1, 2100, 3000, 32, 8), False),   # Sq != Sk, ragged key tail
])
def test_persistent_head_packed(ea, shape, causal):
    # d = 128 with groups of four query heads runs the head-packed wide
    # kernel; with more 64-row tiles than compute units each workgroup runs
    # several tiles in turn (the next tile's Q loaded during the last P V,
    # the finished tile's epilogue after the next tile's first iteration):
    # every output element against the oracle
    B, Sq, Sk, Hq, Hkv = shape
    print(f"[case] persistent head-packed B={B} Sq={Sq} Sk={Sk} Hq={Hq} Hkv={Hkv} causal={causal}", flush=True)
    q, k, v = W.make_dense(B, Sq, Sk, Hq, Hkv, 128, "bf16", seed=31 + B + Sq % 97)
    o, lse = run_dense(ea, q, k, v, causal)
    scale = 1 / math.sqrt(128)
    o_ref, l_ref = A.attention(q, k, v, scale, causal)
    tag = f"persistent B{B} Sq{Sq} Sk{Sk} Hq{Hq} Hkv{Hkv} c{int(causal)}"
    # relative RMS and LSE against the flat gates; the rows whose elements
    # come near the flat max-abs gate (causal rows that see few keys, where
    # the rounding of P and of O is a visible share of |O|) element by
    # element against the derived rounding bound
    og = o.float().cpu().double().numpy()
    err = np.abs(og - o_ref)
    relrms = float(np.sqrt((err ** 2).sum() / (o_ref ** 2).sum()))
    lerr = float(np.abs(lse.cpu().double().numpy() - l_ref).max())
    print(f"[parity] {tag} O max-abs {err.max():.3e} rel-RMS {relrms:.3e} LSE max-abs {lerr:.3e}", flush=True)
    assert relrms <= O_RELRMS, (tag, relrms)
    assert lerr <= LSE_ABS, (tag, lerr)
    rows = np.unique(np.nonzero(err > 0.5 * O_MAXABS)[1])
    if len(rows):
        check_bound(o[:, rows], q, k, v, scale, causal, "bf16", rows, f"{tag} rows near the flat gate")


def test_c4_varlen(ea):
    w = W.CONFIGS["c4"]
    inp = W.make_inputs(w)
    cu = inp["cu_seqlens"]
    o, lse = ea.fwd(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), causal=True,
                    cu_seqlens=torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    # all sequences, heads 0, 5 and 15 in full
    for h in (0, 5, 15):
        o_ref, l_ref = A.attention(inp["q"][:, h:h + 1], inp["k"][:, h:h + 1], inp["v"][:, h:h + 1],
                                   w.scale, True, cu_seqlens=cu)
        compare(o[:, h:h + 1], lse[h:h + 1], o_ref, l_ref, f"c4 head {h}")
