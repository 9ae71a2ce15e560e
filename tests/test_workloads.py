"""The seeded input recipe: shapes, dtypes and the varlen length draw."""
import numpy as np
import torch

import workloads as W


def test_varlen_lengths_seed0():
    L = W.varlen_lengths()
    assert L == [3561, 2795, 2344, 1479, 1615, 658, 781, 571, 1140, 1440]
    assert sum(L) == 16384
    cu = W.cu_seqlens_from_lengths(L)
    assert cu[0] == 0 and cu[-1] == 16384 and cu.dtype == np.int32


def test_inputs_are_rounded_normal_draws():
    w = W.CONFIGS["c1"]
    inp = W.make_inputs(w)
    assert inp["q"].shape == (1, 256, 2, 64) and inp["q"].dtype == torch.bfloat16
    g = torch.Generator().manual_seed(10)
    ref = torch.randn(1, 256, 2, 64, generator=g).to(torch.bfloat16)
    assert torch.equal(inp["q"], ref)
    again = W.make_inputs(w)
    assert torch.equal(again["k"], inp["k"]) and not torch.equal(inp["k"], inp["v"])


def test_outlier_channels_and_signs():
    ch = W.outlier_channels()
    assert sorted(ch.tolist()) == [2, 83, 101, 103]
    s = W.hadamard_signs()
    assert s.shape == (128,) and set(np.unique(s).tolist()) == {-1.0, 1.0}
    assert 40 < (s > 0).sum() < 88
    # splitmix64 with seed 0: the first output (state = golden gamma) is 0xE220A8397B1DCDAF
    assert W.splitmix64(1) == 0xE220A8397B1DCDAF


def test_c5_outliers_scaled():
    w = W.Workload("t", B=1, Hq=2, Hkv=2, Sq=256, Sk=256, d=128, dtype="fp8", causal=False,
                   outliers=True, seed_base=50)
    inp = W.make_inputs(w)
    q = inp["q"]
    assert q.dtype == torch.float32
    ch = W.outlier_channels()
    big = q[..., ch].abs().mean()
    small = q.abs().mean()
    assert big > 10 * small


def test_flop_counts_match_the_oracle_rule():
    # the bench's counting rule (workloads) equals the oracle's on every
    # workload, so the throughput figures and the oracle agree on the work
    from oracle.attention import attention_backward_flops, attention_flops
    for name, w in W.CONFIGS.items():
        if w.varlen:
            lengths = W.varlen_lengths(total=w.Sq)
            assert W.forward_flops(w) == attention_flops(0, 0, w.d, w.causal, H=w.Hq, lengths=lengths)
        else:
            assert W.forward_flops(w) == attention_flops(w.Sq, w.Sk, w.d, w.causal, B=w.B, H=w.Hq)
            assert W.backward_flops(w) == attention_backward_flops(w.Sq, w.Sk, w.d, w.causal, B=w.B, H=w.Hq)
    assert W.forward_flops(W.CONFIGS["c3"]) == 1099645845504.0
