"""attn_fwd_splitkv_noalloc through the C ABI: the entry point for callers
that cannot allocate (its split-KV partials live in a fixed device array
instead of the library's lazily grown workspace).  Its output must equal
attn_fwd_splitkv's on the same inputs and plan -- same kernels, so bit for
bit -- on two calls in a row, the second with a smaller input (the scratch
keeps the first call's partials, which the second must not read), and a
plan beyond the scratch is refused without writing anything."""
import ctypes

import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_75_amd as m
    return m.library()


def call(lib, fn, q, k, v, causal, splits, pack):
    B, Sq, Hq, d = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    o = torch.full(q.shape, float("nan"), dtype=q.dtype, device="cuda")
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device="cuda")
    dt = 0 if q.dtype == torch.bfloat16 else 1
    rc = getattr(lib, fn)(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Sq, Sk,
                          d, ctypes.c_float(d ** -0.5), int(causal), splits, pack, dt,
                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return rc, o, lse


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_noalloc_equals_splitkv_twice(lib, dtype):
    # first the decode shape (B=4 Hq=32 Hkv=8, one query over 16384 keys,
    # library plan: 8 ranges, packed), then a smaller input with a causal
    # prefill-like block and 4 forced ranges
    cases = [((4, 1, 16384, 32, 8, 128), False, 0, -1, 61),
             ((2, 200, 3000, 8, 2, 64), True, 4, 0, 62)]
    for (B, Sq, Sk, Hq, Hkv, d), causal, splits, pack, seed in cases:
        print(f"[case] noalloc {dtype} B={B} Sq={Sq} Sk={Sk} Hq={Hq} Hkv={Hkv} d={d} causal={causal}", flush=True)
        q, k, v = (t.cuda() for t in W.make_dense(B, Sq, Sk, Hq, Hkv, d, dtype, seed=seed))
        rc1, o1, l1 = call(lib, "attn_fwd_splitkv", q, k, v, causal, splits, pack)
        rc2, o2, l2 = call(lib, "attn_fwd_splitkv_noalloc", q, k, v, causal, splits, pack)
        assert rc1 == 0 and rc2 == 0
        assert not torch.isnan(o2.float()).any()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_noalloc_refuses_beyond_scratch_and_writes_nothing(lib):
    q, k, v = (t.cuda() for t in W.make_dense(64, 32, 1024, 32, 8, 128, "bf16", seed=63))
    rc, o, lse = call(lib, "attn_fwd_splitkv_noalloc", q, k, v, False, 16, 0)
    assert rc == -10
    assert torch.isnan(o.float()).all() and torch.isnan(lse).all()
