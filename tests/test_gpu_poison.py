"""LDS-stage poisoning: the debug build (libattn_poison.so, compiled with
-DATTN_DEBUG_POISON) fills every LDS stage with NaN right before the copy that
refills it, i.e. as soon as the barrier that ends the stage's last reads has
released it.  A kernel that read a stage after its release would then see NaN
at once, where the normal build still finds the old tile's values until the
copy lands and so hides the race.  Each kernel family runs here through both
builds on the same inputs: the outputs must be finite and bit-identical (the
poisoning changes no arithmetic, only the timing).
"""

import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_75_amd as m
    m.library()
    return m


@pytest.fixture(scope="module")
def poison(ea):
    return ea.load_library(ea.POISON_LIB_PATH)


def same_in_both(ea, poison, fn, tag):
    """Run fn with the normal library, then with the poisoning one; every
    output must be NaN-free and bit-identical."""
    a = fn()
    torch.cuda.synchronize()
    prev = ea.use_library(poison)
    try:
        b = fn()
        torch.cuda.synchronize()
    finally:
        ea.use_library(prev)
    a = [t for t in a if t is not None]
    b = [t for t in b if t is not None]
    assert len(a) == len(b)
    for i, (x, y) in enumerate(zip(a, b)):
        assert not torch.isnan(x.float()).any(), (tag, i, "normal build")
        assert not torch.isnan(y.float()).any(), (tag, i, "poisoned build")
        assert torch.equal(x, y), (tag, i, float((x.float() - y.float()).abs().max()))
    print(f"[poison] {tag}: {len(a)} outputs bit-identical", flush=True)


def dense(B, Sq, Sk, Hq, Hkv, d, dtype="bf16", seed=700):
    return [t.cuda() for t in W.make_dense(B, Sq, Sk, Hq, Hkv, d, dtype, seed=seed)]


# wide kernel (d = 128 dense): one tile per workgroup, head-packed, and the
# persistent head-packed walk (more tiles than compute units); 8-wave and
# 4-wave kernels (d = 64)
@pytest.mark.parametrize("shape", [(1, 1000, 1000, 2, 2, 128), (1, 777, 1200, 8, 2, 128),
                                   (1, 2560, 2560, 32, 8, 128), (2, 700, 700, 4, 2, 64)])
@pytest.mark.parametrize("causal", [True, False])
def test_forward_dense(ea, poison, shape, causal):
    q, k, v = dense(*shape)
    same_in_both(ea, poison, lambda: ea.fwd(q, k, v, causal=causal), f"fwd {shape} causal={causal}")


@pytest.mark.parametrize("d,dtype", [(64, "fp16"), (128, "bf16")])
@pytest.mark.parametrize("causal", [True, False])
def test_forward_varlen(ea, poison, d, dtype, causal):
    q, k, v, cu = W.make_varlen([300, 1000, 77, 2000], 4, 2, d, dtype, seed=701)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    cu = torch.from_numpy(cu).cuda()
    same_in_both(ea, poison, lambda: ea.fwd(q, k, v, causal=causal, cu_seqlens=cu),
                 f"varlen d={d} causal={causal}")


@pytest.mark.parametrize("softcap,vcol", [(30.0, False), (0.0, True), (30.0, True)])
def test_forward_options(ea, poison, softcap, vcol):
    q, k, v = dense(1, 1000, 1000, 8, 2, 128, seed=702)   # column-major V needs Sk % 8 == 0
    vv = v.permute(0, 2, 3, 1).contiguous() if vcol else v
    same_in_both(ea, poison, lambda: ea.fwd_ext(q, k, vv, causal=True, softcap=softcap, v_colmajor=vcol),
                 f"options softcap={softcap} vcol={vcol}")


def test_splitkv(ea, poison):
    q, k, v = dense(4, 1, 5000, 32, 8, 128, seed=703)
    same_in_both(ea, poison, lambda: ea.fwd_splitkv(q, k, v), "split-KV decode")


@pytest.mark.parametrize("dtype", ["fp8", "fp8_hadamard"])
@pytest.mark.parametrize("causal", [True, False])
def test_fp8(ea, poison, dtype, causal):
    q, k, v = dense(1, 704, 704, 4, 2, 128, dtype="fp8", seed=704)   # fp32 inputs; fp8 needs Sk % 16 == 0
    same_in_both(ea, poison, lambda: ea.fwd(q, k, v, causal=causal, dtype=dtype), f"{dtype} causal={causal}")


@pytest.mark.parametrize("shape", [(1, 1000, 1000, 4, 2, 128), (1, 700, 700, 4, 2, 64)])
@pytest.mark.parametrize("causal", [True, False])
def test_backward_dense(ea, poison, shape, causal):
    q, k, v = dense(*shape, seed=705)
    o, lse = ea.fwd(q, k, v, causal=causal)
    g = torch.Generator().manual_seed(706)
    do = torch.randn(q.shape, generator=g).to(q.dtype).cuda()
    same_in_both(ea, poison, lambda: ea.bwd(q, k, v, o, lse, do, causal=causal),
                 f"bwd {shape} causal={causal}")


@pytest.mark.parametrize("d,dtype", [(64, "fp16"), (128, "bf16")])
def test_backward_varlen(ea, poison, d, dtype):
    q, k, v, cu = W.make_varlen([300, 1000, 77, 600], 4, 2, d, dtype, seed=707)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    cu = torch.from_numpy(cu).cuda()
    o, lse = ea.fwd(q, k, v, causal=True, cu_seqlens=cu)
    g = torch.Generator().manual_seed(708)
    do = torch.randn(q.shape, generator=g).to(q.dtype).cuda()
    same_in_both(ea, poison, lambda: ea.bwd(q, k, v, o, lse, do, causal=True, cu_seqlens=cu),
                 f"bwd varlen d={d}")
