"""The C-ABI boundary without a GPU: the library loads, exports every entry
point the header declares, rejects bad arguments before touching the device,
and its tile scheduler is a bijection with the documented order."""
import ctypes
import os
import re

import pytest

import exact_attention_75_amd as ea
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x1000  # never dereferenced: every call below fails validation first


def header_functions():
    src = open(os.path.join(ROOT, "include", "attn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(attn_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ea.LIB_PATH):
        pytest.skip("libattn.so not built")
    return ea.library()


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert {"attn_fwd", "attn_fp8_prepass", "attn_fwd_fp8", "attn_strerror", "attn_release"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_poisoning_debug_build_exports_and_validates():
    """The LDS-poisoning debug library (build --poison) exports the same
    entry points and validates like the normal one."""
    if not os.path.exists(ea.POISON_LIB_PATH):
        pytest.skip("libattn_poison.so not built")
    L = ea.load_library(ea.POISON_LIB_PATH)
    for n in header_functions():
        assert hasattr(L, n), n
    assert fwd(L, d=96) == -3
    assert fwd(L, q=None) == -1


def fwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, Hq=2, Hkv=2, Sq=256, Sk=256, d=64,
             scale=0.125, causal=0, cu=None, dtype=0)
    a.update(kw)
    return lib.attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Sq"],
                        a["Sk"], a["d"], a["scale"], a["causal"], a["cu"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(v=None), -1),
    (dict(B=0), -2), (dict(Sq=0), -2), (dict(Sk=-3), -2), (dict(Hq=0), -2),
    (dict(cu=FAKE, Sk=255), -2),
    (dict(d=96), -3), (dict(d=256), -3),
    (dict(Hq=6, Hkv=4), -4),
    (dict(dtype=7), -5), (dict(dtype=-1), -5),
    (dict(scale=float("nan")), -6), (dict(scale=float("inf")), -6), (dict(scale=0.0), -6),
    (dict(scale=-0.1), -6),
    (dict(dtype=2, cu=FAKE), -6),
    (dict(dtype=2, d=64), -3),
    (dict(Sq=1 << 30, Hq=64, d=128, Hkv=64), -9),
])
def test_validation_errors(lib, kw, code):
    assert fwd(lib, **kw) == code
    assert lib.attn_strerror(code)


def test_other_entry_points_validate(lib):
    assert lib.attn_fp8_prepass(None, FAKE, FAKE, 1, 128, 1, 128, 0, None, None) == -1
    assert lib.attn_fp8_prepass(FAKE, FAKE, FAKE, 1, 128, 1, 64, 0, None, None) == -3
    assert lib.attn_fp8_prepass(FAKE, FAKE, FAKE, 1, 0, 1, 128, 0, None, None) == -2
    assert lib.attn_fwd_fp8(FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, 1, 1, 1, 128, 128, 128,
                            0.1, 0, None) == -1
    assert lib.attn_fwd_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 1, 1, 128, 128, 64,
                            0.1, 0, None) == -3
    assert lib.attn_strerror(12345) == b"unknown status code"


def test_prepass_qkv_validates(lib):
    ok = [FAKE] * 9 + [1, 2, 2, 128, 128, 128, None, None]
    for i in range(9):
        a = list(ok)
        a[i] = None
        assert lib.attn_fp8_prepass_qkv(*a) == -1
    for i, bad in ((9, 0), (10, 0), (11, -1), (12, 0), (13, 0)):
        a = list(ok)
        a[i] = bad
        assert lib.attn_fp8_prepass_qkv(*a) == -2
    a = list(ok)
    a[14] = 64
    assert lib.attn_fp8_prepass_qkv(*a) == -3
    assert lib.attn_test_fail_next(-8) == 0
    assert lib.attn_fp8_prepass_qkv(*ok) == -8


def test_clock_probe_validates(lib):
    k = ctypes.c_int()
    assert lib.attn_clock_probe(None, 100, ctypes.byref(k), None) == -1
    assert lib.attn_clock_probe(FAKE, 100, None, None) == -1
    assert lib.attn_clock_probe(FAKE, 0, ctypes.byref(k), None) == -6


def test_default_signs_match_generator(lib):
    assert ea.default_signs(128) == W.hadamard_signs(128, 55).tolist()


def tiles(B, Hq, Hkv, Sq, causal, bm=128):
    nM = (Sq + bm - 1) // bm
    return [ea.tile_of(p, B, Hq, Hkv, Sq, bm, causal) for p in range(B * Hq * nM)], nM


@pytest.mark.parametrize("shape", [(1, 2, 2, 256), (4, 16, 16, 2048), (2, 32, 8, 1024), (3, 6, 2, 300),
                                   (1, 8, 1, 129), (2, 32, 8, 8192), (1, 16, 16, 16384)])
@pytest.mark.parametrize("causal", [0, 1])
def test_tile_map_is_bijection(lib, shape, causal):
    B, Hq, Hkv, Sq = shape
    ts, nM = tiles(B, Hq, Hkv, Sq, causal)
    assert sorted(ts) == sorted((b, h, m) for b in range(B) for h in range(Hq) for m in range(nM))


def xcd_runs(ts, group):
    """Per XCD (workgroups p = x mod 8): its workgroups in dispatch order and
    its KV groups in order of first appearance."""
    out = []
    for x in range(8):
        mine = ts[x::8]
        order = []
        for b, h, _ in mine:
            if (b, h // group) not in order:
                order.append((b, h // group))
        out.append((mine, order))
    return out


def test_tile_map_lpt_and_xcd_affinity(lib):
    # causal, 16 KV groups: 2 per XCD, query blocks longest first
    B, Hq, Hkv, Sq = 2, 32, 8, 2048
    group = Hq // Hkv
    ts, nM = tiles(B, Hq, Hkv, Sq, 1)
    for mine, kv in xcd_runs(ts, group):
        ms = [m for _, _, m in mine]
        assert ms == sorted(ms, reverse=True)          # longest (latest) query blocks first
        assert len(kv) == 2                            # whole KV groups per XCD
    # without even XCD split the order is still longest-first globally
    ts, _ = tiles(1, 3, 1, 1024, 1)
    ms = [m for _, _, m in ts]
    assert ms == sorted(ms, reverse=True)


@pytest.mark.parametrize("shape", [(2, 32, 8, 2048), (1, 16, 16, 16384)])
def test_tile_map_group_major_for_full_attention(lib, shape):
    # full attention: every XCD finishes one KV group (all its query blocks
    # and heads) before the next
    B, Hq, Hkv, Sq = shape
    group = Hq // Hkv
    ts, nM = tiles(B, Hq, Hkv, Sq, 0)
    for mine, kv in xcd_runs(ts, group):
        assert len(kv) == B * Hkv // 8
        per = nM * group
        for i, g in enumerate(kv):
            run = mine[i * per:(i + 1) * per]
            assert {(b, h // group) for b, h, _ in run} == {g}
            ms = [m for _, _, m in run]
            assert ms == sorted(ms)


def test_tile_of_rejects_bad_args(lib):
    with pytest.raises(ea.AttnError):
        ea.tile_of(10**6, 1, 2, 2, 256, 128, False)
    with pytest.raises(ea.AttnError):
        ea.tile_of(0, 1, 3, 2, 256, 128, False)


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,n", [
    (4, 32, 8, 1, 16384, 0), (1, 1, 1, 1, 100, 0), (2, 8, 8, 300, 5000, 0), (1, 2, 1, 256, 1000, 3),
    (1, 2, 2, 256, 100, 7), (1, 2, 2, 256, 129, 3), (1, 1, 1, 1, 64, 256), (16, 64, 8, 4096, 4096, 0),
])
def test_split_plan_covers_keys(lib, B, Hq, Hkv, Sq, Sk, n):
    splits, keys, packed = ea.split_plan(B, Hq, Hkv, Sq, Sk, num_splits=n)
    assert keys % 64 == 0 and keys > 0
    # every range non-empty, together exactly [0, Sk)
    assert (splits - 1) * keys < Sk <= splits * keys
    if n > 0:
        assert splits <= n
    else:
        assert 1 <= splits <= 64
        if splits > 1:
            assert keys >= 256


def test_split_plan_auto_decode_shape(lib):
    # decode, GQA 4:1: packed into 32 tiles of 4 rows -> 8 ranges of 2048
    # keys fill the 256 CUs once
    assert ea.split_plan(4, 32, 8, 1, 16384) == (8, 2048, True)
    # unpacked: 128 tiles of one row -> 2 ranges (a third would need a
    # second round of workgroups)
    assert ea.split_plan(4, 32, 8, 1, 16384, pack_gqa=False) == (2, 8192, False)
    # two workgroups per CU with d = 64
    assert ea.split_plan(4, 32, 8, 1, 16384, d=64) == (16, 1024, True)
    # enough tiles already -> one range, no packing
    assert ea.split_plan(2, 32, 8, 8192, 8192) == (1, 8192, False)
    # packing only where it gives fewer tiles
    assert ea.split_plan(1, 8, 2, 100, 1000, num_splits=1)[2] is False     # ceil(200/128)=2 == 2*1
    assert ea.split_plan(1, 8, 2, 64, 1000, num_splits=1)[2] is True       # 1 < 2
    assert ea.split_plan(1, 8, 8, 1, 1000, num_splits=1, pack_gqa=True)[2] is False   # no groups to pack


def test_splitkv_and_combine_validate(lib):
    def sk(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, Hq=2, Hkv=2, Sq=64, Sk=256, d=64,
                 scale=0.125, causal=0, n=2, pack=-1, dtype=0)
        a.update(kw)
        return lib.attn_fwd_splitkv(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                                    a["Sq"], a["Sk"], a["d"], a["scale"], a["causal"], a["n"], a["pack"],
                                    a["dtype"], None)
    assert sk(k=None) == -1
    assert sk(Sk=0) == -2
    assert sk(d=96) == -3
    assert sk(Hq=3) == -4
    assert sk(dtype=2) == -5 and sk(dtype=3) == -5
    assert sk(scale=float("nan")) == -6
    assert sk(n=-1) == -6 and sk(n=257) == -6
    assert sk(pack=2) == -6 and sk(pack=-2) == -6
    assert sk(Hq=6, Hkv=2, pack=1) == -6       # group 3 does not divide 128
    c = lambda **kw: lib.attn_combine(kw.get("op", FAKE), kw.get("lp", FAKE), kw.get("o", FAKE), None,
                                      kw.get("P", 2), kw.get("B", 1), 2, kw.get("Sq", 8), kw.get("d", 64),
                                      kw.get("dtype", 0), None)
    assert c(op=None) == -1 and c(o=None) == -1
    assert c(P=0) == -2 and c(Sq=0) == -2
    assert c(P=257) == -6
    assert c(d=32) == -3
    assert c(dtype=2) == -5
    assert lib.attn_split_plan(1, 1, 1, 1, 1, 64, 0, -1, None, None, None) == -1


def test_bwd_validates(lib):
    def bw(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, dlse=None, dq=FAKE, dk=FAKE, dv=FAKE,
                 B=1, Hq=2, Hkv=2, Sq=64, Sk=64, d=64, scale=0.125, causal=0, cu=None, dtype=0)
        a.update(kw)
        return lib.attn_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dlse"], a["dq"], a["dk"],
                            a["dv"], a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"], a["d"], a["scale"],
                            a["causal"], a["cu"], a["dtype"], None)
    for name in ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv"):
        assert bw(**{name: None}) == -1, name
    assert bw(Sq=0) == -2 and bw(B=-1) == -2
    assert bw(d=32) == -3
    assert bw(Hq=3) == -4
    assert bw(dtype=2) == -5 and bw(dtype=9) == -5
    assert bw(scale=float("inf")) == -6
    assert bw(cu=FAKE, Sk=65) == -2 and bw(cu=FAKE, B=0) == -2   # varlen needs Sq == Sk, B > 0


def test_fwd_ext_validates(lib):
    def fx(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, Hq=2, Hkv=2, Sq=64, Sk=64, d=64,
                 scale=0.125, causal=0, cu=None, dtype=0, cap=1.0, vcol=0)
        a.update(kw)
        return lib.attn_fwd_ext(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Sq"],
                                a["Sk"], a["d"], a["scale"], a["causal"], a["cu"], a["dtype"], a["cap"],
                                a["vcol"], None)
    assert fx(cap=-1.0) == -6 and fx(cap=float("nan")) == -6 and fx(cap=float("inf")) == -6
    assert fx(q=None) == -1
    assert fx(dtype=2) == -6 and fx(dtype=3) == -6        # options: 16-bit types only
    assert fx(dtype=11) == -5
    assert fx(cu=FAKE) == -6                               # options: dense only
    assert fx(cap=0.0, vcol=1, Sk=100) == -2               # column-major rows need Sk % 8 == 0
    assert fx(d=96) == -3 and fx(Hq=3) == -4
    # both options off: plain attn_fwd validation
    assert fx(cap=0.0, Sq=0) == -2


# ---------------------------------------------------------------- failure paths
# attn_test_fail_next arms a one-shot failure that fires before anything is
# enqueued, so these calls (with pointers that are never dereferenced) are
# safe with or without a GPU.
NOMEM, HIPERR = -7, -8


def splitkv(lib, **kw):
    a = dict(B=1, Hq=2, Hkv=2, Sq=256, Sk=4096, d=128, splits=4, pack=0, dtype=0)
    a.update(kw)
    return lib.attn_fwd_splitkv(FAKE, FAKE, FAKE, FAKE, None, a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"], a["d"],
                                0.1, 0, a["splits"], a["pack"], a["dtype"], None)


def bwd(lib):
    return lib.attn_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1, 2, 2, 256, 256, 64, 0.125,
                        0, None, 0, None)


@pytest.mark.parametrize("call", ["fwd_fp8_type", "fwd_fp8_hadamard", "splitkv", "bwd"])
def test_workspace_allocation_failure(lib, call):
    # every path that takes a library workspace reports ATTN_ERR_NOMEM when
    # the allocation fails
    assert lib.attn_test_fail_next(NOMEM) == 0
    if call == "fwd_fp8_type":
        rc = fwd(lib, dtype=2, d=128)
    elif call == "fwd_fp8_hadamard":
        rc = fwd(lib, dtype=3, d=128)
    elif call == "splitkv":
        rc = splitkv(lib)
    else:
        rc = bwd(lib)
    assert rc == NOMEM
    assert lib.attn_strerror(rc) == b"device workspace allocation failed"


@pytest.mark.parametrize("call", ["fwd_dense", "fwd_varlen", "fwd_ext", "fwd_fp8", "prepass", "combine"])
def test_launch_failure(lib, call):
    # a launch that fails maps to ATTN_ERR_HIP with the runtime's text
    assert lib.attn_test_fail_next(HIPERR) == 0
    if call == "fwd_dense":
        rc = fwd(lib)
    elif call == "fwd_varlen":
        rc = fwd(lib, cu=FAKE, B=3, Sq=512, Sk=512)
    elif call == "fwd_ext":
        rc = lib.attn_fwd_ext(FAKE, FAKE, FAKE, FAKE, None, 1, 2, 2, 256, 256, 128, 0.1, 0, None, 0, 30.0, 0, None)
    elif call == "fwd_fp8":
        rc = lib.attn_fwd_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 1, 1, 128, 128, 128, 0.1, 0, None)
    elif call == "prepass":
        rc = lib.attn_fp8_prepass(FAKE, FAKE, FAKE, 1, 128, 1, 128, 0, None, None)
    else:
        rc = lib.attn_combine(FAKE, FAKE, FAKE, None, 4, 1, 2, 16, 128, 0, None)
    assert rc == HIPERR
    msg = lib.attn_strerror(rc).decode()
    assert msg.startswith("HIP error") and "launch" in msg.lower(), msg


def test_failure_hook_is_one_shot_and_validated(lib):
    assert lib.attn_test_fail_next(-3) == -6          # only NOMEM, HIP or 0
    assert lib.attn_test_fail_next(HIPERR) == 0
    assert lib.attn_test_fail_next(0) == 0            # disarmed
    # validation still comes first: an armed failure is not consumed by a
    # call that fails validation
    assert lib.attn_test_fail_next(NOMEM) == 0
    assert fwd(lib, dtype=2, d=64) == -3
    assert fwd(lib, dtype=2, d=128) == NOMEM
    assert lib.attn_test_fail_next(0) == 0


def test_every_status_code_is_covered():
    # the error codes the header declares, each exercised above or in
    # test_validation_errors / test_other_entry_points_validate
    src = open(os.path.join(ROOT, "include", "attn.h")).read()
    codes = dict((n, int(v)) for n, v in re.findall(r"(ATTN_ERR_\w+)\s*=\s*(-\d+)", src))
    assert set(codes.values()) == {-1, -2, -3, -4, -5, -6, -7, -8, -9, -10}


def test_noalloc_rejects_plans_beyond_its_scratch(lib):
    # 16 MiB of partials: B=64 Sq=32 Hq=32 d=128 with 8 ranges needs
    # 8 * 65536 * 129 floats = 258 MiB -> ATTN_ERR_SCRATCH before anything runs
    rc = lib.attn_fwd_splitkv_noalloc(FAKE, FAKE, FAKE, FAKE, None, 64, 32, 8, 32, 16384, 128, 0.1, 0, 8, 0, 0,
                                      None)
    assert rc == -10
    assert b"scratch" in lib.attn_strerror(rc)
    assert lib.attn_fwd_splitkv_noalloc(None, FAKE, FAKE, FAKE, None, 1, 2, 2, 1, 256, 128, 0.1, 0, 0, -1, 0,
                                        None) == -1
    assert lib.attn_fwd_splitkv_noalloc(FAKE, FAKE, FAKE, FAKE, None, 1, 2, 2, 1, 256, 128, 0.1, 0, 0, -1, 2,
                                        None) == -5
