"""CPU tests of the build's assembly checks on the named-register kernels:
AGPRs the inline assembly names must lie inside the AGPR range the kernel
descriptor allocates, the compiler must not use AGPRs itself, and nothing may
spill (exact_attention_75_amd/build.py, scan_pinned_agprs); and in the
LDS-poisoning build every direct-to-LDS copy must follow a completed poison
write (scan_poison_order)."""
import pytest

from exact_attention_75_amd import build as B


def listing(named_top: int, next_free: int, accum: int, compiler_line: str = "", spills: int = 0):
    return f"""_ZN4attn1kEv:
\tv_mov_b32 v1, 0
;;#ASMSTART
\tv_mfma_f32_32x32x16_bf16 v[0:15], a[{named_top - 3}:{named_top}], a[0:3], 0
;;#ASMEND
{compiler_line}
\ts_endpgm
\t.amdhsa_kernel _ZN4attn1kEv
\t\t.amdhsa_next_free_vgpr {next_free}
\t\t.amdhsa_accum_offset {accum}
\t.end_amdhsa_kernel
\t.vgpr_spill_count: {spills}
""".splitlines(True)


def test_agprs_inside_the_allocation_pass():
    B.scan_pinned_agprs("k.hip", listing(95, 168, 72))       # a0..a95 in 96 AGPRs
    B.scan_pinned_agprs("k.hip", listing(255, 456, 200))     # the whole AGPR file


def test_agpr_past_the_allocation_fails():
    with pytest.raises(RuntimeError, match="names a95 but its descriptor allocates 92"):
        B.scan_pinned_agprs("k.hip", listing(95, 164, 72))


def test_compiler_agpr_use_fails():
    with pytest.raises(RuntimeError, match="compiler-generated AGPR use"):
        B.scan_pinned_agprs("k.hip", listing(95, 168, 72, compiler_line="\tv_accvgpr_read_b32 v2, a7"))


def test_spills_fail():
    with pytest.raises(RuntimeError, match="register spills"):
        B.scan_pinned_agprs("k.hip", listing(95, 168, 72, spills=4))


# ---------------------------------------------------------------- poisoning build
POISON_OK = """\tds_write_b128 v1, v[4:7]
\tds_write_b128 v1, v[4:7] offset:1024
;;#ASMSTART
\ts_waitcnt lgkmcnt(0)
;;#ASMEND
\tbuffer_load_dwordx4 v2, s[8:11], 0 offen lds
\tbuffer_load_dwordx4 v3, s[8:11], 0 offen lds
""".splitlines(True)


def test_poison_order_passes():
    B.scan_poison_order("k.hip", POISON_OK)


def test_copy_without_poison_write_fails():
    with pytest.raises(RuntimeError, match="without a completed poison write"):
        B.scan_poison_order("k.hip", POISON_OK + ["\tbuffer_load_dwordx4 v3, s[8:11], 0 offen lds\n"])


def test_poison_write_not_waited_for_fails():
    lines = ["\tds_write_b128 v1, v[4:7]\n", "\tbuffer_load_dwordx4 v2, s[8:11], 0 offen lds\n"]
    with pytest.raises(RuntimeError, match="without a completed poison write"):
        B.scan_poison_order("k.hip", lines)


def test_poisoning_build_without_copies_fails():
    with pytest.raises(RuntimeError, match="no direct-to-LDS copies"):
        B.scan_poison_order("k.hip", ["\ts_endpgm\n"])
