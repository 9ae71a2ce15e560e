"""CPU tests of the build's assembly checks on the named-register kernels:
AGPRs the inline assembly names must lie inside the AGPR range the kernel
descriptor allocates, the compiler must not use AGPRs itself, and nothing may
spill (exact_attention_75_amd/build.py, scan_pinned_agprs)."""
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
