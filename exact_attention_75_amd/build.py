"""Build the HIP library libattn.so in-tree for gfx950.

    python -m exact_attention_75_amd.build [--jobs N] [--save-temps DIR] [--poison]

Each source is compiled by hipcc to an object in ``_build/`` and the objects
are linked into ``exact_attention_75_amd/libattn.so``.  ``--poison`` builds
the LDS-poisoning debug library instead (``-DATTN_DEBUG_POISON``: every copy
into an LDS stage first fills it with NaN), objects in ``_build_poison/``,
library ``exact_attention_75_amd/libattn_poison.so``; the tests compare its
results bit for bit with the normal library's.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libattn.so")
BUILD_POISON = os.path.join(PKG, "_build_poison")
LIB_POISON = os.path.join(PKG, "libattn_poison.so")
SOURCES = ["attn_api.cpp", "attn_fwd.hip", "attn_fwd_wide.hip", "attn_fp8.hip", "attn_combine.hip", "attn_bwd.hip",
           "attn_bwd_dkdv.hip", "attn_bwd_dq.hip", "attn_clock.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def common_flags(poison: bool = False):
    return (["-DATTN_DEBUG_POISON"] if poison else []) + [
        "-O3", "-std=c++2c", "-fPIC", f"--offload-arch={ARCH}",
        # packed fp32 VALU ops stay off: the compiler must not form v_pk_* f32 ops
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Wno-unused-command-line-argument",
    ]


def compile_one(src: str, save_temps: str | None, poison: bool = False) -> str:
    obj = os.path.join(BUILD_POISON if poison else BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags(poison) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        cmd += [f"-save-temps={'obj'}"]
        obj_dir = save_temps
        cmd[cmd.index("-o") + 1] = os.path.join(obj_dir, os.path.basename(obj))
        obj = os.path.join(obj_dir, os.path.basename(obj))
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{msgs}")
    if msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


# Sources whose kernels keep data in AGPRs named in inline assembly: the
# compiler must not use any AGPR itself there (see csrc/wide_regs.h).
PINNED_AGPR_SOURCES = ["attn_fwd_wide.hip", "attn_bwd_dkdv.hip", "attn_bwd_dq.hip"]


def check_pinned_agprs(src: str, poison: bool = False) -> None:
    """Compile `src` to device assembly and fail unless, in every kernel, AGPRs
    appear only inside inline-assembly regions, nothing spills, and the kernel
    descriptor allocates every AGPR the inline assembly names (the AGPRs of a
    wave are the registers from .amdhsa_accum_offset up to
    .amdhsa_next_free_vgpr; one named past that would belong to another
    wave)."""
    asm = os.path.join(BUILD_POISON if poison else BUILD, os.path.splitext(src)[0] + ".s")
    cmd = [hipcc()] + common_flags(poison) + ["--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", asm]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"assembly listing failed: {src}\n{r.stderr}")
    with open(asm) as f:
        scan_pinned_agprs(src, f)


def scan_pinned_agprs(src: str, lines) -> None:
    """The checks of check_pinned_agprs over the lines of an assembly listing."""
    agpr = re.compile(r"\ba\d+\b|\ba\[\d+:\d+\]")
    agpr_index = re.compile(r"\ba(\d+)\b|\ba\[\d+:(\d+)\]")
    in_asm = False
    kernel = None
    named = {}        # kernel -> highest AGPR index its inline assembly names
    desc = None       # kernel whose descriptor is being read
    fields = {}
    for line in lines:
        if line.startswith("_Z") and line.rstrip().endswith(":"):
            kernel = line.split(":")[0]
            named.setdefault(kernel, -1)
        t = line.strip()
        if t.startswith(".amdhsa_kernel "):
            desc, fields = t.split()[1], {}
            continue
        if desc is not None:
            f = t.split()
            if len(f) == 2 and f[0] in (".amdhsa_next_free_vgpr", ".amdhsa_accum_offset"):
                fields[f[0]] = int(f[1])
            if t.startswith(".end_amdhsa_kernel"):
                top = named.get(desc, -1)
                have = fields.get(".amdhsa_next_free_vgpr", 0) - fields.get(".amdhsa_accum_offset", 0)
                if top >= have:
                    raise RuntimeError(f"{src}: {desc} names a{top} but its descriptor allocates {have} AGPRs")
                desc = None
            continue
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        code = t.split(";")[0]
        if kernel and in_asm and code:
            for m in agpr_index.finditer(code):
                named[kernel] = max(named[kernel], int(m.group(1) or m.group(2)))
        if kernel and not in_asm and code and not code.startswith(".") and agpr.search(code):
            raise RuntimeError(f"{src}: compiler-generated AGPR use in {kernel}: {code}")
        m = re.match(r"\.(vgpr_spill_count|private_segment_fixed_size):\s+(\d+)", t)
        if m and int(m.group(2)) != 0:
            raise RuntimeError(f"{src}: {m.group(1)} = {m.group(2)} (register spills)")


def check_poison_order(src: str) -> None:
    """In the device assembly of the poisoning build, every direct-to-LDS
    copy must come after a poison write (ds_write_b128) that an
    s_waitcnt lgkmcnt(0) has completed, one write per copy."""
    asm = os.path.join(BUILD_POISON, os.path.splitext(src)[0] + ".s")
    with open(asm) as f:
        scan_poison_order(src, f)


def scan_poison_order(src: str, lines) -> None:
    """The check of check_poison_order over the lines of an assembly listing."""
    pending = ready = copies = 0
    for line in lines:
        t = line.split(";")[0].strip()
        if t.startswith("ds_write_b128"):
            pending += 1
        elif re.match(r"s_waitcnt\s+lgkmcnt\(0\)$", t):
            ready, pending = ready + pending, 0
        elif re.match(r"buffer_load_dword\w*\s.*\slds$", t):
            copies += 1
            if ready <= 0:
                raise RuntimeError(f"{src}: LDS copy without a completed poison write before it: {t}")
            ready -= 1
    if copies == 0:
        raise RuntimeError(f"{src}: no direct-to-LDS copies found in the poisoning build")


def build(jobs: int = 4, save_temps: str | None = None, poison: bool = False) -> str:
    lib = LIB_POISON if poison else LIB
    os.makedirs(BUILD_POISON if poison else BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: compile_one(s, save_temps, poison), SOURCES))
        list(ex.map(lambda s: check_pinned_agprs(s, poison), PINNED_AGPR_SOURCES))
    if poison:
        for src in PINNED_AGPR_SOURCES:
            check_poison_order(src)
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)
    check_kernels(lib)
    return lib


EXPECTED_KERNELS = ("fwd_kernel", "fwd_wide_kernel", "fwd_fp8_kernel", "prepass_kernel", "combine_kernel",
                    "bwd_pre_kernel", "bwd_dkdv_kernel", "bwd_dkdv_pipe_kernel", "bwd_dq_pipe_kernel")


def check_kernels(path: str) -> None:
    """Fail if the linked library lacks the device code objects of the
    kernels (a host pass that drops a kernel template leaves no error)."""
    blob = open(path, "rb").read()
    if f"amdgcn-amd-amdhsa--{ARCH}".encode() not in blob:
        raise RuntimeError(f"{path}: no {ARCH} code object embedded")
    for name in EXPECTED_KERNELS:
        if blob.count(name.encode()) < 2:
            raise RuntimeError(f"{path}: kernel {name} missing from the device code")


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--save-temps", default=None)
    ap.add_argument("--poison", action="store_true", help="build the LDS-poisoning debug library")
    a = ap.parse_args()
    print(build(a.jobs, a.save_temps, a.poison))
