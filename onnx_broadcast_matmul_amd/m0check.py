"""Build check: the direct global-to-LDS loads own M0 in every kernel that uses them.

The tiled kernels issue gfx950 buffer loads with the LDS destination from
inline asm (``s_mov_b32 m0, sN`` immediately followed by ``buffer_load_dword*
... lds``; the LDS address comes from M0).  The compiler cannot be told that
the asm writes M0, so the kernels are correct only while the compiler itself
neither writes nor reads M0 anywhere in them.  (The compiler-owned builtin
for the same load makes the compiler wait for every outstanding LDS load
before the next LDS read, which serialises the stage pipeline.)

This module disassembles the gfx950 code objects built from this package's
own sources (``llvm-objdump`` on the device half of each object) and fails
when a kernel that contains an LDS load also contains any other M0 access:
an M0 write that is not directly followed by an LDS load, or an instruction
that reads M0 implicitly (relative moves, messages, GWS, interpolation,
LDS-direct operands).
"""
from __future__ import annotations

import os
import re
import subprocess
import tempfile

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
LLVM = os.path.join(ROCM, "llvm", "bin")
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"

# Mnemonic fragments of instructions that read M0 without naming it.
IMPLICIT_M0 = ("movrel", "sendmsg", "ds_gws", "addtid", "v_interp", "lds_direct", "ttracedata", "global_load_lds",
               "scratch_load_lds")
LDS_LOAD = re.compile(r"^\s*buffer_load_\w+\b.*\blds\b")
M0_SET = re.compile(r"^\s*s_mov_b32\s+m0,\s*s\d+\s*$")
FUNC = re.compile(r"^[0-9a-f]+ <(.+)>:$")


def _instructions(disasm: str):
    """{function name: [instruction text]} from llvm-objdump -d output."""
    funcs, cur = {}, None
    for line in disasm.splitlines():
        m = FUNC.match(line.strip())
        if m:
            cur = funcs.setdefault(m.group(1), [])
            continue
        if cur is None:
            continue
        text = line.split("//")[0].strip()
        if text:
            cur.append(text)
    return funcs


def violations(disasm: str):
    """(function, instruction) pairs that break the M0 rule."""
    bad = []
    for name, ins in _instructions(disasm).items():
        if not any(LDS_LOAD.match(i) for i in ins):
            continue
        for k, i in enumerate(ins):
            mn = i.split()[0]
            if M0_SET.match(i):
                if k + 1 >= len(ins) or not LDS_LOAD.match(ins[k + 1]):
                    bad.append((name, i))
            elif re.search(r"\bm0\b", i) or any(f in mn for f in IMPLICIT_M0):
                bad.append((name, i))
    return bad


def disassemble(obj: str) -> str:
    """gfx950 disassembly of the device code bundled in a hipcc object."""
    with tempfile.TemporaryDirectory() as d:
        fat = os.path.join(d, "fatbin")
        host = os.path.join(d, "host.o")
        co = os.path.join(d, "device.co")
        subprocess.run([os.path.join(LLVM, "llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", obj, host],
                       check=True, stdout=subprocess.PIPE, stderr=subprocess.PIPE)
        subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o", f"--input={fat}",
                        f"--targets={TARGET}", f"--output={co}"], check=True, stdout=subprocess.PIPE,
                       stderr=subprocess.PIPE)
        r = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", co], check=True,
                           stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
        return r.stdout


def check_objects(objs) -> int:
    """Raise if any kernel in the objects breaks the M0 rule; returns the
    number of kernels with LDS loads that were checked."""
    checked = 0
    problems = []
    for obj in objs:
        dis = disassemble(obj)
        funcs = _instructions(dis)
        checked += sum(1 for ins in funcs.values() if any(LDS_LOAD.match(i) for i in ins))
        problems += [(os.path.basename(obj), f, i) for f, i in violations(dis)]
    if problems:
        lines = "\n".join(f"  {o}: {f}: {i}" for o, f, i in problems[:20])
        raise RuntimeError(f"M0 is used outside the LDS-load asm in {len(problems)} place(s):\n{lines}")
    return checked
