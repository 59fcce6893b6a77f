"""Build libkdt.so (all HIP sources of the library) for gfx950 with hipcc.

    python -m tree_verify_mla_kdt_amd.build          # or build() from Python

The shared library is written next to this file.  hipcc cross-compiles, so
this runs on a machine without a GPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkdt.so")
SOURCES = ["kdt_abi.hip", "kdt_visibility.hip", "kdt_verify.hip", "kdt_gather.hip", "kdt_accept.hip", "kdt_tree_build.hip",
           "kdt_absorb.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkdt.so)")


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed fp32 VALU ops stay disabled for all device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-result",
    ]


# sources whose device assembly is checked for inline-asm MFMA hazards
ASM_CHECKED = ["kdt_verify.hip"]


def build(verbose: bool = False) -> str:
    from . import asm_check
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *flags(), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    # the device assembly of the checked sources, compiled alongside
    lib_flags = [f for f in flags() if f != "-shared"]
    asm_jobs = []
    for name in ASM_CHECKED:
        out = os.path.join(HERE, f".{name}.s")
        acmd = [hipcc(), *lib_flags, "-S", "--offload-device-only", os.path.join(CSRC, name), "-o", out]
        asm_jobs.append((name, out, subprocess.Popen(acmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                                      text=True)))
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (res.stderr or "").splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        for _, _, proc in asm_jobs:
            proc.wait()
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    for name, out, proc in asm_jobs:
        _, aerr = proc.communicate()
        if proc.returncode != 0:
            raise RuntimeError(f"hipcc -S {name} failed ({proc.returncode}):\n{aerr}")
        with open(out) as f:
            problems = asm_check.check(f.read())
        os.remove(out)
        if problems:
            raise RuntimeError(f"{name}: inline-asm MFMA hazards in the compiled code:\n" + "\n".join(problems[:20]))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
