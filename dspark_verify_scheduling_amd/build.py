"""Build libdspark.so (the C-ABI library with its gfx950 kernels) in-tree.

``python -m dspark_verify_scheduling_amd.build`` or ``build()`` compiles every
HIP source under ``csrc/`` with hipcc for gfx950. A second, host-only library,
``libdspark_hostcheck.so``, exposes the device sigmoid compiled for the CPU so
that its rarely taken exact path can be tested without a GPU.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIB = PKG / "libdspark.so"
HOSTCHECK = PKG / "libdspark_hostcheck.so"
ARCH = "gfx950"

LIB_SOURCES = ["api.hip", "plan.hip", "pack.hip", "accept.hip", "tv.hip", "scatter.hip", "sts.hip", "sampling.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    # no packed fp32 instructions: plain scalar fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no contraction of a product and a sum into one rounding anywhere, also
    # inside inlined header functions such as __fmul_rn (a plain x * y): the
    # exact paths round each operation on its own; FMAs are written as such
    "-ffp-contract=off",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libdspark)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(str(c) for c in cmd), flush=True)
    res = subprocess.run([str(c) for c in cmd], capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"build failed: {cmd[-1]}")


def check_m0_use(asm: str) -> None:
    """The soft accept-rate kernels copy global memory straight into LDS with
    inline assembly that sets M0 (the LDS address) itself, out of the
    compiler's sight. That is sound only while nothing else in the code uses
    M0: raise unless every line of the gfx950 assembly that names m0 is one of
    those inline-assembly statements (an `s_mov_b32 m0, sN` directly followed
    by `s_nop 0` and `global_load_lds_dwordx4`, between the compiler's
    ;;#ASMSTART / ;;#ASMEND markers)."""
    lines = asm.splitlines()
    inside = False
    for i, line in enumerate(lines):
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            inside = True
            continue
        if t.startswith(";;#ASMEND"):
            inside = False
            continue
        if t.startswith((";", ".")) or "m0" not in t.replace(",", " ").split():
            continue
        ok = (inside and t.startswith("s_mov_b32 m0, s") and i + 2 < len(lines)
              and lines[i + 1].strip() == "s_nop 0"
              and lines[i + 2].strip().startswith("global_load_lds_dwordx4"))
        if not ok:
            raise RuntimeError(f"tv.hip: unexpected use of M0 in the generated code: {t!r}")


def build(verbose: bool = False) -> Path:
    """Compile libdspark.so and libdspark_hostcheck.so next to this file."""
    hipcc = _hipcc()
    tmp = LIB.with_suffix(".so.tmp")
    _run([hipcc, *COMMON_FLAGS, "-o", tmp, *[CSRC / s for s in LIB_SOURCES]], verbose)
    asm = LIB.with_suffix(".tv.s")
    flags = [f for f in COMMON_FLAGS if f not in ("-shared", "-fPIC")]
    _run([hipcc, *flags, "-S", "--cuda-device-only", "-o", asm, CSRC / "tv.hip"], verbose)
    try:
        check_m0_use(asm.read_text())
    finally:
        asm.unlink()
    os.replace(tmp, LIB)
    tmp = HOSTCHECK.with_suffix(".so.tmp")
    _run([hipcc, *COMMON_FLAGS, "-o", tmp, CSRC / "hostcheck.hip"], verbose)
    os.replace(tmp, HOSTCHECK)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
