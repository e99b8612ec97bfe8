"""Build the HIP library ``libttc_attn.so`` in-tree with hipcc for gfx950.

Usage: ``python -m tiled_tensor_core_amd.build [--isa DIR]``.  ``--isa`` also
keeps the device assembly (gfx950 ISA of this build) in DIR for inspection.
"""

from __future__ import annotations

import argparse
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_NAME = "libttc_attn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

SOURCES = [os.path.join(CSRC, "attn_fwd_kernel.hip"), os.path.join(CSRC, "softmax_kernel.hip"),
           os.path.join(CSRC, "gemm_kernel.hip"), os.path.join(CSRC, "unfused_kernel.hip"),
           os.path.join(CSRC, "attn_api.cpp")]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep the compiler from forming packed fp32 VALU ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the kernels' per-tile step loops are unrolled in full by pragma; the
    # default size limit would leave the largest one rolled, and its
    # register arrays in scratch memory
    "-mllvm", "-pragma-unroll-threshold=1000000",
    # per-kernel resource report, checked below for scratch use
    "-Rpass-analysis=kernel-resource-usage",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(isa_dir: str | None = None, verbose: bool = False) -> str:
    """Compile every HIP source into the in-tree shared library; return its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *SOURCES, "-o", tmp]
    cwd = None
    if isa_dir:
        os.makedirs(isa_dir, exist_ok=True)
        cmd.insert(1, "--save-temps")
        cwd = isa_dir
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    lines = [line for line in res.stderr.splitlines() if noise not in line]
    report = [line for line in lines if "kernel-resource-usage" in line]
    err = "\n".join(line for line in lines if "kernel-resource-usage" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    # every kernel is designed to live in registers: scratch means spills or
    # a register array the compiler could not keep in registers
    kernel = None
    spills = []
    for line in report:
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            kernel = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0:
            spills.append(f"{kernel}: {m.group(1)} bytes of scratch per lane")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    if spills:
        os.remove(tmp)
        raise RuntimeError("kernels spill registers to scratch memory:\n  " + "\n  ".join(spills))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--isa", default=None, help="keep device assembly in this directory")
    a = ap.parse_args()
    print(build(isa_dir=a.isa, verbose=True))
