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


def _compile(src: str, obj: str, isa_dir: str | None) -> subprocess.CompletedProcess:
    flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    cmd = [hipcc(), *flags, "-c", src, "-o", obj]
    if isa_dir:
        cmd.insert(1, "--save-temps")
    return subprocess.run(cmd, cwd=isa_dir, capture_output=True, text=True)


def build(isa_dir: str | None = None, verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every HIP source (in parallel, one hipcc per source) and link
    the in-tree shared library; return its path."""
    import concurrent.futures
    import tempfile

    tmp = LIB_PATH + ".tmp"
    if isa_dir:
        os.makedirs(isa_dir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, min(8, (os.cpu_count() or 1))))
    with tempfile.TemporaryDirectory(prefix="ttc_build_") as objdir:
        objs = [os.path.join(objdir, os.path.basename(src) + ".o") for src in SOURCES]
        if verbose:
            print(f"compiling {len(SOURCES)} sources with {jobs} jobs", flush=True)
        with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
            results = list(ex.map(lambda so: _compile(so[0], so[1], isa_dir), zip(SOURCES, objs)))
        link = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                              capture_output=True, text=True)
        results.append(link)
    noise = "is not a recognized feature for this target"
    lines = [line for r in results for line in r.stderr.splitlines() if noise not in line]
    report = [line for line in lines if "kernel-resource-usage" in line]
    err = "\n".join(line for line in lines if "kernel-resource-usage" not in line)
    failed = [r for r in results if r.returncode != 0]
    if failed:
        raise RuntimeError(f"hipcc failed ({failed[0].returncode}):\n{err}")
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
