"""Build libtitans_mem.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtitans_mem.so")
OBJDIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 VALU instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
# Per-source extra flags.  The fused scans keep 256 (single workgroup) or 128 (pair)
# fp32 state registers per lane live across the chunk loop; MFMA results in VGPRs (AGPRs then serve as spill
# space) keep it out of scratch memory.
SOURCES = {
    "abi.hip": [],
    "scan_generic.hip": [],
    "scan_phased.hip": [],
    "scan_backward.hip": [],
    "scan_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "scan_pair.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "retrieve_mfma.hip": [],
    "retrieve_wide.hip": [],
    "mag.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src, extra, verbose):
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c",
           os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    return obj


def build(extra_flags=(), out=LIB, verbose=False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda kv: _compile(kv[0], [*kv[1], *extra_flags], verbose),
                           SOURCES.items()))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
