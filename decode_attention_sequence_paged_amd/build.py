"""Compile the HIP library (libdcp.so) for gfx950, in-tree, with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libdcp.so")
SOURCES = ["dcp_api.hip", "mla_partial.hip", "gqa_partial.hip", "reduce.hip", "append.hip",
           "merge_steps.hip", "noalloc.hip"]
ARCH = os.environ.get("DCP_OFFLOAD_ARCH", "gfx950")

# Packed fp32 VALU forms are disabled: hipcc must not emit v_pk_{add,mul,fma}_f32.
# MFMA accumulators are allocated in VGPRs (the "VGPR form"), which leaves the
# accumulation registers to the MLA kernel's query slice and avoids copying the
# O accumulator between register files every tile.
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=" + ARCH,
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-mllvm", "-amdgpu-mfma-vgpr-form",
               "-I", os.path.join(ROOT, "include")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in proc.stdout.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError("build failed: %s\n%s" % (" ".join(cmd), out))
    return out


def build_lib(verbose: bool = False) -> str:
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    out = _run(cmd)
    os.replace(tmp, LIB_PATH)
    if verbose and out.strip():
        print(out)
    return LIB_PATH


if __name__ == "__main__":
    print(build_lib(verbose="-v" in sys.argv))
