"""Compile the seeded input generators: the host one (gcc, OpenMP) and the device one (hipcc)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ARCH = os.environ.get("DCP_OFFLOAD_ARCH", "gfx950")


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if proc.returncode != 0:
        raise RuntimeError("build failed: %s\n%s" % (" ".join(cmd), proc.stdout))


def build_all() -> None:
    host = os.path.join(HERE, "libdcp_synth_host.so")
    _run(["gcc", "-O3", "-fopenmp", "-shared", "-fPIC", os.path.join(HERE, "csrc", "synth_host.c"),
          "-o", host + ".tmp"])
    os.replace(host + ".tmp", host)
    dev = os.path.join(HERE, "libdcp_synth.so")
    _run(["/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else "hipcc",
          "-O3", "-fPIC", "-shared", "--offload-arch=" + ARCH,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          os.path.join(HERE, "csrc", "synth_fill.hip"), os.path.join(HERE, "csrc", "hbm_probe.hip"),
          "-o", dev + ".tmp"])
    os.replace(dev + ".tmp", dev)


if __name__ == "__main__":
    build_all()
