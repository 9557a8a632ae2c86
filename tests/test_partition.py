"""The span partition shared by the partial-attention kernels and the split-K merge
(decode_attention_sequence_paged_amd/csrc/dcp_partition.h), checked exhaustively on the
host by a C program (tests/partition_check.c) built with gcc, with AddressSanitizer and
UndefinedBehaviorSanitizer where the toolchain has them."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_sequence_paged_amd", "csrc")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_span_partition_exhaustive(tmp_path):
    exe = str(tmp_path / "partition_check")
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-Wall", "-Werror", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", CSRC, os.path.join(ROOT, "tests", "partition_check.c"),
           "-o", exe]
    subprocess.run(cmd, check=True)
    proc = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    print(proc.stdout[-3000:])
    assert proc.returncode == 0, proc.stdout[-3000:]
    assert proc.stdout.strip().endswith("0 failures")
