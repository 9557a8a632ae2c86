"""The C ABI from C: a client compiled with gcc against include/dcp.h and linked to
libdcp.so calls the host entry points and the device entry points' argument checks."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "decode_attention_sequence_paged_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_client_against_the_header(tmp_path):
    if not os.path.exists(os.path.join(LIB_DIR, "libdcp.so")):
        pytest.fail("libdcp.so is not built; run __graft_entry__.build()")
    exe = str(tmp_path / "c_abi_client")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_abi_client.c"), "-L", LIB_DIR, "-ldcp",
                    "-Wl,-rpath," + LIB_DIR, "-o", exe], check=True)
    proc = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    print(proc.stdout)
    assert proc.returncode == 0, proc.stdout
    assert "0 failures" in proc.stdout
