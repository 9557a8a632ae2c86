"""Host code of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

dcp_api.hip (argument validation, planning, workspace sizing, the shard map) is compiled
host-only with the sanitizers (hipcc, `-Xarch_host -fsanitize=...`), linked with a stand-in
launch layer (tests/host_launch_stubs.cpp) into two C programs built with clang and the
same sanitizers:
* tests/c_abi_client.c, the host entry points and the device entry points' argument
  checks;
* tests/shard_sweep.c, an exhaustive sweep of dcp_shard_map / dcp_shard_locate /
  dcp_shard_global over request lengths L <= 4096, N = 1..8 and I in {1, 2, 3, 7, 16, 64,
  128, 1000}, compared here with the oracle's enumeration of which positions each rank
  holds (bit-exact).
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_sequence_paged_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
LMAX = 4096
IS = (1, 2, 3, 7, 16, 64, 128, 1000)
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                                reason="needs the ROCm toolchain")


def _run(cmd, **kw):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert proc.returncode == 0, "%s\n%s" % (" ".join(cmd), proc.stdout[-4000:])
    return proc.stdout


@pytest.fixture(scope="module")
def programs(tmp_path_factory):
    d = tmp_path_factory.mktemp("hostsan")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    host_san = []
    for f in SAN:
        host_san += ["-Xarch_host", f]
    objs = []
    for src in (os.path.join(CSRC, "dcp_api.hip"), os.path.join(ROOT, "tests", "host_launch_stubs.cpp")):
        o = str(d / (os.path.basename(src) + ".o"))
        _run([HIPCC, "--offload-host-only", "-x", "hip", "-O1", "-g", "-std=c++17", "-fPIC"] + host_san
             + inc + ["-c", src, "-o", o])
        objs.append(o)
    exes = {}
    for name in ("c_abi_client", "shard_sweep"):
        o = str(d / (name + ".o"))
        # (the allocation-free entry point lives beside its device scratch array, which a
        # host-only build cannot hold: the client skips that check here)
        _run([CLANG, "-std=c99", "-O1", "-g", "-Wall", "-Werror", "-DDCP_CLIENT_HOST_ONLY"] + SAN + inc
             + ["-c", os.path.join(ROOT, "tests", name + ".c"), "-o", o])
        exe = str(d / name)
        _run([CLANG + "++"] + SAN + [o] + objs + ["-L/opt/rocm/lib", "-lamdhip64",
                                                  "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
        exes[name] = exe
    return d, exes


def test_c_client_under_sanitizers(programs):
    _, exes = programs
    out = _run([exes["c_abi_client"]], timeout=120)
    assert "0 failures" in out


def test_shard_sweep_against_oracle_enumeration(programs):
    d, exes = programs
    path = str(d / "sweep.bin")
    out = _run([exes["shard_sweep"], path], timeout=300)
    assert "done" in out
    data = np.fromfile(path, dtype=np.int64)
    off = 0
    t = np.arange(LMAX)
    for N in range(1, 9):
        for I in IS:
            owner_ref = oracle.owner_rank(t, N, I)
            for r in range(N):
                toks = oracle.rank_tokens(LMAX, N, I, r)
                lens = data[off:off + LMAX + 1]; off += LMAX + 1
                owner = data[off:off + LMAX]; off += LMAX
                local = data[off:off + LMAX]; off += LMAX
                # L_r(L) = how many of the rank's positions lie below L
                assert np.array_equal(lens, np.searchsorted(toks, np.arange(LMAX + 1))), (N, I, r)
                assert np.array_equal(owner, owner_ref), (N, I, r)
                assert np.array_equal(local[toks], np.arange(toks.size)), (N, I, r)
                glob = data[off:off + toks.size]; off += toks.size
                assert np.array_equal(glob, toks), (N, I, r)
    assert off == data.size
