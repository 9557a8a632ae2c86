"""Generated-code check of the partial kernels' inline-asm query loads (CPU only: hipcc -S).

The query slices are loaded with inline asm so that the compiler's wait counting, which
cannot see the direct-to-LDS tile copies either, does not drain the copy ring before
every use.  The compiler then treats the destination registers as written when the asm
issues: nothing may read, write or move those registers before an explicit
`s_waitcnt vmcnt(n)` that covers the load.  The covering count is the number of younger
memory operations the kernel lets stay in flight at that wait: 0 in the MLA kernels
(the score waves issue no copies), 8 in the GQA kernel (one copy round issued after the
load).  The test compiles the kernels with the library's flags and checks, in program
order after every such load, that its registers are untouched until a covering wait.
A copy of the MLA kernel whose query slice is never used (so the compiler may reuse its
registers while the loads are in flight) must fail the same check.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_sequence_paged_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form", "-I", os.path.join(ROOT, "include")]

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")

_LOAD = re.compile(r"global_load_dwordx4 v\[(\d+):(\d+)\], v\[\d+:\d+\], off")
_WAIT = re.compile(r"s_waitcnt vmcnt\((\d+)\)")
_REG = re.compile(r"v\[(\d+):(\d+)\]|\bv(\d+)\b")


def _compile(src, out, extra=()):
    proc = subprocess.run([HIPCC] + FLAGS + list(extra) + [src, "-o", out],
                          stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert proc.returncode == 0, proc.stdout[-3000:]
    with open(out) as f:
        return f.read()


def _hazards(asm, covering):
    """{kernel: (asm query loads, loads whose registers are touched before a covering
    wait, loads never followed by one)}."""
    res = {}
    for name in re.findall(r"^(_Z\S+):\s*;\s*@", asm, re.M):
        i = asm.index(name + ":")
        body = asm[i:asm.index("s_endpgm", i)].split("\n")
        loads = touched = uncovered = 0
        in_asm = False
        for k, line in enumerate(body):
            if ";;#ASMSTART" in line or ";;#ASMEND" in line:
                in_asm = ";;#ASMSTART" in line
                continue
            m = _LOAD.search(line) if in_asm else None
            if not m:
                continue
            loads += 1
            regs = set(range(int(m.group(1)), int(m.group(2)) + 1))
            covered, asm2 = False, False
            for l2 in body[k + 1:]:
                if ";;#ASMSTART" in l2 or ";;#ASMEND" in l2:
                    asm2 = ";;#ASMSTART" in l2
                    continue
                code = l2.split(";")[0]
                w = _WAIT.search(code)
                if w and int(w.group(1)) <= covering:
                    covered = True
                    break
                if asm2 and _LOAD.search(code):
                    continue  # the slice's other loads
                hit = False
                for r in _REG.finditer(code):
                    rr = {int(r.group(3))} if r.group(3) else set(range(int(r.group(1)), int(r.group(2)) + 1))
                    hit = hit or bool(rr & regs)
                if hit:
                    touched += 1
                    break
            uncovered += 0 if covered else 1
        res[name] = (loads, touched, uncovered)
    return res


@pytest.mark.parametrize("src,covering", [("mla_partial.hip", 0), ("gqa_partial.hip", 8)])
def test_asm_query_loads_are_waited_for(tmp_path, src, covering):
    res = _hazards(_compile(os.path.join(CSRC, src), str(tmp_path / "k.s")), covering)
    checked = {n: v for n, v in res.items() if v[0] > 0}
    assert checked, "no inline-asm query load found in %s" % src
    for name, (loads, touched, uncovered) in checked.items():
        assert touched == 0 and uncovered == 0, (name, loads, touched, uncovered)


def test_check_catches_an_unused_asm_slice(tmp_path):
    """A copy of the MLA kernel whose score waves never use the slice they load."""
    with open(os.path.join(CSRC, "mla_partial.hip")) as f:
        s = f.read()
    old = "      f32x4 s0, s1;\n      qk(tb, s0, s1);"
    assert s.count(old) == 1
    s = s.replace(old, "      f32x4 s0, s1;\n      (void)qk;\n      s0 = f32x4{(float)(lane & 7), 1.f, 2.f, 3.f};\n"
                       "      s1 = s0;")
    s = s.replace('#include "../../include/dcp.h"', '#include "dcp.h"')
    src = tmp_path / "mla_partial.hip"
    src.write_text(s)
    res = _hazards(_compile(str(src), str(tmp_path / "k.s"), ["-I", CSRC]), 0)
    assert any(v[0] > 0 and (v[1] > 0 or v[2] > 0) for v in res.values()), res
