"""The GEMM's explicit vmcnt waits count the vector-memory loads each stage issues. This test
compiles gemm.hip for gfx950 (device code only, no GPU needed) and checks, in the generated
assembly of every block-scaled kernel, that the compiler issues exactly the loads those counts
assume:
- the prologue (up to the first barrier) holds the scale loads of its even stages: two stages
  with five buffers, one with two;
- each K-loop body holds D direct-to-LDS loads per stage plus TM + SB scale loads per even stage.
A compiler that merged or dropped a scale load would make the waits too permissive."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "fp8_block_scaled_pf8_amd", "csrc", "gemm.hip")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "gemm.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "--cuda-device-only", "-S", "-o", str(out), SRC]
    subprocess.run(cmd, check=True, capture_output=True, timeout=900)
    return out.read_text()


def _functions(text):
    funcs, cur = {}, None
    for line in text.split("\n"):
        m = re.match(r"^(_Z\S+):\s*(;.*)?$", line)
        if m:
            cur = m.group(1)
            funcs[cur] = []
        elif cur:
            funcs[cur].append(line)
    return funcs


def _loops(body):
    """Instruction lists of the natural loops (label to its backward branch)."""
    out = []
    for i, line in enumerate(body):
        m = re.match(r"^(\.LBB\d+_\d+):.*Loop Header", line)
        if not m:
            continue
        for j in range(i + 1, len(body)):
            if re.search(r"s_cbranch_\w+\s+" + re.escape(m.group(1)) + r"\s*$", body[j]):
                out.append(body[i:j + 1])
                break
    return out


def _is_load(line):
    t = line.strip()
    return t.startswith(("global_load", "buffer_load"))


def test_scale_and_operand_load_counts(asm):
    kern = re.compile(r"_ZN3pf814gemm_mx_kernelILi(\d+)ELi(\d+)ELb(\d)ELb(\d)ELi(\d)ELb(\d)ELb(\d)E")
    checked = 0
    for name, body in _functions(asm).items():
        m = kern.match(name)
        if not m:
            continue
        bm, bn, row_b, _, nst, _, bf16in = (int(x) for x in m.groups())
        wm, wn = bm // 2, bn // 2
        tm, tn = wm // 32, wn // 32
        sb = 1 if (not row_b and 128 % wn == 0) else tn  # one B scale when the wave's columns share a tile
        d = bm // 64 + bn // 64                         # direct-to-LDS loads per stage and wave
        ss = 0 if bf16in else tm + sb                    # scale loads per even stage and wave
        prologue = []
        for line in body:
            if line.strip().startswith("s_barrier"):
                break
            prologue.append(line)
        scale_loads = sum(1 for ln in prologue if ln.strip().startswith("global_load_dword "))
        assert scale_loads == (2 if nst == 5 else 1) * ss, f"{name}: prologue scale loads {scale_loads}"
        loops = _loops(body)
        assert loops, name
        for lp in loops:
            n = sum(1 for ln in lp if _is_load(ln))
            want = 10 * d + 5 * ss if nst == 5 else 2 * d + ss
            assert n == want, f"{name}: a K-loop trip issues {n} loads, expected {want}"
        checked += 1
    assert checked >= 40, checked
