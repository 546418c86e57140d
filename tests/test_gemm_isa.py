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


def test_whole_kernel_load_totals_match_the_stage_layout(asm):
    """Every load the stage layout issues, counted over the whole kernel: the five prologue and
    head paths (head length h = 1, 3, 5, 7, 9), the K loop and the tail. This covers the head
    stages, whose refills carry scale loads under the same explicit waits.

    Per path with five buffers: stages 0..3 whole plus stage 4's A part (4 D + A_DMA direct-to-LDS
    loads, scales of stages 0 and 2), then h head stages, each finishing one refill and starting
    the next (D loads, scales when the finished refill's stage is even, i.e. for (h + 1) / 2 of
    them). The loop trip holds 10 D loads and 5 scale sets; the tail finishes the last refill
    (B_DMA loads of an odd stage, no scales). With two buffers: stage 0 and stage 1's A part, a
    two-stage loop trip, and the tail's B part."""
    kern = re.compile(r"_ZN3pf814gemm_mx_kernelILi(\d+)ELi(\d+)ELb(\d)ELb(\d)ELi(\d)ELb(\d)ELb(\d)E")
    checked = 0
    for name, body in _functions(asm).items():
        m = kern.match(name)
        if not m:
            continue
        bm, bn, row_b, _, nst, f32, bf16in = (int(x) for x in m.groups())
        wm, wn = bm // 2, bn // 2
        tm, tn = wm // 32, wn // 32
        sb = 1 if (not row_b and 128 % wn == 0) else tn
        a_dma, b_dma = bm // 64, bn // 64
        d = a_dma + b_dma
        ss = 0 if bf16in else tm + sb
        heads = (1, 3, 5, 7, 9)
        if nst == 5:
            want_lds = sum(4 * d + a_dma + h * d for h in heads) + 10 * d + b_dma
            want_scale = sum(2 * ss + (h + 1) // 2 * ss for h in heads) + 5 * ss
        else:
            want_lds = d + a_dma + 2 * d + b_dma
            want_scale = ss + ss
        lds = sum(1 for ln in body if ln.strip().startswith("buffer_load_dword") and " lds" in ln)
        scale = sum(1 for ln in body if ln.strip().startswith("global_load_dword "))
        assert lds == want_lds, f"{name}: {lds} direct-to-LDS loads, expected {want_lds}"
        if f32:
            # the FP32 epilogue's edge path reads old values one float at a time with the same opcode
            assert scale >= want_scale, f"{name}: {scale} dword loads, expected at least {want_scale}"
        else:
            assert scale == want_scale, f"{name}: {scale} scale loads, expected {want_scale}"
        checked += 1
    assert checked >= 40, checked


def _inner_loops(body):
    """Natural loops whose header label is followed (on its line or the next) by a 'Loop Header'
    comment and which contain no other loop header."""
    out = []
    for i, line in enumerate(body):
        m = re.match(r"^(\.LBB\d+_\d+):", line)
        if not m or not any("Loop Header" in ln for ln in body[i:i + 2]):
            continue
        for j in range(i + 1, len(body)):
            if re.search(r"s_cbranch_\w+\s+" + re.escape(m.group(1)) + r"\s*$", body[j]):
                inner = body[i + 2:j]
                if not any("Loop Header" in ln for ln in inner):
                    out.append(body[i:j + 1])
                break
    return out


def test_persistent_kernel_load_counts(asm):
    """The persistent kernel's waits count its loads per stage and the output stores per tile.

    Over the whole kernel: the prologue's four stages (4 D direct-to-LDS loads, scales of stages 0
    and 2), tile 0's first body, the K loop body, the last body and the next tile's first body
    (4 A + 3 B, 4 D, 4 A + 5 B and 4 A + 3 B loads; two scale sets each), i.e. 20 A_DMA + 19 B_DMA
    direct-to-LDS loads and 10 scale sets; 8 stores per thread and 64-row slab. The K loop's trip
    holds four stages: 4 D loads and two scale sets."""
    kern = re.compile(r"_ZN3pf825gemm_mx_persistent_kernelILi(\d+)ELb(\d)E")
    checked = 0
    for name, body in _functions(asm).items():
        m = kern.match(name)
        if not m:
            continue
        bm, row_b = int(m.group(1)), int(m.group(2))
        a_dma, b_dma, tm = bm // 64, 4, bm // 64
        ss = tm + (4 if row_b else 1)
        lds = sum(1 for ln in body if ln.strip().startswith("buffer_load_dword") and " lds" in ln)
        scale = sum(1 for ln in body if ln.strip().startswith("global_load_dword "))
        stores = sum(1 for ln in body if ln.strip().startswith(("global_store", "buffer_store")))
        assert lds == 20 * a_dma + 19 * b_dma, f"{name}: {lds} direct-to-LDS loads"
        assert scale == 10 * ss, f"{name}: {scale} scale loads"
        assert stores == 8 * tm, f"{name}: {stores} stores"
        # the K loops (the staggered start's sleep loop holds no MFMA)
        loops = [lp for lp in _inner_loops(body) if any(ln.strip().startswith("v_mfma") for ln in lp)]
        assert loops, name
        for lp in loops:
            n_lds = sum(1 for ln in lp if ln.strip().startswith("buffer_load_dword") and " lds" in ln)
            n_sc = sum(1 for ln in lp if ln.strip().startswith("global_load_dword "))
            n_st = sum(1 for ln in lp if ln.strip().startswith(("global_store", "buffer_store")))
            assert (n_lds, n_sc, n_st) == (4 * (a_dma + b_dma), 2 * ss, 0), f"{name}: loop trip {n_lds}, {n_sc}, {n_st}"
        checked += 1
    assert checked == 4, checked
