"""The C ABI on the host: the library loads without a GPU, exports every declared symbol, and
rejects bad arguments with the documented status before touching a device (CPU only)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pf8.h")

L = pytest.importorskip("fp8_block_scaled_pf8_amd._lib", reason="libpf8.so not built (run __graft_entry__.build())")

A16 = 0x10000  # fake, aligned device addresses: validation never dereferences them
B16 = 0x20000
C16 = 0x30000
S4 = 0x40000


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|pf8_status|const char\*)\s+(pf8_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert names == sorted(["pf8_quant_act_1x128", "pf8_quant_act_dual", "pf8_quant_fwd", "pf8_quant_w_128x128",
                            "pf8_block_gemm",
                            "pf8_block_gemm_variant", "pf8_block_gemm_f32", "pf8_gemm_bf16", "pf8_strerror",
                            "pf8_abi_version"])
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.SIGNATURES)


def test_constants_match_header():
    text = open(HEADER).read()
    defs = dict(re.findall(r"#define\s+(PF8_\w+)\s+(\d+)", text))
    for name in ["PF8_OK", "PF8_EINVAL", "PF8_ESHAPE", "PF8_EALIGN", "PF8_ENODEV", "PF8_ELAUNCH", "PF8_ALONG_COLS",
                 "PF8_ALONG_ROWS", "PF8_FPROP", "PF8_DGRAD", "PF8_WGRAD", "PF8_GEMM_AUTO", "PF8_GEMM_MX_SCALED",
                 "PF8_GEMM_PROMOTE"]:
        assert int(defs[name]) == getattr(L, name), name
    assert int(defs["PF8_ABI_VERSION"]) == L.pf8_abi_version() == L.ABI_VERSION


def test_strerror_covers_every_status():
    msgs = {s: L.pf8_strerror(s) for s in range(6)}
    assert len(set(msgs.values())) == 6
    assert L.pf8_strerror(99) == "unknown status"
    assert L.pf8_strerror(-1) == "unknown status"


def _qa(**kw):
    a = dict(x=A16, rows=256, cols=512, ldx=512, axis=L.PF8_ALONG_COLS, q=B16, ldq=512, dscale=S4, ld_s=256)
    a.update(kw)
    return L.pf8_quant_act_1x128(a["x"], a["rows"], a["cols"], a["ldx"], a["axis"], a["q"], a["ldq"], a["dscale"],
                                 a["ld_s"], 0)


def test_quant_act_validation():
    assert _qa(x=0) == L.PF8_EINVAL
    assert _qa(q=0) == L.PF8_EINVAL
    assert _qa(dscale=0) == L.PF8_EINVAL
    assert _qa(axis=2) == L.PF8_EINVAL
    assert _qa(rows=0) == L.PF8_EINVAL
    assert _qa(cols=-128) == L.PF8_EINVAL
    assert _qa(ldx=256) == L.PF8_EINVAL
    assert _qa(cols=500, ldx=512, ldq=512) == L.PF8_ESHAPE
    assert _qa(ldq=256) == L.PF8_EINVAL
    assert _qa(ld_s=100) == L.PF8_EINVAL
    assert _qa(x=A16 + 2) == L.PF8_EALIGN
    assert _qa(q=B16 + 8) == L.PF8_EALIGN
    assert _qa(dscale=S4 + 2) == L.PF8_EALIGN
    assert _qa(ldx=516) == L.PF8_EALIGN  # 1032-byte pitch
    assert _qa(ldq=520) == L.PF8_EALIGN
    # col mode: rows must be a multiple of 128 and cols of 8; q is [cols, rows]
    assert _qa(axis=L.PF8_ALONG_ROWS, rows=200, ldq=512, ld_s=512) == L.PF8_ESHAPE
    assert _qa(axis=L.PF8_ALONG_ROWS, cols=508, ldx=512, ldq=256, ld_s=508) == L.PF8_ESHAPE
    assert _qa(axis=L.PF8_ALONG_ROWS, ldq=128, ld_s=512) == L.PF8_EINVAL
    assert _qa(axis=L.PF8_ALONG_ROWS, ldq=256, ld_s=500) == L.PF8_EINVAL


def _qd(**kw):
    a = dict(x=A16, rows=256, cols=384, ldx=384, qr=B16, ldqr=384, sr=S4, ld_sr=256, qc=C16, ldqc=256, sc=S4,
             ld_sc=384)
    a.update(kw)
    return L.pf8_quant_act_dual(a["x"], a["rows"], a["cols"], a["ldx"], a["qr"], a["ldqr"], a["sr"], a["ld_sr"],
                                a["qc"], a["ldqc"], a["sc"], a["ld_sc"], 0)


def test_quant_dual_validation():
    for key in ["x", "qr", "sr", "qc", "sc"]:
        assert _qd(**{key: 0}) == L.PF8_EINVAL, key
    assert _qd(rows=0) == L.PF8_EINVAL
    assert _qd(cols=-128) == L.PF8_EINVAL
    assert _qd(rows=200) == L.PF8_ESHAPE  # both dimensions are grouped
    assert _qd(cols=200, ldx=384) == L.PF8_ESHAPE
    assert _qd(ldx=256) == L.PF8_EINVAL
    assert _qd(ldqr=256) == L.PF8_EINVAL
    assert _qd(ld_sr=128) == L.PF8_EINVAL
    assert _qd(ldqc=128) == L.PF8_EINVAL
    assert _qd(ld_sc=256) == L.PF8_EINVAL
    assert _qd(x=A16 + 2) == L.PF8_EALIGN
    assert _qd(qr=B16 + 8) == L.PF8_EALIGN
    assert _qd(qc=C16 + 4) == L.PF8_EALIGN
    assert _qd(sc=S4 + 2) == L.PF8_EALIGN
    assert _qd(ldx=388) == L.PF8_EALIGN  # 776-byte pitch
    assert _qd(ldqc=264) == L.PF8_EALIGN


def _qf(**kw):
    a = dict(x=A16, m=256, k=384, ldx=384, qx=B16, ldqx=384, sx=S4, ld_sx=256, qxt=C16, ldqxt=256, sxt=S4,
             ld_sxt=384, w=A16, n=512, ldw=384, qw=B16, ldqw=384, qwt=C16, ldqwt=512, sw=S4, ld_sw=3)
    a.update(kw)
    return L.pf8_quant_fwd(a["x"], a["m"], a["k"], a["ldx"], a["qx"], a["ldqx"], a["sx"], a["ld_sx"], a["qxt"],
                           a["ldqxt"], a["sxt"], a["ld_sxt"], a["w"], a["n"], a["ldw"], a["qw"], a["ldqw"], a["qwt"],
                           a["ldqwt"], a["sw"], a["ld_sw"], 0)


def test_quant_fwd_validation():
    for key in ["x", "qx", "sx", "qxt", "sxt", "w", "qw", "sw"]:
        assert _qf(**{key: 0}) == L.PF8_EINVAL, key
    assert _qf(m=0) == L.PF8_EINVAL
    assert _qf(m=200) == L.PF8_ESHAPE
    assert _qf(n=200) == L.PF8_ESHAPE
    assert _qf(k=200, ldx=384, ldw=384) == L.PF8_ESHAPE
    assert _qf(ldx=256) == L.PF8_EINVAL
    assert _qf(ld_sx=128) == L.PF8_EINVAL
    assert _qf(ldqxt=128) == L.PF8_EINVAL
    assert _qf(ld_sw=2) == L.PF8_EINVAL
    assert _qf(ldqwt=256) == L.PF8_EINVAL
    assert _qf(x=A16 + 2) == L.PF8_EALIGN
    assert _qf(qwt=C16 + 4) == L.PF8_EALIGN
    assert _qf(ldw=388) == L.PF8_EALIGN


def _qw(**kw):
    a = dict(w=A16, n=256, k=384, ldw=384, q=B16, ldq=384, qt=C16, ldqt=256, dscale=S4, ld_s=3)
    a.update(kw)
    return L.pf8_quant_w_128x128(a["w"], a["n"], a["k"], a["ldw"], a["q"], a["ldq"], a["qt"], a["ldqt"], a["dscale"],
                                 a["ld_s"], 0)


def test_quant_w_validation():
    assert _qw(w=0) == L.PF8_EINVAL
    assert _qw(q=0) == L.PF8_EINVAL
    assert _qw(dscale=0) == L.PF8_EINVAL
    assert _qw(n=0) == L.PF8_EINVAL
    assert _qw(n=200) == L.PF8_ESHAPE
    assert _qw(k=200, ldw=384) == L.PF8_ESHAPE
    assert _qw(ldw=256) == L.PF8_EINVAL
    assert _qw(ld_s=2) == L.PF8_EINVAL
    assert _qw(ldqt=128) == L.PF8_EINVAL
    assert _qw(qt=C16 + 4) == L.PF8_EALIGN
    assert _qw(ldqt=264) == L.PF8_EALIGN
    assert _qw(ldw=388) == L.PF8_EALIGN  # 776-byte pitch


def _gm(**kw):
    a = dict(variant=L.PF8_GEMM_AUTO, layout=L.PF8_FPROP, m=256, n=384, k=512, a=A16, lda=512, a_dscale=S4, ld_as=256,
             b=B16, ldb=512, b_dscale=S4, sb_n=4, sb_k=1, d=C16, ldd=384)
    a.update(kw)
    return L.pf8_block_gemm_variant(a["variant"], a["layout"], a["m"], a["n"], a["k"], a["a"], a["lda"], a["a_dscale"],
                                    a["ld_as"], a["b"], a["ldb"], a["b_dscale"], a["sb_n"], a["sb_k"], a["d"], a["ldd"],
                                    0)


def test_gemm_validation():
    assert _gm(variant=3) == L.PF8_EINVAL
    assert _gm(layout=7) == L.PF8_EINVAL
    for key in ["a", "b", "d", "a_dscale", "b_dscale"]:
        assert _gm(**{key: 0}) == L.PF8_EINVAL, key
    assert _gm(m=0) == L.PF8_EINVAL
    assert _gm(n=-1) == L.PF8_EINVAL
    assert _gm(k=0) == L.PF8_EINVAL
    assert _gm(k=500, lda=512, ldb=512) == L.PF8_ESHAPE
    assert _gm(lda=256) == L.PF8_EINVAL
    assert _gm(ldb=256) == L.PF8_EINVAL
    assert _gm(ldd=100) == L.PF8_EINVAL
    assert _gm(ld_as=100) == L.PF8_EINVAL
    assert _gm(sb_n=0) == L.PF8_EINVAL
    assert _gm(sb_k=0) == L.PF8_EINVAL
    assert _gm(a=A16 + 1) == L.PF8_EALIGN
    assert _gm(d=C16 + 8) == L.PF8_EALIGN
    assert _gm(b_dscale=S4 + 1) == L.PF8_EALIGN
    assert _gm(lda=520) == L.PF8_EALIGN
    assert _gm(ldd=388) == L.PF8_EALIGN  # 776-byte pitch
    assert _gm(lda=1 << 24, ldb=1 << 24) == L.PF8_ESHAPE  # pitch beyond the 32-bit tile offset range


def _gf(**kw):
    a = dict(layout=L.PF8_WGRAD, m=256, n=384, k=512, a=A16, lda=512, a_dscale=S4, ld_as=256, b=B16, ldb=512,
             b_dscale=S4, sb_n=1, sb_k=384, d=C16, ldd=384, accumulate=1)
    a.update(kw)
    return L.pf8_block_gemm_f32(a["layout"], a["m"], a["n"], a["k"], a["a"], a["lda"], a["a_dscale"], a["ld_as"],
                                a["b"], a["ldb"], a["b_dscale"], a["sb_n"], a["sb_k"], a["d"], a["ldd"],
                                a["accumulate"], 0)


def test_gemm_f32_validation():
    assert _gf(layout=5) == L.PF8_EINVAL
    assert _gf(accumulate=2) == L.PF8_EINVAL
    assert _gf(accumulate=-1) == L.PF8_EINVAL
    for key in ["a", "b", "d", "a_dscale", "b_dscale"]:
        assert _gf(**{key: 0}) == L.PF8_EINVAL, key
    assert _gf(m=0) == L.PF8_EINVAL
    assert _gf(k=200, lda=512, ldb=512) == L.PF8_ESHAPE
    assert _gf(ldd=300) == L.PF8_EINVAL
    assert _gf(ld_as=128) == L.PF8_EINVAL
    assert _gf(d=C16 + 8) == L.PF8_EALIGN
    assert _gf(ldd=386) == L.PF8_EALIGN  # 1544-byte pitch
    assert _gf(a=A16 + 4) == L.PF8_EALIGN
    assert _gf(lda=1 << 24, ldb=1 << 24) == L.PF8_ESHAPE


def _gb(**kw):
    a = dict(m=256, n=384, k=512, a=A16, lda=512, b=B16, ldb=512, d=C16, ldd=384)
    a.update(kw)
    return L.pf8_gemm_bf16(a["m"], a["n"], a["k"], a["a"], a["lda"], a["b"], a["ldb"], a["d"], a["ldd"], 0)


def test_gemm_bf16_validation():
    for key in ["a", "b", "d"]:
        assert _gb(**{key: 0}) == L.PF8_EINVAL, key
    assert _gb(n=0) == L.PF8_EINVAL
    assert _gb(k=200, lda=512, ldb=512) == L.PF8_ESHAPE
    assert _gb(lda=256) == L.PF8_EINVAL
    assert _gb(ldd=300) == L.PF8_EINVAL
    assert _gb(a=A16 + 2) == L.PF8_EALIGN
    assert _gb(lda=516) == L.PF8_EALIGN  # 1032-byte pitch
    assert _gb(ldd=388) == L.PF8_EALIGN
    assert _gb(lda=1 << 23, ldb=1 << 23) == L.PF8_ESHAPE


def test_no_device_is_reported_after_validation():
    # valid arguments pass validation and then find no device; with a GPU present these fake
    # addresses would reach a kernel, so this runs only where there is none
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _qa(rows=3, ld_s=3) == L.PF8_ENODEV  # row mode accepts any row count
    assert _qw(qt=0, ldqt=0) == L.PF8_ENODEV  # no transposed copy requested
    assert _gm(m=1, n=3, ld_as=1, ldd=8) == L.PF8_ENODEV  # ragged M and N are accepted
    assert _qa() == L.PF8_ENODEV
    assert _qd() == L.PF8_ENODEV
    assert _qf() == L.PF8_ENODEV
    assert _qf(qwt=0, ldqwt=0) == L.PF8_ENODEV
    assert _gf() == L.PF8_ENODEV
    assert _gb() == L.PF8_ENODEV
    assert _gf(accumulate=0, m=3, n=5, ld_as=3, ldd=8) == L.PF8_ENODEV
    assert _qw() == L.PF8_ENODEV
    assert _gm() == L.PF8_ENODEV
    assert L.pf8_block_gemm(L.PF8_WGRAD, 256, 384, 512, A16, 512, S4, 256, B16, 512, S4, 1, 4, C16, 384, 0) == \
        L.PF8_ENODEV


def test_size_limits_are_exact():
    """The largest accepted sizes pass validation (and then find no device here); one step beyond
    is PF8_ESHAPE. Limits: 65535 grid rows of 128-groups in the quantisers, and a row pitch whose
    256-row tile offsets fit a signed 32-bit offset in the GEMMs."""
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present (the fake addresses would reach a kernel)")
    gmax = 65535 * 128
    pmax = ((1 << 31) - 1) // 256
    kmax = pmax // 128 * 128
    # row mode: one grid row per 128-group of a row
    assert _qa(rows=1, cols=gmax, ldx=gmax, ldq=gmax, ld_s=1) == L.PF8_ENODEV
    assert _qa(rows=1, cols=gmax + 128, ldx=gmax + 128, ldq=gmax + 128, ld_s=1) == L.PF8_ESHAPE
    # col mode: one grid row per 128-row band
    assert _qa(axis=L.PF8_ALONG_ROWS, rows=gmax, cols=8, ldx=8, ldq=gmax, ld_s=8) == L.PF8_ENODEV
    assert _qa(axis=L.PF8_ALONG_ROWS, rows=gmax + 128, cols=8, ldx=8, ldq=gmax + 128, ld_s=8) == L.PF8_ESHAPE
    # dual: grid rows are the 128-row bands
    assert _qd(rows=gmax, cols=128, ldx=128, ldqr=128, ld_sr=gmax, ldqc=gmax, ld_sc=128) == L.PF8_ENODEV
    assert _qd(rows=gmax + 128, cols=128, ldx=128, ldqr=128, ld_sr=gmax + 128, ldqc=gmax + 128,
               ld_sc=128) == L.PF8_ESHAPE
    # weight tiles: one grid row per 128-row tile band
    assert _qw(n=gmax, k=128, ldw=128, ldq=128, ldqt=gmax, ld_s=1) == L.PF8_ENODEV
    assert _qw(n=gmax + 128, k=128, ldw=128, ldq=128, ldqt=gmax + 128, ld_s=1) == L.PF8_ESHAPE
    # GEMM row pitch (FP8 codes: bytes; the BF16 GEMM's pitch is in elements of 2 bytes)
    assert _gm(m=3, n=2, k=kmax, lda=pmax // 16 * 16, ldb=kmax, ld_as=3, ldd=8, sb_n=kmax // 128) == L.PF8_ENODEV
    assert _gm(m=3, n=2, k=kmax, lda=pmax // 16 * 16 + 16, ldb=kmax, ld_as=3, ldd=8,
               sb_n=kmax // 128) == L.PF8_ESHAPE
    assert _gf(m=3, n=2, k=kmax, lda=kmax, ldb=kmax, ld_as=3, sb_n=1, sb_k=2, ldd=4) == L.PF8_ENODEV
    assert _gf(m=3, n=2, k=kmax + 128, lda=kmax + 128, ldb=kmax + 128, ld_as=3, sb_n=1, sb_k=2,
               ldd=4) == L.PF8_ESHAPE
