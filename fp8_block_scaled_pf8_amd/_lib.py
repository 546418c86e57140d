"""ctypes binding of libpf8 (include/pf8.h): the C entry points under the same names.

Argument marshalling only: pointers are passed as Python ints (device addresses), sizes as
ints, the stream as a hipStream_t handle (int, 0 = null stream). Every function returns the
library's int status; ``check`` turns a non-zero status into a RuntimeError.

Loading fails loudly (ImportError) when libpf8.so has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

# libpf8 must run on the same HIP runtime as PyTorch (the streams and device pointers it receives
# come from PyTorch). Loading PyTorch first makes the dynamic linker resolve libpf8's
# libamdhip64.so.7 to PyTorch's copy instead of pulling in a second runtime.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpf8.so")

PF8_OK, PF8_EINVAL, PF8_ESHAPE, PF8_EALIGN, PF8_ENODEV, PF8_ELAUNCH = range(6)
PF8_ALONG_COLS, PF8_ALONG_ROWS = 0, 1
PF8_FPROP, PF8_DGRAD, PF8_WGRAD = 0, 1, 2
PF8_GEMM_AUTO, PF8_GEMM_MX_SCALED, PF8_GEMM_PROMOTE = 0, 1, 2
ABI_VERSION = 5

_i64 = ctypes.c_int64
_int = ctypes.c_int
_vp = ctypes.c_void_p

# name -> (restype, argtypes); mirrors include/pf8.h
SIGNATURES = {
    "pf8_quant_act_1x128": (_int, [_vp, _i64, _i64, _i64, _int, _vp, _i64, _vp, _i64, _vp]),
    "pf8_quant_act_dual": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]),
    "pf8_quant_fwd": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _vp,
                             _i64, _vp, _i64, _vp, _i64, _vp]),
    "pf8_quant_w_128x128": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]),
    "pf8_block_gemm": (_int, [_int, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _vp, _i64, _vp]),
    "pf8_block_gemm_variant": (
        _int, [_int, _int, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _vp, _i64, _vp]),
    "pf8_block_gemm_f32": (
        _int, [_int, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _vp, _i64, _int, _vp]),
    "pf8_gemm_bf16": (_int, [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]),
    "pf8_strerror": (ctypes.c_char_p, [_int]),
    "pf8_abi_version": (_int, []),
}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libpf8.so is not built ({LIB_PATH}); run `python fp8_block_scaled_pf8_amd/build.py` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.pf8_abi_version() != ABI_VERSION:
        raise ImportError(f"libpf8 ABI version {lib.pf8_abi_version()} != {ABI_VERSION}")
    return lib


LIB = _load()


def pf8_quant_act_1x128(x, rows, cols, ldx, axis, q, ldq, dscale, ld_s, hip_stream=0) -> int:
    return LIB.pf8_quant_act_1x128(x, rows, cols, ldx, axis, q, ldq, dscale, ld_s, hip_stream)


def pf8_quant_act_dual(x, rows, cols, ldx, q_row, ldq_row, dscale_row, ld_sr, q_col, ldq_col, dscale_col, ld_sc,
                       hip_stream=0) -> int:
    return LIB.pf8_quant_act_dual(x, rows, cols, ldx, q_row, ldq_row, dscale_row, ld_sr, q_col, ldq_col, dscale_col,
                                  ld_sc, hip_stream)


def pf8_quant_fwd(x, m, k, ldx, qx, ldqx, sx, ld_sx, qxt, ldqxt, sxt, ld_sxt, w, n, ldw, qw, ldqw, qwt, ldqwt, sw,
                  ld_sw, hip_stream=0) -> int:
    return LIB.pf8_quant_fwd(x, m, k, ldx, qx, ldqx, sx, ld_sx, qxt, ldqxt, sxt, ld_sxt, w, n, ldw, qw, ldqw, qwt,
                             ldqwt, sw, ld_sw, hip_stream)


def pf8_quant_w_128x128(w, n, k, ldw, q, ldq, qt, ldqt, dscale, ld_s, hip_stream=0) -> int:
    return LIB.pf8_quant_w_128x128(w, n, k, ldw, q, ldq, qt, ldqt, dscale, ld_s, hip_stream)


def pf8_block_gemm(layout, m, n, k, a, lda, a_dscale, ld_as, b, ldb, b_dscale, sb_n, sb_k, d, ldd,
                   hip_stream=0) -> int:
    return LIB.pf8_block_gemm(layout, m, n, k, a, lda, a_dscale, ld_as, b, ldb, b_dscale, sb_n, sb_k, d, ldd,
                              hip_stream)


def pf8_block_gemm_variant(variant, layout, m, n, k, a, lda, a_dscale, ld_as, b, ldb, b_dscale, sb_n, sb_k, d,
                           ldd, hip_stream=0) -> int:
    return LIB.pf8_block_gemm_variant(variant, layout, m, n, k, a, lda, a_dscale, ld_as, b, ldb, b_dscale, sb_n,
                                      sb_k, d, ldd, hip_stream)


def pf8_block_gemm_f32(layout, m, n, k, a, lda, a_dscale, ld_as, b, ldb, b_dscale, sb_n, sb_k, d, ldd, accumulate,
                       hip_stream=0) -> int:
    return LIB.pf8_block_gemm_f32(layout, m, n, k, a, lda, a_dscale, ld_as, b, ldb, b_dscale, sb_n, sb_k, d, ldd,
                                  accumulate, hip_stream)


def pf8_gemm_bf16(m, n, k, a, lda, b, ldb, d, ldd, hip_stream=0) -> int:
    return LIB.pf8_gemm_bf16(m, n, k, a, lda, b, ldb, d, ldd, hip_stream)


def pf8_strerror(status: int) -> str:
    return LIB.pf8_strerror(status).decode()


def pf8_abi_version() -> int:
    return LIB.pf8_abi_version()


def check(status: int, what: str = "libpf8") -> None:
    if status != PF8_OK:
        raise RuntimeError(f"{what}: {pf8_strerror(status)} (status {status})")
