"""Build libpf8.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python fp8_block_scaled_pf8_amd/build.py [--asm DIR]

(run as a file: importing the package first would load the library being rebuilt)

--asm DIR additionally writes the gfx950 assembly of every source into DIR.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
SOURCES = ["quant.hip", "gemm.hip", "abi.hip"]
LIB_NAME = "libpf8.so"
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # keep hipcc from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpf8)")


def lib_path() -> str:
    return os.path.join(PKG_DIR, LIB_NAME)


def build(asm_dir: "str | None" = None, verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libpf8.so next to this file. Returns its path."""
    cc = hipcc()
    out = lib_path()
    tmp = out + ".tmp"
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    cmd = [cc, *HIPCC_FLAGS, "-shared", "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in (res.stderr or "").splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    if verbose and errs:
        print("\n".join(errs), file=sys.stderr)
    os.replace(tmp, out)
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        for s in srcs:
            base = os.path.splitext(os.path.basename(s))[0]
            subprocess.run([cc, *HIPCC_FLAGS, "--cuda-device-only", "-S", "-o", os.path.join(asm_dir, base + ".s"), s],
                           check=True, capture_output=True)
    return out


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--asm", default=None, help="also write gfx950 assembly into this directory")
    args = ap.parse_args()
    print(build(args.asm, verbose=True))


if __name__ == "__main__":
    main()
