"""Builds libfa.so (C ABI + gfx950 HIP kernels) in-tree with hipcc, and libfa_calib.so, the
sustained matrix-core rate probe that the benchmark reports beside the nominal peak.

    python -m exact_attention_126_amd.build [--save-temps]

The object code targets gfx950 only.  Packed fp32 VALU instructions are disabled for all
device code (-packed-fp32-ops).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")
SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_fwd_fp8.hip", "fa_decode.hip", "fa_bwd.hip", "fa_mask.hip"]
CALIB_LIB = os.path.join(PKG, "libfa_calib.so")
CALIB_SOURCES = ["calib_mfma.hip"]


def hipcc() -> str:
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def flags(save_temps: bool = False):
    f = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-result", "-Wl,--no-undefined", "-I", INCLUDE, "-I", CSRC]
    if save_temps:
        f.append("--save-temps")
    return f


def build(verbose: bool = False, save_temps: bool = False, out: str = LIB, sources=None) -> str:
    srcs = [os.path.join(CSRC, s) for s in (sources or SOURCES)]
    fd, tmp = tempfile.mkstemp(suffix=".so.tmp", dir=os.path.dirname(out))
    os.close(fd)
    cmd = [hipcc(), *flags(save_temps), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    cwd = tempfile.mkdtemp(prefix="fa_build_") if save_temps else None
    try:
        r = subprocess.run(cmd, capture_output=True, text=True, cwd=cwd)
        # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless.
        err = "\n".join(ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
        os.replace(tmp, out)
    finally:
        if os.path.exists(tmp):
            os.remove(tmp)
    if save_temps:
        print("temps in", cwd)
    return out


def build_calib(verbose: bool = False) -> str:
    return build(verbose=verbose, out=CALIB_LIB, sources=CALIB_SOURCES)


if __name__ == "__main__":
    build(verbose=True, save_temps="--save-temps" in sys.argv)
    build_calib(verbose=True)
