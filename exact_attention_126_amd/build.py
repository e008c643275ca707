"""Builds libfa.so (C ABI + gfx950 HIP kernels) in-tree with hipcc, and libfa_calib.so, the
sustained matrix-core rate probe that the benchmark reports beside the nominal peak.

    python -m exact_attention_126_amd.build [--save-temps]

The object code targets gfx950 only.  Packed fp32 VALU instructions are disabled for all
device code (-packed-fp32-ops).  Each source is compiled to its own object, with the options of
SOURCE_FLAGS where it has any, and the objects are linked into the shared library.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")
SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_fwd_fp8.hip", "fa_decode.hip", "fa_bwd.hip", "fa_mask.hip"]
# Per-source code generation options.  The dK/dV kernel runs one wave per SIMD and feeds its S and
# dP accumulators straight to VALU arithmetic, so its matrix instructions are selected in the form
# that accumulates in VGPRs (otherwise every tile's S and dP are copied out of the AGPRs).
SOURCE_FLAGS = {"fa_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
CALIB_LIB = os.path.join(PKG, "libfa_calib.so")
# The same sources built with FA_DEBUG_POISON_LDS=1 (retired LDS ring slots overwritten with NaN
# before they are refilled); a test checks that it gives the normal library's outputs bit for bit.
POISON_LIB = os.path.join(PKG, "libfa_poison.so")
CALIB_SOURCES = ["calib_mfma.hip"]


def hipcc() -> str:
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def flags(save_temps: bool = False):
    f = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC]
    if save_temps:
        f.append("--save-temps")
    return f


def _run(cmd, verbose: bool, cwd=None):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=cwd)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless.
    err = "\n".join(ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False, save_temps: bool = False, out: str = LIB, sources=None, extra=()) -> str:
    """Compiles every source to an object (in parallel, each with its own options and extra), then links."""
    names = sources or SOURCES
    objdir = tempfile.mkdtemp(prefix="fa_build_")
    fd, tmp = tempfile.mkstemp(suffix=".so.tmp", dir=os.path.dirname(out))
    os.close(fd)
    try:
        objs = [os.path.join(objdir, n + ".o") for n in names]
        cmds = [[hipcc(), *flags(save_temps), *SOURCE_FLAGS.get(n, []), *extra, "-c", "-o", o, os.path.join(CSRC, n)]
                for n, o in zip(names, objs)]
        workers = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", "0")) or len(os.sched_getaffinity(0))))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            for f in [ex.submit(_run, c, verbose, objdir) for c in cmds]:
                f.result()
        _run([hipcc(), "--hip-link", "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp,
              *objs], verbose)
        os.replace(tmp, out)
    finally:
        if os.path.exists(tmp):
            os.remove(tmp)
        if not save_temps:
            shutil.rmtree(objdir, ignore_errors=True)
    if save_temps:
        print("temps in", objdir)
    return out


def build_calib(verbose: bool = False) -> str:
    return build(verbose=verbose, out=CALIB_LIB, sources=CALIB_SOURCES)


def build_poison(verbose: bool = False) -> str:
    return build(verbose=verbose, out=POISON_LIB, extra=("-DFA_DEBUG_POISON_LDS=1",))


if __name__ == "__main__":
    build(verbose=True, save_temps="--save-temps" in sys.argv)
    build_calib(verbose=True)
    build_poison(verbose=True)
