"""Build libmla.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc, and
libmla_debug.so, the same sources with the MLA_DEBUG_BOUNDS device checks.

    python -m mla_latent_kv_05_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmla.so")
DEBUG_LIB = os.path.join(PKG, "libmla_debug.so")
OBJDIR = os.path.join(PKG, "_build")
SOURCES = ["mla_api.cpp", "kernels_generic.hip", "kernels_mfma.hip", "kernels_decode.hip",
           "kernels_decode8.hip", "kernels_decode128.hip", "kernels_append.hip", "kernels_prefill.hip",
           "kernels_expand.hip", "kernels_step_persistent.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          # no packed-fp32 VALU instructions in device code
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function"]


def _compile(src: str, debug: bool) -> str:
    obj = os.path.join(OBJDIR, ("debug_" if debug else "") + os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + (["-DMLA_DEBUG_BOUNDS"] if debug else []) + ["-x", "hip", "-c", os.path.join(CSRC, src),
                                                                       "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = [(src, dbg) for dbg in (False, True) for src in SOURCES]
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    n = len(SOURCES)
    _link(objs[:n], LIB)
    _link(objs[n:], DEBUG_LIB)
    if verbose:
        print(f"built {LIB} and {DEBUG_LIB}")
    return LIB


def clean() -> None:
    shutil.rmtree(OBJDIR, ignore_errors=True)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
