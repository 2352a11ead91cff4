"""Host code under AddressSanitizer + UndefinedBehaviorSanitizer (CPU only):
the C ABI's host side (mla_api.cpp: validation, planner, workspace, argument
rejection; built with the sanitizers on its host code only, linked with the
kernel objects of the regular build) and the oracle's C code, each driven by a
small program under tests/sanitize/.  Any sanitizer report fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_latent_kv_05_amd", "csrc")
OBJDIR = os.path.join(ROOT, "mla_latent_kv_05_amd", "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc missing")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    run(["gcc", "-O1", "-g", "-std=c11"] + SAN + [os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
                                                  "-lm", "-o", exe])
    r = run([exe], env=ENV)
    assert "oracle driver ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc missing")
def test_abi_host_code_under_sanitizers(tmp_path):
    objs = sorted(os.path.join(OBJDIR, f) for f in os.listdir(OBJDIR) if f.startswith("kernels_") and f.endswith(".o")) \
        if os.path.isdir(OBJDIR) else []
    if len(objs) < 8:
        from mla_latent_kv_05_amd import build as B
        B.build()
        objs = sorted(os.path.join(OBJDIR, f) for f in os.listdir(OBJDIR) if f.startswith("kernels_") and f.endswith(".o"))
    api = str(tmp_path / "mla_api_san.o")
    host_san = []
    for f in SAN:
        host_san += ["-Xarch_host", f]
    run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"),
         "-I", CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + host_san +
        ["-x", "hip", "-c", os.path.join(CSRC, "mla_api.cpp"), "-o", api])
    exe = str(tmp_path / "abi_driver")
    run(["g++", "-O1", "-g"] + SAN + ["-I", os.path.join(ROOT, "include"),
                                      os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), api] + objs +
        ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    r = run([exe], env=ENV)
    assert "abi driver ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
