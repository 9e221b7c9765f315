"""The C ABI's host layer (argument checks, map carving, workspace and
scratch layout) under AddressSanitizer, on the CPU.

pba_api.cpp is rebuilt with its host half instrumented and linked, with the
library's other objects as built, into tests/asan_abi_driver.cpp, which
drives every host-side rejection path (no device work is ever enqueued).  The
run must exit 0 with no AddressSanitizer report."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "block_sparse_attention_pack_amd")
ROCM = "/opt/rocm"
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
# Host-only instrumentation: -Xarch_host directly before each sanitizer flag.
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm toolchain not installed")
def test_host_layer_under_asan(tmp_path):
    from block_sparse_attention_pack_amd.build import BUILD, FLAGS, SOURCES, build
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "pba_api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        build()
    api_o = str(tmp_path / "pba_api_asan.o")
    drv_o = str(tmp_path / "driver_asan.o")
    exe = str(tmp_path / "abi_asan")
    _run([HIPCC, *FLAGS, "-g", "-O1", *HOST_ASAN, "-x", "hip", "-c", os.path.join(PKG, "csrc", "pba_api.cpp"),
          "-o", api_o])
    _run([CLANGXX, "-std=c++17", "-g", "-O1", "-fsanitize=address", "-fno-omit-frame-pointer", "-c",
          os.path.join(ROOT, "tests", "asan_abi_driver.cpp"), "-o", drv_o])
    _run([CLANGXX, "-fsanitize=address", drv_o, api_o, *objs, "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
          "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out
    assert r.returncode == 0, out
    assert "ok: 0 failed checks" in r.stdout, out
