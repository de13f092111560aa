"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

* api.cpp (argument validation, kernel-family choice, grid sizing) linked with recording stubs
  of the kernel launchers (tests/native/api_fuzz.cpp): random valid, edge and invalid arguments
  for every entry point; a refused call launches nothing, an accepted one hands the kernels a
  consistent launch.
* vmm.cpp (the virtual-memory pool's bookkeeping) linked with a host model of HIP's virtual
  memory calls (tests/native/vmm_fuzz.cpp): every reservation, mapping, access change, copy and
  release is checked against the model, failures are injected, and destroy leaves nothing.

Both are compiled for the host only (no device code is built); the harness that stands in for
a C caller passes enum arguments outside their enumerators, which C allows, so only its own
translation unit is built without the enum check."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CXX = shutil.which("amdclang++") or os.path.join(ROCM, "bin", "amdclang++")
CSRC = os.path.join(ROOT, "paged_kv_cache_247_amd", "csrc")
NATIVE = os.path.join(ROOT, "tests", "native")
HOST_ONLY = ["-x", "hip", "--offload-host-only", "--offload-arch=gfx950", "-std=c++17", "-O1",
             "-g", "-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host",
             "-fno-sanitize-recover=undefined", "-fno-gpu-sanitize", "-fno-omit-frame-pointer",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
HIP_RUNTIME = ["-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"]


def _build(tmp_path, name, units, libs=()):
    objs = []
    for src, extra in units:
        obj = tmp_path / (os.path.basename(src) + ".o")
        r = subprocess.run([CXX, *HOST_ONLY, *extra, "-c", src, "-o", str(obj)],
                           capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(str(obj))
    exe = tmp_path / name
    r = subprocess.run([CXX, *objs, "-fsanitize=address,undefined", *libs, "-o", str(exe)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    return str(exe)


def _run(exe, ok_line):
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and ok_line in r.stdout, out[-3000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-3000:]


@pytest.mark.skipif(not os.path.exists(CXX), reason="amdclang++ not found")
def test_api_validation_under_sanitizers(tmp_path):
    exe = _build(tmp_path, "api_fuzz", [
        (os.path.join(CSRC, "api.cpp"), []),
        (os.path.join(NATIVE, "api_fuzz.cpp"), ["-Xarch_host", "-fno-sanitize=enum"])],
        HIP_RUNTIME)  # hipGetErrorString
    _run(exe, "api fuzz ok")


@pytest.mark.skipif(not os.path.exists(CXX), reason="amdclang++ not found")
def test_vmm_pool_bookkeeping_under_sanitizers(tmp_path):
    exe = _build(tmp_path, "vmm_fuzz", [
        (os.path.join(CSRC, "vmm.cpp"), []),
        (os.path.join(NATIVE, "vmm_fuzz.cpp"), []),
        (os.path.join(NATIVE, "host_error_stubs.cpp"), [])])  # no HIP runtime: the model only
    _run(exe, "vmm fuzz ok")
