"""Build libpagedkv.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree.

    python -m paged_kv_cache_247_amd.build [--jobs N] [--verbose]

Every source is compiled to an object under paged_kv_cache_247_amd/_build/ and the objects are
linked into paged_kv_cache_247_amd/libpagedkv.so; the two decode sources are compiled once per
block size (-DPKV_BLOCK_SIZE=S), so the objects build in parallel. Packed-fp32 instruction
selection is switched off for all device code (-packed-fp32-ops).
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpagedkv.so")
BLOCK_SIZES = (16, 32, 64, 128, 256)
PER_BLOCK_SIZE = ("decode_valu.hip", "decode_mfma.hip")
SOURCES = ["api.cpp", "vmm.cpp", "block_manager.cpp", "cache_ops.hip", *PER_BLOCK_SIZE,
           "reduce.hip", "prefill.hip", "probe.hip", "static_workspace.hip"]
# (source, object stem, defines): one unit of parallel compilation each
UNITS = [(src, f"{os.path.splitext(src)[0]}_s{S}", [f"-DPKV_BLOCK_SIZE={S}"])
         for src in PER_BLOCK_SIZE for S in BLOCK_SIZES] + \
        [(src, os.path.splitext(src)[0], []) for src in SOURCES if src not in PER_BLOCK_SIZE]
ARCH = "gfx950"
# Per-source extra flags. The decode MFMA kernel keeps its accumulators in ordinary VGPRs:
# with the default heuristic the compiler puts them in AGPRs and copies them back and forth for
# the per-chunk rescale, which costs instructions and pushes the 128-wide head past the
# register budget of two waves per SIMD. The prefill kernel does the same, and is built without
# NaN semantics (no arithmetic in it meets a NaN), so its maxima need no quieting instructions.
EXTRA_FLAGS = {"decode_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpagedkv.so)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument"]


def _compile(unit, verbose: bool) -> str:
    src, stem, defines = unit
    obj = os.path.join(BUILD, stem + ".o")
    cmd = [hipcc(), "-x", "hip", *common_flags(), *EXTRA_FLAGS.get(src, []), *defines, "-c",
           os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    noise = "packed-fp32-ops"  # the host pass does not know the device feature: harmless
    warn = "\n".join(ln for ln in r.stderr.splitlines() if noise not in ln).strip()
    if warn and verbose:
        print(warn, file=sys.stderr)
    return obj


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(UNITS), os.cpu_count() or 4, 16)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda u: _compile(u, verbose), UNITS))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args()
    print(build(args.jobs, args.verbose))


if __name__ == "__main__":
    main()
