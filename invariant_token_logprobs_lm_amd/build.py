"""Compile the HIP sources into the in-tree shared library libitl.so (gfx950).

    python -m invariant_token_logprobs_lm_amd.build [-v]

Each csrc/*.hip file is compiled separately (in parallel) with hipcc for
gfx950 only, then linked into invariant_token_logprobs_lm_amd/libitl.so.
build_probe() links the benchmark's matrix-core probe (bench_mfma_probe.hip,
beside bench.py) into its own libitl_bench_probe.so there; the library
never uses it. Packed-fp32 instruction selection is disabled for device
code.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libitl.so")
PROBE_LIB = os.path.join(ROOT, "libitl_bench_probe.so")
PROBE_SRC = os.path.join(ROOT, "bench_mfma_probe.hip")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

DEVICE_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # Every rounding is the one the source writes: no a * b + c is fused
    # unless the code asks for fmaf. Kernels that must give the same bits
    # (wide and narrow, any batch) would otherwise depend on which products
    # the compiler chose to fuse in each of them.
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def sources(folder=CSRC):
    return sorted(os.path.join(folder, f) for f in os.listdir(folder) if f.endswith(".hip"))


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(os.path.dirname(src)) + "_" + os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *DEVICE_FLAGS, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err)
    return obj


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
           "-Wl,-rpath,/opt/rocm/lib", "-Wl,--no-undefined"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)


def build(verbose=False):
    """Compile every HIP source and link libitl.so. Always recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    _link(objs, LIB, verbose)
    return LIB


def build_probe(verbose=False):
    """Compile the benchmark's matrix-core probe into libitl_bench_probe.so."""
    os.makedirs(BUILD, exist_ok=True)
    _link([_compile(PROBE_SRC, verbose)], PROBE_LIB, verbose)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_probe(verbose="-v" in sys.argv))
