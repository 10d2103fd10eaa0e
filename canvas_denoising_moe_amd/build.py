"""Build the gfx950 HIP library ``_lib/libdg.so`` in-tree with hipcc.

Run ``python -m canvas_denoising_moe_amd.build`` (or call :func:`build`).
Each ``csrc/*.hip`` file is compiled to an object under ``_build/`` and the
objects are linked into one shared library exporting the C ABI of
``include/dg.h``.
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
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIB_DIR, "libdg.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 VALU forms in generated device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: with the default AGPR form the LM
    # head's 128 accumulators were shuffled between register files on every
    # loop iteration
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # loops marked for full unrolling stay unrolled even when large (the LM
    # head's sampler epilogue indexes its accumulators with the loop counters)
    "-mllvm", "-pragma-unroll-threshold=65536",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# Debug build of the host side under AddressSanitizer (device code unchanged):
# the runtime's argument checks and error paths run instrumented in a host
# process, on any machine with hipcc and no GPU.  The library lands outside the
# package, under _build/asan/, and is loaded only by the test that asks for it.
ASAN_HOST_FLAGS = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-g",
]
ASAN_LIB = os.path.join(BUILD_DIR, "asan", "libdg.so")


def _compile(src: str, verbose: bool, asan: bool = False) -> str:
    out_dir = os.path.join(BUILD_DIR, "asan") if asan else BUILD_DIR
    obj = os.path.join(out_dir, os.path.basename(src)[:-4] + ".o")
    flags = HIPCC_FLAGS + (ASAN_HOST_FLAGS if asan else [])
    cmd = [hipcc(), *flags, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False, asan: bool = False) -> str:
    """Compile every HIP source for gfx950 and link ``libdg.so``; returns its path.

    ``asan``: the AddressSanitizer debug build of the host side instead
    (``ASAN_LIB``); the product library is left alone."""
    out = ASAN_LIB if asan else LIB
    os.makedirs(os.path.dirname(out), exist_ok=True)
    os.makedirs(os.path.join(BUILD_DIR, "asan") if asan else BUILD_DIR, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, asan), srcs))
    tmp = out + ".tmp"
    link_flags = ["-Xarch_host", "-fsanitize=address"] if asan else []
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *link_flags, "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
