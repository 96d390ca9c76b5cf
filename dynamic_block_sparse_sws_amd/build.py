"""Build the HIP library libsws.so in-tree with hipcc for gfx950.

    python -m dynamic_block_sparse_sws_amd.build          # or build() from Python
    python -m dynamic_block_sparse_sws_amd.build --asan   # + libsws_asan.so

build() also builds ceiling_probe, a standalone program (csrc/ceiling_probe.hip,
not part of the library) that measures the MFMA, exp2 and LDS ceilings the
attention kernels' roofline fractions are read against.

The --asan variant compiles the host side of the C ABI layer (sws_api.hip:
argument validation, error reporting, the scratch address lookup) with
AddressSanitizer; the GPU code is built as usual.  Load it with the ASan
runtime preloaded (asan_runtime() gives its path) and SWS_LIBRARY pointing
at it; tests/test_asan_host.py runs the host-validation tests that way.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsws.so")
LIB_ASAN = os.path.join(PKG, "libsws_asan.so")
PROBE = os.path.join(PKG, "ceiling_probe")
SOURCES = ["sws_api.hip", "sketch.hip", "walk.hip", "walk_variant.hip", "select.hip",
           "attn_prefill.hip", "attn_prefill_f32.hip", "attn_decode.hip"]
ARCH = os.environ.get("SWS_OFFLOAD_ARCH", "gfx950")

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the Sketch&Walk HIP library cannot be built")


# AddressSanitizer on the host compilation only (the GPU code is unchanged)
ASAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, extra=(), suffix: str = "") -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + suffix + ".o")
    cmd = [hipcc()] + COMMON_FLAGS + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


# roctx ranges around the C ABI calls (rocprofiler-sdk's marker library)
LINK_LIBS = ["-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx", "-Wl,-rpath,/opt/rocm/lib"]


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs + LINK_LIBS
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (to preload)."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the AddressSanitizer runtime of the HIP compiler was not found")
    return path


def build_asan(verbose: bool = False) -> str:
    """libsws_asan.so: sws_api.hip's host code with AddressSanitizer, every
    other source as in build() (reusing its objects when present)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    for src in SOURCES:
        if src == "sws_api.hip":
            objs.append(_compile(src, ASAN_HOST_FLAGS, "_asan"))
        else:
            obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
            fresh = (os.path.exists(obj) and
                     os.path.getmtime(obj) >= os.path.getmtime(os.path.join(CSRC, src)) and
                     os.path.getmtime(obj) >= os.path.getmtime(os.path.join(CSRC, "sws_common.h")))
            objs.append(obj if fresh else _compile(src))
    _link(objs, LIB_ASAN)
    if verbose:
        print(f"built {LIB_ASAN}")
    return LIB_ASAN


def build_probe(verbose: bool = False) -> str:
    """The ceiling-probe program, next to this file."""
    tmp = PROBE + ".tmp"
    cmd = [hipcc()] + [f for f in COMMON_FLAGS if f != "-fPIC"] + [
        os.path.join(CSRC, "ceiling_probe.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on ceiling_probe.hip:\n{r.stderr}")
    os.replace(tmp, PROBE)
    if verbose:
        print(f"built {PROBE}")
    return PROBE


def build(verbose: bool = False, jobs: int = 6) -> str:
    """Compile every source and link libsws.so next to this file; build the
    ceiling-probe program."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES) + 1))) as ex:
        probe = ex.submit(build_probe)
        objs = list(ex.map(_compile, SOURCES))
        probe.result()
    _link(objs, LIB)
    if verbose:
        print(f"built {LIB}")
        print(f"built {PROBE}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    if "--asan" in sys.argv[1:]:
        build_asan(verbose=True)
    sys.exit(0)
