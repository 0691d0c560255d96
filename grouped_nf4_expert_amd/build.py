"""Build libgnf4.so (hand-written HIP for gfx950) in the package directory.

    python -m grouped_nf4_expert_amd.build

Each translation unit is compiled with hipcc for gfx950 only, in parallel,
then linked into one shared library next to this file.  Packed fp32 VALU
instructions are disabled for every device compile.  The machine-ceiling
probes (ceilings.hip, include/gnf4_ceilings.h) are linked into a library of
their own, libgnf4_ceilings.so, which the GEMM library does not use.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgnf4.so")
SOURCES = ["api.hip", "pack.hip", "route.hip", "gather.hip", "decode.hip", "tile.hip",
           "glue.hip", "dgrad.hip", "validate.hip"]
CEIL_SOURCES = ["ceilings.hip"]
CEIL_LIB = os.path.join(PKG, "libgnf4_ceilings.so")
ARCH = "gfx950"


def hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libgnf4")


def common_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I", INCLUDE, "-I", CSRC,
    ]


# Per-source flags.  decode.hip: its kernels take their first scalar
# arguments preloaded into SGPRs at wavefront launch (gfx950 kernel-argument
# preloading), so the first dependent loads need no argument-segment read.
EXTRA_FLAGS = {"decode.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=7"]}


def _compile(src, extra=()):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *common_flags(), *EXTRA_FLAGS.get(src, []), *extra, "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib, extra=()):
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose=False, extra_compile=(), extra_link=(), timeline=True):
    """Compile every source and link the libraries (with `timeline`, also the
    phase-stamped diagnostic build, timeline_build.py).  extra_compile /
    extra_link: further hipcc flags (build_sanitized.py passes host-only
    sanitizer flags)."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CEIL_SOURCES
    with ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, extra_compile), srcs)))
    _link([objs[s] for s in SOURCES], LIB, extra_link)
    _link([objs[s] for s in CEIL_SOURCES], CEIL_LIB, extra_link)
    if verbose:
        print(f"built {LIB} and {CEIL_LIB}")
    if timeline:
        from grouped_nf4_expert_amd import timeline_build
        timeline_build.build(verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
