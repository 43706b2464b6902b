"""Build libfa.so for gfx950 with hipcc (in-tree, no JIT cache).

Every call compiles every source again (the build check must really build).
Objects are compiled in parallel and linked into
``exact_attention_115_amd/libfa.so``. The same sources are also built with
-DFA_STAGE_BARRIERS into ``libfa_stagesync.so``, the debug build whose
kernels wait for every copy and meet at a barrier between the copy and the
compute of each pipeline step; the tests check that it gives bit-identical
results. Nothing but the tests loads it.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")
STAGESYNC_LIB = os.path.join(PKG, "libfa_stagesync.so")

ARCH = "gfx950"
SOURCES = [
    "fa_api.cpp",
    "fa_fwd_f32.hip",
    "fa_fwd.hip",
    "fa_decode.hip",
    "fa_bwd.hip",
    "fa_bwd_dq.hip",
    "fa_dropout.hip",
    "fa_fwd_fp8.hip",
    "fa_noalloc.hip",
]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    f"--offload-arch={ARCH}",
    # Keep the compiler from forming packed-FP32 vector ops.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
    "-Wall",
    "-Wno-unused-function",
    "-I", INCLUDE,
    "-I", CSRC,
]


VARIANTS = {LIB: [], STAGESYNC_LIB: ["-DFA_STAGE_BARRIERS"]}


def _compile(job) -> str:
    src, out_dir, defines = job
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *COMMON, *defines, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(lib: str, objs) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile all sources, link libfa.so and the stage-barrier debug
    library; returns the path of libfa.so."""
    if os.path.isdir(BUILD):
        shutil.rmtree(BUILD)
    jobs = []
    for lib, defines in VARIANTS.items():
        out_dir = os.path.join(BUILD, os.path.splitext(os.path.basename(lib))[0])
        os.makedirs(out_dir)
        jobs += [(src, out_dir, defines) for src in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(_compile, jobs))
    n = len(SOURCES)
    for i, lib in enumerate(VARIANTS):
        _link(lib, objs[i * n:(i + 1) * n])
        if verbose:
            print(f"built {lib}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
