"""Compile libmla.so (all HIP sources of the package) for gfx950, in-tree.

Usage: ``python mla_latent_kv_06_amd/build.py`` (a plain script, so the package
itself, which needs the library, is not imported) or ``build_library()``.
The library is placed next to this file so that the binding finds it and
so that it travels with the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla.so")
ARCH = "gfx950"

SOURCES = ["mla_api.hip", "decode.hip", "combine.hip", "combine_up.hip", "gemm.hip", "gather.hip", "append.hip", "decompress.hip", "prefill_mha.hip", "step.hip", "static_step.hip", "ceilings.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmla)")


FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # inline asm that touches a reserved register (M0, EXEC, ...) without
    # telling the compiler fails the build
    "-Werror=inline-asm",
]


def compile_command(src: str, obj: str) -> list[str]:
    return [hipcc()] + FLAGS + ["-c", src, "-o", obj]


def link_command(objs: list[str], out: str = LIB) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out] + objs


def build_library(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source to an object (in parallel) and link libmla.so."""
    from concurrent.futures import ThreadPoolExecutor

    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, min(16, int(os.environ.get("MAX_JOBS", os.cpu_count() or 1)))))

    def one(src):
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        cmd = compile_command(os.path.join(CSRC, src), obj)
        if verbose:
            print(" ".join(cmd), flush=True)
        return obj, subprocess.run(cmd, capture_output=True, text=True)

    with ThreadPoolExecutor(jobs) as pool:
        results = list(pool.map(one, SOURCES))
    failed = [(o, r) for o, r in results if r.returncode != 0]
    for _, r in failed:
        sys.stderr.write(r.stdout + r.stderr)
    if failed:
        raise RuntimeError(f"hipcc failed on {', '.join(os.path.basename(o) for o, _ in failed)}")
    tmp = LIB + ".tmp"
    cmd = link_command([o for o, _ in results], tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc link failed with exit code {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
