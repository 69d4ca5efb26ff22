"""Compiles libtis.so (the HIP kernels and their C-ABI) for gfx950, in place.

    python -m tree_indexed_sparse_build_amd._build

Uses hipcc directly: one shared library, no torch extension machinery.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtis.so")
SOURCES = ["tis_api.hip", "build.hip", "route.hip", "attend.hip", "attend_group.hip", "decode.hip",
           "cache.hip", "sphere.hip", "prefill.hip", "probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libtis)")


FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions stay off (their use is left to no one)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs: the prefill's output tile
    # is rescaled by vector code between products, which in AGPRs would cost
    # a copy out and back every step
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def command(out: str = LIB) -> list:
    """The whole build as one hipcc command (what build_library runs, split
    into one compile per source plus a link so the sources build in parallel)."""
    return [hipcc()] + FLAGS + ["-shared", "-o", out] + [os.path.join(CSRC, s) for s in SOURCES]


def _run(cmd: list) -> subprocess.CompletedProcess:
    return subprocess.run(cmd, capture_output=True, text=True)


def build_library(verbose: bool = False) -> str:
    """Compiles every source to an object (in parallel), links libtis.so."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="libtis_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [[cc] + FLAGS + ["-c", "-o", o, os.path.join(CSRC, s)]
                for s, o in zip(SOURCES, objs)]
        tmp = LIB + ".tmp"
        cmds_link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
        workers = max(1, min(len(cmds), os.cpu_count() or 1, 8))
        with ThreadPoolExecutor(workers) as ex:
            results = list(ex.map(_run, cmds))
        results.append(_run(cmds_link) if all(r.returncode == 0 for r in results) else None)
        for cmd, r in zip(cmds + [cmds_link], results):
            if r is None:
                continue
            if verbose:
                print(" ".join(cmd), flush=True)
            if r.returncode != 0:
                sys.stderr.write(r.stdout + r.stderr)
                raise RuntimeError(f"hipcc failed with status {r.returncode}")
            if verbose and r.stderr.strip():
                sys.stderr.write(r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
