"""Builds ``libhisparse.so`` (C ABI + HIP kernels for gfx950) in place.

Usage: ``python -m sparse_attention_kv_request_amd.build`` (or ``build()``).
Each source compiles to an object under ``_build/`` in parallel, then one
link produces the shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import pathlib
import shutil
import subprocess

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIB = PKG / "libhisparse.so"
BUILD = ROOT / "_build"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}",
]


def sources():
    return sorted(list(CSRC.glob("*.hip")) + list(CSRC.glob("*.cpp")))


def _compile(src: pathlib.Path, objdir: pathlib.Path, defines) -> pathlib.Path:
    obj = objdir / (src.name + ".o")
    cmd = [HIPCC, *FLAGS, *defines, "-c", str(src), "-o", str(obj)]
    if src.suffix == ".cpp":
        cmd[1:1] = ["-x", "hip"]
    subprocess.run(cmd, check=True)
    return obj


def build(verbose: bool = False, defines=(), lib: pathlib.Path = LIB) -> pathlib.Path:
    """The library at `lib`; `defines` (``-DNAME=VALUE``) build a variant,
    e.g. the phase-clock instrumentation, into its own object folder."""
    objdir = BUILD if not defines else BUILD / ("variant_" + lib.parent.name)
    objdir.mkdir(parents=True, exist_ok=True)
    lib.parent.mkdir(parents=True, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, objdir, list(defines)), srcs))
    tmp = lib.with_suffix(".so.tmp")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC",
                    *[str(o) for o in objs], "-o", str(tmp)], check=True)
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True)
