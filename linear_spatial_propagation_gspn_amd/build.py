"""Build libgspn.so in-tree with hipcc for gfx950.

    python -m linear_spatial_propagation_gspn_amd.build

Every HIP source is compiled to an object under ``_build/`` (git-ignored) and
linked into ``libgspn.so`` next to this file.  Flags: gfx950 only, -O3, no
packed-fp32 instruction forms (plain fp32 VALU code only).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgspn.so")
SOURCES = ["api.cpp", "scan.hip", "scan_f32_vert.hip", "scan_f32_horiz.hip", "scan_bf16_vert.hip",
           "scan_bf16_horiz.hip", "scan_bf16pair_vert.hip", "scan_bf16pair_horiz.hip", "scan4_f32.hip",
           "scan4_bf16.hip", "scan4_bf16pair.hip", "scan4_f32x.hip", "elementwise.hip", "transpose.hip", "project.hip",
           "plane4.hip", "backward.hip", "adjplane.hip", "noalloc.hip",
           "seq4.hip", "wgrad.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++20", "-fPIC", "-Wall", "-Wno-unused-function",
    "-I" + INCLUDE, "-I" + CSRC,
]
DEVICE = [
    "--offload-arch=" + ARCH,
    # no hand-picked or compiler-formed packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str, build_dir: str = BUILD, defines: tuple = ()) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(build_dir, src + ".o")
    cmd = [HIPCC] + COMMON + DEVICE + ["-D" + d for d in defines] + ["-x", "hip", "-c", path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), res.stderr))
    return obj


def build(verbose: bool = False, out: str = LIB, defines: tuple = ()) -> str:
    """Compile every source and link libgspn.so (always rebuilds).  ``out`` and
    ``defines`` (preprocessor NAME=VALUE pairs, e.g. launch-configuration
    overrides) allow variant builds elsewhere."""
    build_dir = BUILD if out == LIB else os.path.join(os.path.dirname(os.path.abspath(out)), "_build")
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, tuple(defines)), SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


CHECK_LIB = os.path.join(PKG, "libgspn_check.so")
CHECK_BUILD = os.path.join(BUILD, "check")


def build_check(verbose: bool = False, out: str = CHECK_LIB) -> str:
    """Compile the host-only checking library libgspn_check.so (always
    rebuilds): every source's host code with GSPN_CHECK_LAUNCHES, so that the
    C ABI runs as usual while each launch replays its kernel's accesses on the
    host instead of queueing it (csrc/check.hpp), plus the checker's registry
    (csrc/check.cpp).  No device code is compiled."""
    os.makedirs(CHECK_BUILD, exist_ok=True)

    def one(src: str) -> str:
        obj = os.path.join(CHECK_BUILD, src + ".o")
        cmd = [HIPCC] + COMMON + ["-DGSPN_CHECK_LAUNCHES", "-x", "hip", "--offload-host-only", "-c",
                                  os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc (host only) failed for %s:\n%s\n%s" % (src, " ".join(cmd), res.stderr))
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES) + 1, os.cpu_count() or 4)) as ex:
        objs = list(ex.map(one, SOURCES + ["check.cpp"]))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    build_check(verbose=True)
    sys.exit(0)
