"""Builds the gfx950 shared library ``libqknorm_rope_attn.so`` in-tree with hipcc.

Every source is compiled for gfx950 only.  Packed-fp32 VALU instructions are
disabled for the device code (``-target-feature -packed-fp32-ops``); hipcc's
host pass warns that it does not know that feature, which is harmless.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT_DIR, "include")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_NAME = "libqknorm_rope_attn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["qknorm_rope.hip", "prefill_mfma.hip", "prefill_fp32.hip", "decode.hip", "decode_mfma.hip", "layer_ops.hip", "api.hip"]
# The benchmark's roofline calibration kernels: a library of their own, outside the attention ABI.
CALIB_SOURCES = ["calibrate.hip"]
CALIB_LIB_PATH = os.path.join(PKG_DIR, "libqkra_calibrate.so")
# The profiling build: the same sources with per-workgroup phase stamps in the
# bf16 prefill attention kernels (include/qkra_phase_stamps.h).
STAMPS_LIB_PATH = os.path.join(PKG_DIR, "libqknorm_rope_attn_stamps.so")
STAMPS_BUILD_DIR = os.path.join(PKG_DIR, "_build_stamps")
ARCH = "gfx950"
CFLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the gfx950 library)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in proc.stdout.splitlines() if "packed-fp32-ops" not in line)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build_library(verbose: bool = False, jobs: int | None = None, extra_flags=None, out_path: str | None = None,
                  build_dir: str | None = None, sources=None) -> str:
    """Compile every HIP source for gfx950 and link the shared library; returns its path."""
    hipcc = _hipcc()
    build_dir = build_dir or BUILD_DIR
    out_path = out_path or LIB_PATH
    os.makedirs(build_dir, exist_ok=True)
    flags = CFLAGS + list(extra_flags or [])
    objs = []
    cmds = []
    for src in sources or SOURCES:
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([hipcc] + flags + ["-c", os.path.join(CSRC, src), "-o", obj])
    workers = jobs or min(len(cmds), max(1, (os.cpu_count() or 4) // 2), 8)
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as pool:
        for fut in [pool.submit(_run, c, verbose) for c in cmds]:
            fut.result()
    tmp = out_path + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, out_path)
    return out_path


def build_calibration(verbose: bool = False) -> str:
    """The roofline calibration library (libqkra_calibrate.so); returns its path."""
    return build_library(verbose, out_path=CALIB_LIB_PATH, sources=CALIB_SOURCES)


def build_phase_stamps(verbose: bool = False) -> str:
    """The profiling build with phase stamps (libqknorm_rope_attn_stamps.so); returns its path."""
    return build_library(verbose, extra_flags=["-DQKRA_PHASE_STAMPS"], out_path=STAMPS_LIB_PATH,
                         build_dir=STAMPS_BUILD_DIR)


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
    print(build_calibration(verbose="-v" in sys.argv))
    print(build_phase_stamps(verbose="-v" in sys.argv))
