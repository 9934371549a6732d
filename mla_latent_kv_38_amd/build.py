"""Compile the HIP/C++ sources into the in-tree shared library (gfx950)."""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_NAME = "libmla_gfx950.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["mla_api.hip", "k_generic.hip", "k_decode_e4m3_h64.hip", "k_decode_fp8.hip", "k_proj_mfma.hip",
           "k_kvproj.hip",
           "k_decode_h64w.hip", "probes.hip"]

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
# Packed-fp32 VALU forms are disabled for every device pass.
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def build(jobs: int = 8) -> str:
    """Compile every source and link the library; returns its path."""
    obj_dir = os.path.join(ROOT, "_build")
    os.makedirs(obj_dir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        _run([HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
