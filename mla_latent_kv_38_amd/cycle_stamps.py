"""Cycle stamps of the bf16 decode kernel (a measurement tool, not part of
the decode path).

Builds the library once more with -DMLA_CYCLE_STAMPS into a directory of
its own (never the package's library): the decode kernel then accumulates
s_memtime stamps around its phases and wave 0 of every workgroup writes them
to a device array.  Runs mla_decode on a synthetic batch (random bf16 cache
and queries, sequential pages, every sequence the same length) and prints
one JSON line: per-workgroup means of each phase in shader cycles, the
workgroups' durations by s_memrealtime (100 MHz) and the shader clock that
the two imply.

    python -m mla_latent_kv_38_amd.cycle_stamps --build-dir /tmp/mla_stamps \\
        [--batch 16] [--len 4096] [--heads 128]
"""
from __future__ import annotations

import argparse
import concurrent.futures
import ctypes
import json
import os

import numpy as np

from . import build as _build

FIELDS = ["total", "locate_end", "query_issue", "loop_start", "wait", "barrier", "qk", "softmax", "pv", "pages",
          "epilogue", "rt_start", "rt_end", "written"]


def build_stamped(out_dir: str, jobs: int = 8) -> str:
    os.makedirs(out_dir, exist_ok=True)
    common = [*_build.COMMON, "-DMLA_CYCLE_STAMPS"]

    def one(src):
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        _build._run([_build.HIPCC, *common, "-c", os.path.join(_build.CSRC, src), "-o", obj])
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(one, _build.SOURCES))
    lib = os.path.join(out_dir, "libmla_stamps_gfx950.so")
    _build._run([_build.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", lib])
    return lib


def measure(lib_path: str, B: int, L: int, n_h: int, reps: int = 5) -> dict:
    import torch

    from . import _lib
    from . import ops as mla
    lib = _lib.lib(lib_path)
    _lib._LIB = lib                                  # the ops bind to the stamped library
    lib.mla_stamps_read.restype, lib.mla_stamps_read.argtypes = ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t]
    nf = int(lib.mla_stamps_fields())
    d = mla.make_dims(n_h, 128, 512, 64, 64, act="bf16", kv="bf16")
    pages_per = (L + 63) // 64
    g = torch.Generator(device="cuda").manual_seed(0)
    cache = torch.randn((B * pages_per, 64, 576), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((B, n_h, 576), generator=g, device="cuda").to(torch.bfloat16)
    bt = torch.arange(B * pages_per, dtype=torch.int32, device="cuda").view(B, pages_per)
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    for _ in range(reps):
        mla.decode(d, q, cache, bt, lens)
    torch.cuda.synchronize()
    buf = (ctypes.c_ulonglong * (4096 * nf))()
    if lib.mla_stamps_read(buf, ctypes.sizeof(buf)) != 0:
        raise RuntimeError("reading the stamps failed")
    a = np.frombuffer(buf, dtype=np.uint64).reshape(4096, nf).astype(np.float64)
    a = a[a[:, FIELDS.index("written")] > 0]
    col = {f: a[:, i] for i, f in enumerate(FIELDS)}
    pages = np.maximum(col["pages"], 1)
    dur_us = (col["rt_end"] - col["rt_start"]) / 100.0
    start_us = (col["rt_start"] - col["rt_start"].min()) / 100.0
    pct = lambda x: [round(float(np.percentile(x, p)), 2) for p in (0, 50, 100)]
    return {
        "workload": {"batch": B, "len": L, "n_heads": n_h, "workgroups": int(len(a)),
                     "pages_per_workgroup": pct(col["pages"])},
        "cycles_per_workgroup": {
            "total": round(float(col["total"].mean()), 1),
            "set_up_locate": round(float(col["locate_end"].mean()), 1),
            "set_up_to_query_loads": round(float((col["query_issue"] - col["locate_end"]).mean()), 1),
            "set_up_to_first_page": round(float((col["loop_start"] - col["query_issue"]).mean()), 1),
            "pages": round(float((col["wait"] + col["barrier"] + col["qk"] + col["softmax"] + col["pv"]).mean()), 1),
            "segment_end": round(float(col["epilogue"].mean()), 1)},
        "cycles_per_page": {f: round(float((col[f] / pages).mean()), 1) for f in ("wait", "barrier", "qk", "softmax", "pv")},
        "realtime_us": {"workgroup_duration": pct(dur_us), "start_offset": pct(start_us)},
        "shader_clock_ghz": round(float((col["total"] / (dur_us * 1e3)).mean()), 3),
    }


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--build-dir", required=True)
    p.add_argument("--batch", type=int, default=16)
    p.add_argument("--len", type=int, default=4096)
    p.add_argument("--heads", type=int, default=128)
    p.add_argument("--no-build", action="store_true")
    a = p.parse_args()
    lib = os.path.join(a.build_dir, "libmla_stamps_gfx950.so") if a.no_build else build_stamped(a.build_dir)
    print(json.dumps(measure(lib, a.batch, a.len, a.heads)))


if __name__ == "__main__":
    main()
