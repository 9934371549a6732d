"""Shared helpers for GPU parity tests: run the four-call decode chain through
the C ABI binding and compute the float64 oracle references on the same
seeded inputs."""
from __future__ import annotations

import numpy as np
import torch

import mla_inputs as W
import mla_latent_kv_38_amd as mla
from oracle import e4m3 as E
from oracle import mla_oracle as O

TOL = {"f32": 1e-5, "bf16": 1e-2, "e4m3": 3e-2}

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def dims_of(w: W.Workload):
    return mla.make_dims(w.n_h, w.d_h, w.d_c, w.d_R, w.block_size, act=w.act, kv=w.kv,
                         softmax_scale=w.scale, rope_base=w.rope_base)


def to_dev(a, dtype, dev="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dtype)


def tiny_inputs(w: W.Workload):
    """The tiny workload projects h with the oracle; both sides get the float32 rounding."""
    r = w.raw
    c_kv, k_r, q_c, q_r = O.project(r["h"], r["w_dkv"], r["w_kr"], r["w_q"], w.n_h, w.d_h, w.d_R)
    w.c_kv = [W.round_to(c_kv, w.act)]
    w.k_r = [W.round_to(k_r, w.act)]
    w.q_c = W.round_to(q_c, w.act)[None]
    w.q_r = W.round_to(q_r, w.act)[None]
    return w


def new_cache(w: W.Workload, dev="cuda", poison=True):
    """Cache pool; rows never appended hold NaN patterns when ``poison``."""
    shape = (w.num_pages, w.block_size, w.D)
    if w.kv == "e4m3":
        cache = torch.full(shape, 0x7F if poison else 0, dtype=torch.uint8, device=dev)
        scale = torch.full(shape[:2], float("nan") if poison else 1.0, dtype=torch.float32, device=dev)
        return cache, scale
    dt = _DT[w.kv]
    cache = torch.full(shape, float("nan") if poison else 0.0, dtype=dt, device=dev)
    return cache, None


def run_chain(w: W.Workload, num_splits: int = 0, dev="cuda", cache=None, append=True):
    """absorb_q -> cache_append (every token) -> decode -> up_v on the GPU."""
    d = dims_of(w)
    at = _DT[w.act]
    if cache is None:
        cache, scale = new_cache(w, dev)
    else:
        cache, scale = cache
    if append and w.total_tokens() > 0:
        c_all = np.concatenate([w.c_kv[b] for b in range(w.B)])
        k_all = np.concatenate([w.k_r[b] for b in range(w.B)])
        pos = np.concatenate([np.arange(w.lens[b]) for b in range(w.B)]).astype(np.int32)
        slots = np.concatenate([w.slots(b) for b in range(w.B)])
        mla.cache_append(d, to_dev(c_all, at, dev), to_dev(k_all, at, dev), to_dev(pos, torch.int32, dev),
                         to_dev(slots, torch.int64, dev), cache, scale)
    q_abs = mla.absorb_q(d, to_dev(w.q_c, at, dev), to_dev(w.q_r, at, dev),
                         to_dev(w.q_pos, torch.int32, dev), to_dev(w.w_uk, at, dev))
    o_lat, lse = mla.decode(d, q_abs, cache, to_dev(w.block_table, torch.int32, dev),
                            to_dev(w.lens, torch.int32, dev), kv_scale=scale, num_splits=num_splits)
    out = mla.up_v(d, o_lat, to_dev(w.w_uv, at, dev))
    torch.cuda.synchronize()
    return dict(q_abs=q_abs, cache=cache, scale=scale, o_lat=o_lat, lse=lse, out=out)


def f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def oracle_rows(w: W.Workload, b: int):
    """Expected cache rows of sequence b: float64 rows, rounded as stored, and
    (E4M3) the oracle's own codes and scales."""
    rows = O.cache_rows(w.c_kv[b], w.k_r[b], np.arange(w.lens[b]), w.rope_base)
    if w.kv == "f32":
        return dict(stored=O.to_f32(rows).astype(np.float64))
    if w.kv == "bf16":
        return dict(stored=O.to_bf16(rows).astype(np.float64))
    codes, s = E.quantize_rows(O.to_f32(rows))
    return dict(codes=codes, scales=s, stored=E.dequantize_rows(codes, s))


def oracle_decode(w: W.Workload, b: int, heads=None):
    """Explicit-form oracle for sequence b (E4M3: on the oracle's dequantised rows)."""
    kw = dict(scale=w.scale, base=w.rope_base, heads=heads)
    if w.kv == "e4m3":
        rows = oracle_rows(w, b)["stored"]
        return O.explicit_decode(w.q_c[b], w.q_r[b], rows[:, :w.d_c], rows[:, w.d_c:], w.w_uk, w.w_uv,
                                 k_r_rotated=True, **kw)
    return O.explicit_decode(w.q_c[b], w.q_r[b], w.c_kv[b], w.k_r[b], w.w_uk, w.w_uv, **kw)


def gather_rows(w: W.Workload, res, b: int):
    """GPU cache rows of sequence b read back through its page table (float64)."""
    L = int(w.lens[b])
    j = np.arange(L)
    pages = torch.from_numpy(w.block_table[b, j // w.block_size].astype(np.int64))
    offs = torch.from_numpy((j % w.block_size).astype(np.int64))
    cache = res["cache"].cpu()
    if w.kv == "e4m3":
        codes = cache[pages, offs].numpy()
        s = res["scale"].cpu()[pages, offs].numpy()
        return dict(codes=codes, scales=s, stored=E.dequantize_rows(codes, s))
    return dict(stored=cache[pages, offs].to(torch.float64).numpy())


def rel_err(got, ref):
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(np.asarray(got, np.float64) - ref).max() / (den if den > 0 else 1.0))


def lse_err(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin) and np.all(got[~fin] == ref[~fin])
    if not fin.any():
        return 0.0
    return float((np.abs(got[fin] - ref[fin]) / np.maximum(1.0, np.abs(ref[fin]))).max())
