"""Torch-facing binding: the four calls of include/mla.h with the same names.

Argument marshalling only (dtype/shape/device checks, data pointers, the
current HIP stream).  Every step of the computation runs in the HIP library;
there is no CPU or PyTorch fallback.

The library does not read device-resident indices on the host (slots, page
ids, lengths): out-of-range values there are undefined behaviour on the GPU.
Setting MLA_VALIDATE=1 in the environment makes the calls below copy those
small index tensors to the host first and raise ValueError on any violation
(`check_slots`, `check_paging`); this synchronises the stream and is meant
for debugging.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

from . import _lib
from ._lib import MLA_BF16, MLA_E4M3, MLA_F32, Dims, check

_TORCH = {MLA_F32: torch.float32, MLA_BF16: torch.bfloat16}


def make_dims(n_heads: int, d_head: int, d_latent: int, d_rope: int, block_size: int = 64,
              act: str = "bf16", kv: str = "bf16", softmax_scale: float | None = None,
              rope_base: float = 10000.0) -> Dims:
    codes = {"f32": MLA_F32, "bf16": MLA_BF16, "e4m3": MLA_E4M3}
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d_head + d_rope)
    return Dims(n_heads, d_head, d_latent, d_rope, block_size, codes[act], codes[kv],
                softmax_scale, rope_base)


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _validating() -> bool:
    return os.environ.get("MLA_VALIDATE", "") not in ("", "0")


def check_slots(slot, num_pages: int, block_size: int):
    """Host check of an append's slots: 0 <= slot < num_pages * block_size and
    no slot twice (two rows written to one place in one call)."""
    s = slot.detach().cpu().to(torch.int64)
    cap = int(num_pages) * int(block_size)
    bad = ((s < 0) | (s >= cap)).nonzero().flatten()
    if bad.numel():
        i = int(bad[0])
        raise ValueError(f"slot[{i}] = {int(s[i])} outside [0, {cap})")
    if torch.unique(s).numel() != s.numel():
        raise ValueError("slots repeat within one call")


def check_paging(block_table, seq_lens, num_pages: int, block_size: int, seq_starts=None):
    """Host check of a decode's paging: 0 <= seq_starts[b] and
    0 <= seq_lens[b] <= max_pages * block_size, and every block-table entry the
    decode reads (pages seq_starts[b] // block_size .. ceil(L / block_size) - 1)
    names a page in [0, num_pages)."""
    bt = block_table.detach().cpu().to(torch.int64)
    lens = seq_lens.detach().cpu().to(torch.int64)
    starts = torch.zeros_like(lens) if seq_starts is None else seq_starts.detach().cpu().to(torch.int64)
    max_pages = bt.shape[1]
    for b in range(lens.numel()):
        L, st = int(lens[b]), int(starts[b])
        if L < 0 or L > max_pages * block_size:
            raise ValueError(f"seq_lens[{b}] = {L} outside [0, {max_pages * block_size}]")
        if st < 0:
            raise ValueError(f"seq_starts[{b}] = {st} < 0")
        if st >= L:
            continue
        used = bt[b, st // block_size:(L + block_size - 1) // block_size]
        bad = ((used < 0) | (used >= num_pages)).nonzero().flatten()
        if bad.numel():
            k = st // block_size + int(bad[0])
            raise ValueError(f"block_table[{b}, {k}] = {int(bt[b, k])} outside [0, {num_pages})")


def _kv_torch(d: Dims):
    return (torch.uint8, torch.float8_e4m3fn) if d.kv_dtype == MLA_E4M3 else _TORCH[d.kv_dtype]


def absorb_q(d: Dims, q_c, q_r, q_pos, w_uk, q_abs=None, stream=None):
    """q_abs = [W_UK^T q_C || RoPE(q_R, q_pos)] per batch row and head."""
    at = _TORCH[d.act_dtype]
    B = q_c.shape[0]
    D = d.d_latent + d.d_rope
    _need(q_c, "q_c", at, (B, d.n_heads, d.d_head))
    if d.d_rope:
        _need(q_r, "q_r", at, (B, d.n_heads, d.d_rope))
    _need(q_pos, "q_pos", torch.int32, (B,))
    _need(w_uk, "w_uk", at, (d.n_heads, d.d_head, d.d_latent))
    if q_abs is None:
        q_abs = torch.empty((B, d.n_heads, D), dtype=at, device=q_c.device)
    _need(q_abs, "q_abs", at, (B, d.n_heads, D))
    check(_lib.lib().mla_absorb_q(ctypes.byref(d), B, _ptr(q_c), _ptr(q_r), _ptr(q_pos), _ptr(w_uk),
                                  _ptr(q_abs), _stream(stream)), "mla_absorb_q")
    return q_abs


def cache_append(d: Dims, c_kv, k_r, pos, slot, kv_cache, kv_scale=None, stream=None):
    """Write [c_kv || RoPE(k_r, pos)] rows into kv_cache at the given slots."""
    at = _TORCH[d.act_dtype]
    T = c_kv.shape[0]
    D = d.d_latent + d.d_rope
    _need(c_kv, "c_kv", at, (T, d.d_latent))
    if d.d_rope:
        _need(k_r, "k_r", at, (T, d.d_rope))
    _need(pos, "pos", torch.int32, (T,))
    _need(slot, "slot", torch.int64, (T,))
    _need(kv_cache, "kv_cache", _kv_torch(d))
    if kv_cache.dim() != 3 or kv_cache.shape[1] != d.block_size or kv_cache.shape[2] != D:
        raise ValueError(f"kv_cache shape {tuple(kv_cache.shape)}")
    if d.kv_dtype == MLA_E4M3:
        _need(kv_scale, "kv_scale", torch.float32, kv_cache.shape[:2])
    if _validating():
        check_slots(slot, kv_cache.shape[0], d.block_size)
    check(_lib.lib().mla_cache_append(ctypes.byref(d), T, _ptr(c_kv), _ptr(k_r), _ptr(pos), _ptr(slot),
                                      kv_cache.shape[0], _ptr(kv_cache), _ptr(kv_scale), _stream(stream)),
          "mla_cache_append")


def absorb_q_append(d: Dims, q_c, q_r, q_pos, w_uk, c_kv, k_r, pos, slot, kv_cache, kv_scale=None, q_abs=None,
                    stream=None):
    """absorb_q and cache_append in one call (one launch where the shapes
    allow); returns q_abs."""
    at = _TORCH[d.act_dtype]
    B = q_c.shape[0]
    D = d.d_latent + d.d_rope
    _need(q_c, "q_c", at, (B, d.n_heads, d.d_head))
    if d.d_rope:
        _need(q_r, "q_r", at, (B, d.n_heads, d.d_rope))
    _need(q_pos, "q_pos", torch.int32, (B,))
    _need(w_uk, "w_uk", at, (d.n_heads, d.d_head, d.d_latent))
    if q_abs is None:
        q_abs = torch.empty((B, d.n_heads, D), dtype=at, device=q_c.device)
    _need(q_abs, "q_abs", at, (B, d.n_heads, D))
    T = c_kv.shape[0]
    _need(c_kv, "c_kv", at, (T, d.d_latent))
    if d.d_rope:
        _need(k_r, "k_r", at, (T, d.d_rope))
    _need(pos, "pos", torch.int32, (T,))
    _need(slot, "slot", torch.int64, (T,))
    _need(kv_cache, "kv_cache", _kv_torch(d))
    if kv_cache.dim() != 3 or kv_cache.shape[1] != d.block_size or kv_cache.shape[2] != D:
        raise ValueError(f"kv_cache shape {tuple(kv_cache.shape)}")
    if d.kv_dtype == MLA_E4M3:
        _need(kv_scale, "kv_scale", torch.float32, kv_cache.shape[:2])
    if _validating():
        check_slots(slot, kv_cache.shape[0], d.block_size)
    check(_lib.lib().mla_absorb_q_append(ctypes.byref(d), B, _ptr(q_c), _ptr(q_r), _ptr(q_pos), _ptr(w_uk),
                                         _ptr(q_abs), T, _ptr(c_kv), _ptr(k_r), _ptr(pos), _ptr(slot),
                                         kv_cache.shape[0], _ptr(kv_cache), _ptr(kv_scale), _stream(stream)),
          "mla_absorb_q_append")
    return q_abs


def kv_project_workspace_bytes(d: Dims, n_tokens: int, d_model: int) -> int:
    return int(_lib.lib().mla_kv_project_workspace_bytes(ctypes.byref(d), n_tokens, d_model))


def kv_project_append(d: Dims, h, w_dkv, w_kr, pos, slot, kv_cache, kv_scale=None, workspace=None,
                      stream=None):
    """c_kv = W_DKV h, k_R = W_KR h (rounded to the activation type), appended
    as [c_kv || RoPE(k_R, pos)] rows at the given slots."""
    at = _TORCH[d.act_dtype]
    T, dm = h.shape
    _need(h, "h", at, (T, dm))
    _need(w_dkv, "w_dkv", at, (d.d_latent, dm))
    if d.d_rope:
        _need(w_kr, "w_kr", at, (d.d_rope, dm))
    _need(pos, "pos", torch.int32, (T,))
    _need(slot, "slot", torch.int64, (T,))
    _need(kv_cache, "kv_cache", _kv_torch(d))
    if kv_cache.dim() != 3 or kv_cache.shape[1] != d.block_size or kv_cache.shape[2] != d.d_latent + d.d_rope:
        raise ValueError(f"kv_cache shape {tuple(kv_cache.shape)}")
    if d.kv_dtype == MLA_E4M3:
        _need(kv_scale, "kv_scale", torch.float32, kv_cache.shape[:2])
    if _validating():
        check_slots(slot, kv_cache.shape[0], d.block_size)
    need = kv_project_workspace_bytes(d, T, dm)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=h.device)
    check(_lib.lib().mla_kv_project_append(ctypes.byref(d), T, dm, _ptr(h), _ptr(w_dkv), _ptr(w_kr), _ptr(pos),
                                           _ptr(slot), kv_cache.shape[0], _ptr(kv_cache), _ptr(kv_scale),
                                           _ptr(workspace), workspace.numel() * workspace.element_size(),
                                           _stream(stream)), "mla_kv_project_append")


def decode_workspace_bytes(d: Dims, batch: int, num_splits: int = 0) -> int:
    return int(_lib.lib().mla_decode_workspace_bytes(ctypes.byref(d), batch, num_splits))


def decode(d: Dims, q_abs, kv_cache, block_table, seq_lens, kv_scale=None, num_splits: int = 0,
           workspace=None, o_lat=None, lse=None, stream=None, seq_starts=None):
    """Absorbed attention over the paged latent cache; returns (o_lat, lse).
    With seq_starts, sequence b attends only to its rows [seq_starts[b], L_b)
    (mla_decode_window)."""
    at = _TORCH[d.act_dtype]
    B = q_abs.shape[0]
    D = d.d_latent + d.d_rope
    _need(q_abs, "q_abs", at, (B, d.n_heads, D))
    _need(kv_cache, "kv_cache", _kv_torch(d))
    _need(block_table, "block_table", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [batch, max_pages]")
    _need(seq_lens, "seq_lens", torch.int32, (B,))
    if seq_starts is not None:
        _need(seq_starts, "seq_starts", torch.int32, (B,))
    if d.kv_dtype == MLA_E4M3:
        _need(kv_scale, "kv_scale", torch.float32, kv_cache.shape[:2])
    if _validating():
        check_paging(block_table, seq_lens, kv_cache.shape[0], d.block_size, seq_starts)
    need = decode_workspace_bytes(d, B, num_splits)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_abs.device)
    if o_lat is None:
        o_lat = torch.empty((B, d.n_heads, d.d_latent), dtype=at, device=q_abs.device)
    _need(o_lat, "o_lat", at, (B, d.n_heads, d.d_latent))
    if lse is None:
        lse = torch.empty((B, d.n_heads), dtype=torch.float32, device=q_abs.device)
    _need(lse, "lse", torch.float32, (B, d.n_heads))
    if seq_starts is None:
        check(_lib.lib().mla_decode(ctypes.byref(d), B, _ptr(q_abs), _ptr(kv_cache), _ptr(kv_scale),
                                    _ptr(block_table), block_table.shape[1], _ptr(seq_lens), num_splits,
                                    _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _ptr(o_lat), _ptr(lse), _stream(stream)), "mla_decode")
    else:
        check(_lib.lib().mla_decode_window(ctypes.byref(d), B, _ptr(q_abs), _ptr(kv_cache), _ptr(kv_scale),
                                           _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
                                           _ptr(seq_starts), num_splits, _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _ptr(o_lat),
                                           _ptr(lse), _stream(stream)), "mla_decode_window")
    return o_lat, lse


def decode_noalloc(d: Dims, q_abs, kv_cache, block_table, seq_lens, kv_scale=None, num_splits: int = 0,
                   o_lat=None, lse=None, stream=None, seq_starts=None):
    """decode without a workspace: the split-KV partials live in the
    library's own device scratch (mla_decode_noalloc).  Allocates nothing
    when o_lat and lse are given.  Calls that overlap on one GPU race."""
    at = _TORCH[d.act_dtype]
    B = q_abs.shape[0]
    D = d.d_latent + d.d_rope
    _need(q_abs, "q_abs", at, (B, d.n_heads, D))
    _need(kv_cache, "kv_cache", _kv_torch(d))
    _need(block_table, "block_table", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [batch, max_pages]")
    _need(seq_lens, "seq_lens", torch.int32, (B,))
    if seq_starts is not None:
        _need(seq_starts, "seq_starts", torch.int32, (B,))
    if d.kv_dtype == MLA_E4M3:
        _need(kv_scale, "kv_scale", torch.float32, kv_cache.shape[:2])
    if _validating():
        check_paging(block_table, seq_lens, kv_cache.shape[0], d.block_size, seq_starts)
    if o_lat is None:
        o_lat = torch.empty((B, d.n_heads, d.d_latent), dtype=at, device=q_abs.device)
    _need(o_lat, "o_lat", at, (B, d.n_heads, d.d_latent))
    if lse is None:
        lse = torch.empty((B, d.n_heads), dtype=torch.float32, device=q_abs.device)
    _need(lse, "lse", torch.float32, (B, d.n_heads))
    check(_lib.lib().mla_decode_noalloc(ctypes.byref(d), B, _ptr(q_abs), _ptr(kv_cache), _ptr(kv_scale),
                                        _ptr(block_table), block_table.shape[1], _ptr(seq_lens), _ptr(seq_starts),
                                        num_splits, _ptr(o_lat), _ptr(lse), _stream(stream)), "mla_decode_noalloc")
    return o_lat, lse


def decode_multi(d: Dims, q_abs, kv_cache, block_table, seq_lens, kv_scale=None, num_splits: int = 0,
                 seq_starts=None, workspace=None, o_lat=None, lse=None, stream=None):
    """q_len query tokens per sequence (q_abs [batch, q_len, n_h, D]), each
    attending causally over its sequence's rows; returns (o_lat, lse) of
    shapes [batch, q_len, n_h, d_c] and [batch, q_len, n_h]."""
    at = _TORCH[d.act_dtype]
    B, q = q_abs.shape[0], q_abs.shape[1]
    D = d.d_latent + d.d_rope
    _need(q_abs, "q_abs", at, (B, q, d.n_heads, D))
    _need(kv_cache, "kv_cache", _kv_torch(d))
    _need(block_table, "block_table", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [batch, max_pages]")
    _need(seq_lens, "seq_lens", torch.int32, (B,))
    if seq_starts is not None:
        _need(seq_starts, "seq_starts", torch.int32, (B,))
    if d.kv_dtype == MLA_E4M3:
        _need(kv_scale, "kv_scale", torch.float32, kv_cache.shape[:2])
    if _validating():
        check_paging(block_table, seq_lens, kv_cache.shape[0], d.block_size, seq_starts)
    need = int(_lib.lib().mla_decode_multi_workspace_bytes(ctypes.byref(d), B, q, num_splits))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_abs.device)
    if o_lat is None:
        o_lat = torch.empty((B, q, d.n_heads, d.d_latent), dtype=at, device=q_abs.device)
    _need(o_lat, "o_lat", at, (B, q, d.n_heads, d.d_latent))
    if lse is None:
        lse = torch.empty((B, q, d.n_heads), dtype=torch.float32, device=q_abs.device)
    _need(lse, "lse", torch.float32, (B, q, d.n_heads))
    check(_lib.lib().mla_decode_multi(ctypes.byref(d), B, q, _ptr(q_abs), _ptr(kv_cache), _ptr(kv_scale),
                                      _ptr(block_table), block_table.shape[1], _ptr(seq_lens), _ptr(seq_starts),
                                      num_splits, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _ptr(o_lat), _ptr(lse), _stream(stream)), "mla_decode_multi")
    return o_lat, lse


def up_v(d: Dims, o_lat, w_uv, out=None, stream=None):
    """out = W_UV o_lat per batch row and head."""
    at = _TORCH[d.act_dtype]
    B = o_lat.shape[0]
    _need(o_lat, "o_lat", at, (B, d.n_heads, d.d_latent))
    _need(w_uv, "w_uv", at, (d.n_heads, d.d_head, d.d_latent))
    if out is None:
        out = torch.empty((B, d.n_heads, d.d_head), dtype=at, device=o_lat.device)
    _need(out, "out", at, (B, d.n_heads, d.d_head))
    check(_lib.lib().mla_up_v(ctypes.byref(d), B, _ptr(o_lat), _ptr(w_uv), _ptr(out), _stream(stream)),
          "mla_up_v")
    return out
