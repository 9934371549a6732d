"""Plain float64 CPU oracle for DeepSeek-V2-style Multi-head Latent Attention decode.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or run this module.  The
library (``mla_latent_kv_38_amd``) never imports it and shares no code with it.

What it computes, and the page passage each step follows:

* [P2] keybo.xyz, "MLA 之后，KV cache 确实得重新理解一遍"
    - section "第一步，训练时": c_kv(t) = W_DKV x(t); k(t) = W_UK c_kv(t);
      v(t) = W_UV c_kv(t).
    - section "第二步，推理时的吸收": score(i,j) = q(i)^T W_UK c_kv(j)
      = (W_UK^T q(i))^T c_kv(j); o(i) = sum_j a(i,j) v(j)
      = W_UV (sum_j a(i,j) c_kv(j)).
    - section "RoPE 为什么必须解耦": RoPE is a position rotation R_p with
      (R_i q)^T (R_j k) = q^T R_(j-i) k; the decoupled key
      k_R(t) = RoPE(W_KR x(t)) has 64 dims and is shared by every head;
      score = q_C^T k_C + q_R^T k_R.
* [P3] dgblog.top, "MLA 是什么 | dg's Blog": sections "1. 下采样（压缩）" and
  "2. 上采样（还原）" (c_KV = W_DKV h_t, k_t = W_UK c_KV, v_t = W_UV c_KV),
  "一个简化的计算示例" (the worked example the tests pin), "PyTorch 代码示例"
  (scores, softmax over cached tokens, weighted sum of values).
* [P4] algomooc.com MLA interview page, section "先区分 KV Cache 与 MLA": a
  decode step appends the new token's key/value and then attends over the
  history plus the current token.

The explicit form below rebuilds k_C and v per head and runs ordinary softmax
attention; the absorbed form (``absorbed_decode``/``latent_decode``) exists so
the tests can check the absorption identity against it.

Readings where the pages leave a step open:
  * q_R has one d_R-vector per head; k_R is one d_R-vector per token shared by
    all heads.
  * RoPE pairs dimensions (2i, 2i+1); theta_i = base^(-2i/d_R); positions are
    0-based token indices; the query token sits at position L-1.
  * The cache length L includes the current token (append, then attend).
  * Softmax scale 1/sqrt(d_h + d_R) multiplies the sum of both score terms.
  * L = 0 gives o_lat = 0, out = 0 and lse = -inf.

Pins: every function here is exercised by ``tests/test_oracle_*.py`` against
the pages' worked example, closed forms, invariants or scalar brute force.
No function is "parity unpinned".
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


# ----------------------------------------------------------------------------
# RoPE  ([P2] section "RoPE 为什么必须解耦": rotation R_p per position)
# ----------------------------------------------------------------------------
def rope_inv_freq(d_rope: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/d_rope) for i in [0, d_rope/2)."""
    i = np.arange(d_rope // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * i / np.float64(d_rope))


def rope(x, pos, base: float) -> np.ndarray:
    """Rotate each pair (x[2i], x[2i+1]) by the angle pos * theta_i.

    ``x`` has shape [..., d]; ``pos`` broadcasts against ``x.shape[:-1]``.
    d = 0 returns an empty copy (no positional part).
    """
    x = _f64(x)
    d = x.shape[-1]
    if d == 0:
        return x.copy()
    if d % 2:
        raise ValueError("RoPE needs an even dimension")
    ang = _f64(pos)[..., None] * rope_inv_freq(d, base)
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    shape = np.broadcast_shapes(x.shape[:-1], ang.shape[:-1]) + (d,)
    out = np.empty(shape, dtype=np.float64)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


# ----------------------------------------------------------------------------
# Projections ([P2] "第一步，训练时"; [P3] "1. 下采样", "2. 上采样")
# ----------------------------------------------------------------------------
def project(h, w_dkv, w_kr, w_q, n_heads: int, d_head: int, d_rope: int):
    """Down-projection of every token plus the query of the last token.

    h: [L, d_model].  Returns (c_kv [L, d_c], k_r_raw [L, d_R],
    q_c [n_heads, d_head], q_r [n_heads, d_rope]); k_r_raw is not rotated yet.
    The query map is one matrix W_Q whose output is read as
    [n_heads, d_head + d_rope] and split into the content and RoPE parts.
    """
    h = _f64(h)
    c_kv = h @ _f64(w_dkv).T
    k_r_raw = h @ _f64(w_kr).T if d_rope else np.zeros((h.shape[0], 0))
    q = (_f64(w_q) @ h[-1]).reshape(n_heads, d_head + d_rope)
    return c_kv, k_r_raw, q[:, :d_head].copy(), q[:, d_head:].copy()


def up_project(c_kv, w_h):
    """Row-wise up-projection of latents by one head's matrix: W c_kv(t).

    c_kv: [L, d_c]; w_h: [d_head, d_c].  Returns [L, d_head].
    """
    return _f64(c_kv) @ _f64(w_h).T


def reconstruct_kv(c_kv, w_uk_h, w_uv_h):
    """Per-head k_C = W_UK c_kv and v = W_UV c_kv for every row of c_kv."""
    return up_project(c_kv, w_uk_h), up_project(c_kv, w_uv_h)


# ----------------------------------------------------------------------------
# Explicit attention: the oracle's definition of one decode step
# ----------------------------------------------------------------------------
def explicit_decode(q_c, q_r, c_kv, k_r, w_uk, w_uv, *, scale: float, base: float,
                    q_pos=None, k_pos=None, k_r_rotated: bool = False,
                    heads=None, chunk: int = 2048, return_weights: bool = False):
    """One sequence, one query token, every listed head.

    q_c [n_h, d_h], q_r [n_h, d_R] (pre-RoPE), c_kv [L, d_c], k_r [L, d_R]
    (pre-RoPE unless ``k_r_rotated``), w_uk/w_uv [n_h, d_h, d_c].

    For each head: k_C = W_UK c_kv and v = W_UV c_kv are rebuilt explicitly,
    s_j = (q_C . k_C(j) + RoPE(q_R) . RoPE(k_R(j))) * scale, a = softmax(s)
    (two passes: all scores, then normalise), out = sum_j a_j v(j).
    Secondary outputs: lse = log sum_j exp(s_j) and o_lat = sum_j a_j c_kv(j).
    """
    q_c, q_r, c_kv, k_r = _f64(q_c), _f64(q_r), _f64(c_kv), _f64(k_r)
    L = c_kv.shape[0]
    n_h, d_h = q_c.shape
    d_c = c_kv.shape[1]
    heads = list(range(n_h)) if heads is None else list(heads)
    if q_pos is None:
        q_pos = L - 1
    if k_pos is None:
        k_pos = np.arange(L)
    out = np.zeros((len(heads), d_h))
    o_lat = np.zeros((len(heads), d_c))
    lse = np.full(len(heads), -np.inf)
    weights = np.zeros((len(heads), L)) if return_weights else None
    if L == 0:
        return dict(out=out, o_lat=o_lat, lse=lse, weights=weights, heads=heads)
    k_rot = k_r if k_r_rotated else rope(k_r, k_pos, base)  # shared by all heads
    for n, h in enumerate(heads):
        q_rot = rope(q_r[h], q_pos, base)
        s = np.empty(L)
        for j0 in range(0, L, chunk):
            k_c = up_project(c_kv[j0:j0 + chunk], w_uk[h])
            s[j0:j0 + chunk] = (k_c @ q_c[h] + k_rot[j0:j0 + chunk] @ q_rot) * scale
        m = s.max()
        e = np.exp(s - m)
        denom = e.sum()
        a = e / denom
        for j0 in range(0, L, chunk):
            v = up_project(c_kv[j0:j0 + chunk], w_uv[h])
            out[n] += a[j0:j0 + chunk] @ v
        o_lat[n] = a @ c_kv
        lse[n] = m + np.log(denom)
        if return_weights:
            weights[n] = a
    return dict(out=out, o_lat=o_lat, lse=lse, weights=weights, heads=heads)


def window_decode(q_c, q_r, c_kv, k_r, w_uk, w_uv, *, start: int, scale: float, base: float,
                  k_r_rotated: bool = False, heads=None):
    """Decode of one sequence that attends only to its rows j >= start.

    ([P2] "所以 cache 逻辑到底哪里要重写": with the cache paged by token
    latent, eviction such as a sliding window works as before.)  The rows
    keep their absolute positions (RoPE of row j uses position j) and the
    query stays at position L - 1; rows before ``start`` simply take no part.
    An empty window (start >= L) gives o_lat = 0, out = 0, lse = -inf.
    """
    c_kv, k_r = _f64(c_kv), _f64(k_r)
    L = c_kv.shape[0]
    start = min(max(int(start), 0), L)
    return explicit_decode(q_c, q_r, c_kv[start:], k_r[start:], w_uk, w_uv, scale=scale, base=base,
                           q_pos=L - 1, k_pos=np.arange(start, L), k_r_rotated=k_r_rotated, heads=heads)


def multi_query_decode(q_c, q_r, c_kv, k_r, w_uk, w_uv, *, scale: float, base: float, start: int = 0,
                       k_r_rotated: bool = False, heads=None):
    """Several new tokens of one sequence, each attending causally.

    ([P4] "先区分 KV Cache 与 MLA": new tokens are appended, then attend over
    history plus current; [P2] "第一步，训练时": a token attends over the
    tokens up to itself.)  q_c [q, n_h, d_h], q_r [q, n_h, d_R]; the last q of
    the L rows are the queries' own, so query i sits at position
    p = L - q + i and attends to rows start .. p.  Returns per-query lists
    stacked: out [q, heads, d_h], o_lat [q, heads, d_c], lse [q, heads]; a
    query with no row (p < start) gets zeros and -inf.
    """
    q_c, q_r, c_kv, k_r = _f64(q_c), _f64(q_r), _f64(c_kv), _f64(k_r)
    q, L = q_c.shape[0], c_kv.shape[0]
    res = []
    for i in range(q):
        p = L - q + i
        lo = min(max(int(start), 0), max(p + 1, 0))
        hi = max(p + 1, 0)
        res.append(explicit_decode(q_c[i], q_r[i], c_kv[lo:hi], k_r[lo:hi], w_uk, w_uv, scale=scale, base=base,
                                   q_pos=p, k_pos=np.arange(lo, hi), k_r_rotated=k_r_rotated, heads=heads))
    return dict(out=np.stack([r["out"] for r in res]), o_lat=np.stack([r["o_lat"] for r in res]),
                lse=np.stack([r["lse"] for r in res]), heads=res[0]["heads"])


# ----------------------------------------------------------------------------
# Absorbed form ([P2] "第二步，推理时的吸收"; [P3] "3. 一个聪明的优化")
# ----------------------------------------------------------------------------
def absorb_q(q_c, q_r, w_uk, pos, base: float):
    """q_abs[b, h] = [W_UK[h]^T q_C[b, h] || RoPE(q_R[b, h], pos[b])].

    q_c [B, n_h, d_h], q_r [B, n_h, d_R], w_uk [n_h, d_h, d_c], pos [B].
    Returns [B, n_h, d_c + d_R].
    """
    q_c, q_r, w_uk = _f64(q_c), _f64(q_r), _f64(w_uk)
    B, n_h, _ = q_c.shape
    d_c = w_uk.shape[2]
    q_lat = np.empty((B, n_h, d_c))
    for h in range(n_h):
        q_lat[:, h, :] = q_c[:, h, :] @ w_uk[h]
    q_rot = rope(q_r, _f64(pos)[:, None], base)
    return np.concatenate([q_lat, q_rot], axis=-1)


def cache_rows(c_kv, k_r_raw, pos, base: float):
    """The latent cache row of each token: [c_kv || RoPE(k_R, pos)], [T, d_c + d_R].

    ([P2] "第三步，结论": 512 + 64 values per token per layer; the RoPE key is
    rotated before it is cached.)
    """
    return np.concatenate([_f64(c_kv), rope(k_r_raw, _f64(pos), base)], axis=-1)


def projected_rows(h, w_dkv, w_kr, pos, base: float, act: str):
    """Cache rows of new tokens straight from their hidden states.

    ([P2] "第一步，训练时": c_kv = W_DKV x, only the latent is cached; [P2]
    "RoPE 为什么必须解耦": k_R = RoPE(W_KR x), rotated before caching.)  The
    projections are stored in the activation type before they are appended,
    so each is rounded once to ``act`` ("f32" or "bf16"); the row is then
    [c_kv || RoPE(k_R, pos)] as in ``cache_rows``.
    """
    rnd = to_bf16 if act == "bf16" else to_f32
    h = _f64(h)
    c_kv = rnd(h @ _f64(w_dkv).T).astype(np.float64)
    k_r = rnd(h @ _f64(w_kr).T).astype(np.float64) if np.asarray(w_kr).size else np.zeros((h.shape[0], 0))
    return cache_rows(c_kv, k_r, pos, base)


def latent_decode(q_abs, rows, d_c: int, scale: float):
    """Attention of absorbed queries over latent rows, as plainly defined.

    q_abs [n_h, D], rows [L, D] with D = d_c + d_R.  s_j = scale * q_abs . row_j,
    a = softmax(s), o_lat = sum_j a_j row_j[:d_c], lse = log sum_j exp(s_j).
    """
    q_abs, rows = _f64(q_abs), _f64(rows)
    n_h = q_abs.shape[0]
    L = rows.shape[0]
    if L == 0:
        return dict(o_lat=np.zeros((n_h, d_c)), lse=np.full(n_h, -np.inf))
    s = (q_abs @ rows.T) * scale              # [n_h, L]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    denom = e.sum(axis=1, keepdims=True)
    a = e / denom
    return dict(o_lat=a @ rows[:, :d_c], lse=(m + np.log(denom))[:, 0], weights=a)


def up_v(o_lat, w_uv):
    """out[b, h] = W_UV[h] o_lat[b, h]; o_lat [B, n_h, d_c], w_uv [n_h, d_h, d_c]."""
    o_lat, w_uv = _f64(o_lat), _f64(w_uv)
    out = np.empty(o_lat.shape[:2] + (w_uv.shape[1],))
    for h in range(w_uv.shape[0]):
        out[:, h, :] = o_lat[:, h, :] @ w_uv[h].T
    return out


def absorbed_decode(q_c, q_r, c_kv, k_r_raw, w_uk, w_uv, *, scale: float, base: float):
    """The absorbed computation for one sequence: absorb the query, attend over
    latent rows, then one W_UV up-projection.  Used only to check the
    absorption identity against ``explicit_decode``."""
    L = _f64(c_kv).shape[0]
    q_abs = absorb_q(_f64(q_c)[None], _f64(q_r)[None], w_uk, np.array([L - 1]), base)[0]
    rows = cache_rows(c_kv, k_r_raw, np.arange(L), base)
    res = latent_decode(q_abs, rows, _f64(c_kv).shape[1], scale)
    res["out"] = up_v(res["o_lat"][None], w_uv)[0]
    return res


# ----------------------------------------------------------------------------
# Paged cache ([P2] "所以 cache 逻辑到底哪里要重写": paged by token latent)
# ----------------------------------------------------------------------------
def slot_of(block_table_row, j: int, block_size: int) -> int:
    """Physical slot of logical token j of one sequence."""
    return int(block_table_row[j // block_size]) * block_size + j % block_size


def gather_pages(pool, block_table_row, L: int):
    """Read a sequence's L rows through its page table; pool is [pages, bs, D]."""
    pool = np.asarray(pool)
    bs = pool.shape[1]
    idx = np.arange(L)
    pages = np.asarray(block_table_row)[idx // bs]
    return pool[pages, idx % bs]


# ----------------------------------------------------------------------------
# Rounding of expected values to device storage types (the oracle's own)
# ----------------------------------------------------------------------------
def to_f32(x) -> np.ndarray:
    """Round float64 to the nearest float32 (ties to even)."""
    return _f64(x).astype(np.float32)


def to_bf16(x) -> np.ndarray:
    """Round to float32 (nearest-even), then to bfloat16 (nearest-even).

    Returned as float32 holding bfloat16 values.  The bfloat16 step keeps the
    upper 16 bits and rounds up when the dropped half exceeds 0x8000, or equals
    it and the kept part is odd.
    """
    u = to_f32(x).view(np.uint32).astype(np.uint64)
    kept = u & 0xFFFF0000
    dropped = u & 0xFFFF
    odd = (kept >> 16) & 1
    up = (dropped > 0x8000) | ((dropped == 0x8000) & (odd == 1))
    return (kept + np.where(up, 0x10000, 0)).astype(np.uint32).view(np.float32)
