"""Pins for the float64 oracle: each check rests on something other than the
oracle itself (the pages' worked example, closed forms, invariants of the
mathematics, pure-Python brute force, or an independent library routine)."""
import json
import math
import os

import numpy as np
import pytest

from oracle import mla_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden():
    with open(os.path.join(HERE, "golden", "worked_example.json")) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Worked example printed on the page (dgblog.top, "一个简化的计算示例")
# ---------------------------------------------------------------------------
def test_worked_example_projection():
    g = _golden()
    h = np.array(g["h"], float)[None, :]
    c_kv, k_r, q_c, q_r = O.project(h, g["W_DKV"], np.zeros((0, 4)), np.zeros((3, 4)),
                                    n_heads=1, d_head=3, d_rope=0)
    assert c_kv[0].tolist() == g["expected"]["c_KV"]
    k, v = O.reconstruct_kv(c_kv, g["W_UK"], g["W_UV"])
    assert k[0].tolist() == g["expected"]["k"]
    assert v[0].tolist() == g["expected"]["v"]
    # cached numbers: k and v per head (2 * n_heads * d_n) against the latent (d_c)
    assert 2 * g["n_heads"] * g["d_n"] == g["expected"]["cached_numbers_before"]
    assert c_kv.shape[1] == g["expected"]["cached_numbers_after"]


def test_project_unit_hidden_states_pick_weight_columns():
    """h_j = e_(k_j) (one-hot rows): c_kv[j] is column k_j of W_DKV, the raw
    RoPE key k_r[j] is column k_j of W_KR, and the query of the last token is
    column k_(L-1) of W_Q read as [n_h, d_h + d_R]: its first d_h entries per
    head are q_C, the remaining d_R are q_R.  Checked entry by entry with
    scalar indexing."""
    rng = np.random.default_rng(21)
    n_h, d_h, d_r, d_c, dm = 3, 4, 2, 5, 7
    w_dkv = rng.standard_normal((d_c, dm))
    w_kr = rng.standard_normal((d_r, dm))
    w_q = rng.standard_normal((n_h * (d_h + d_r), dm))
    ks = [3, 0, 6, 2]
    h = np.zeros((len(ks), dm))
    for j, k in enumerate(ks):
        h[j, k] = 1.0
    c_kv, k_r, q_c, q_r = O.project(h, w_dkv, w_kr, w_q, n_h, d_h, d_r)
    for j, k in enumerate(ks):
        for c in range(d_c):
            assert c_kv[j, c] == w_dkv[c, k]
        for i in range(d_r):
            assert k_r[j, i] == w_kr[i, k]
    kq = ks[-1]
    for hh in range(n_h):
        for i in range(d_h):
            assert q_c[hh, i] == w_q[hh * (d_h + d_r) + i, kq]
        for i in range(d_r):
            assert q_r[hh, i] == w_q[hh * (d_h + d_r) + d_h + i, kq]


def test_project_is_linear_in_the_hidden_state():
    """Two one-hot rows added give the sum of their columns (the map is the
    matrix product, nothing else)."""
    rng = np.random.default_rng(22)
    n_h, d_h, d_r, d_c, dm = 2, 3, 2, 4, 5
    w_dkv, w_kr = rng.standard_normal((d_c, dm)), rng.standard_normal((d_r, dm))
    w_q = rng.standard_normal((n_h * (d_h + d_r), dm))
    h = np.zeros((1, dm))
    h[0, 1], h[0, 4] = 2.0, -3.0
    c_kv, k_r, q_c, q_r = O.project(h, w_dkv, w_kr, w_q, n_h, d_h, d_r)
    np.testing.assert_allclose(c_kv[0], 2 * w_dkv[:, 1] - 3 * w_dkv[:, 4], rtol=0, atol=1e-14)
    np.testing.assert_allclose(k_r[0], 2 * w_kr[:, 1] - 3 * w_kr[:, 4], rtol=0, atol=1e-14)
    q = (2 * w_q[:, 1] - 3 * w_q[:, 4]).reshape(n_h, d_h + d_r)
    np.testing.assert_allclose(q_c, q[:, :d_h], rtol=0, atol=1e-14)
    np.testing.assert_allclose(q_r, q[:, d_h:], rtol=0, atol=1e-14)


def test_worked_example_single_token_attends_to_its_value():
    """With one cached token the softmax weight is 1, so out = v exactly."""
    g = _golden()
    c_kv = np.array([g["expected"]["c_KV"]], float)
    w_uk = np.array(g["W_UK"], float)[None]
    w_uv = np.array(g["W_UV"], float)[None]
    for q in ([1.0, 1.0, 1.0], [-3.0, 0.5, 7.0]):
        res = O.explicit_decode(np.array([q]), np.zeros((1, 0)), c_kv, np.zeros((1, 0)),
                                w_uk, w_uv, scale=1 / math.sqrt(3), base=10000.0)
        assert res["out"][0].tolist() == g["expected"]["v"]
        assert res["o_lat"][0].tolist() == g["expected"]["c_KV"]


def test_worked_example_absorbed_score():
    """q . k = (W_UK^T q) . c_KV for the page's matrices: 6 both ways."""
    g = _golden()
    q = np.array([1.0, 1.0, 1.0])
    k = np.array(g["expected"]["k"], float)
    q_abs = O.absorb_q(q[None, None], np.zeros((1, 1, 0)), np.array(g["W_UK"], float)[None],
                       np.array([0]), 10000.0)[0, 0]
    assert q_abs.tolist() == [2.0, 2.0]
    assert float(q @ k) == 6.0
    assert float(q_abs @ np.array(g["expected"]["c_KV"], float)) == 6.0


# ---------------------------------------------------------------------------
# Pure-Python brute force (scalar loops, math.fsum) on tiny shapes
# ---------------------------------------------------------------------------
def _bf_rope(vec, p, base):
    d = len(vec)
    out = []
    for i in range(d // 2):
        a = p * base ** (-2.0 * i / d)
        x, y = vec[2 * i], vec[2 * i + 1]
        out += [x * math.cos(a) - y * math.sin(a), x * math.sin(a) + y * math.cos(a)]
    return out


def _bf_decode(q_c, q_r, c_kv, k_r, w_uk, w_uv, scale, base, start=0):
    n_h, d_h = len(q_c), len(q_c[0])
    L, d_c = len(c_kv), len(c_kv[0])
    outs, lses, olats = [], [], []
    for h in range(n_h):
        qr = _bf_rope(q_r[h], L - 1, base)
        s, vs = [], []
        for j in range(start, L):
            kc = [math.fsum(w_uk[h][i][c] * c_kv[j][c] for c in range(d_c)) for i in range(d_h)]
            vs.append([math.fsum(w_uv[h][i][c] * c_kv[j][c] for c in range(d_c)) for i in range(d_h)])
            kr = _bf_rope(k_r[j], j, base)
            s.append((math.fsum(q_c[h][i] * kc[i] for i in range(d_h))
                      + math.fsum(qr[i] * kr[i] for i in range(len(kr)))) * scale)
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = math.fsum(e)
        a = [x / z for x in e]
        n = len(s)
        outs.append([math.fsum(a[j] * vs[j][i] for j in range(n)) for i in range(d_h)])
        olats.append([math.fsum(a[j] * c_kv[start + j][c] for j in range(n)) for c in range(d_c)])
        lses.append(m + math.log(z))
    return np.array(outs), np.array(olats), np.array(lses)


@pytest.mark.parametrize("n_h,d_h,d_c,d_r,L", [
    (1, 3, 2, 0, 1), (1, 3, 2, 2, 2), (2, 4, 4, 2, 5), (2, 3, 4, 4, 6), (1, 4, 2, 4, 6),
])
def test_brute_force_matches_oracle(n_h, d_h, d_c, d_r, L):
    rng = np.random.default_rng(100 + 7 * L + d_r)
    q_c = rng.standard_normal((n_h, d_h))
    q_r = rng.standard_normal((n_h, d_r))
    c_kv = rng.standard_normal((L, d_c))
    k_r = rng.standard_normal((L, d_r))
    w_uk = rng.standard_normal((n_h, d_h, d_c))
    w_uv = rng.standard_normal((n_h, d_h, d_c))
    scale, base = 1 / math.sqrt(d_h + d_r), 50.0
    bo, bl, bs = _bf_decode(q_c.tolist(), q_r.tolist(), c_kv.tolist(), k_r.tolist(),
                            w_uk.tolist(), w_uv.tolist(), scale, base)
    ex = O.explicit_decode(q_c, q_r, c_kv, k_r, w_uk, w_uv, scale=scale, base=base, chunk=2)
    ab = O.absorbed_decode(q_c, q_r, c_kv, k_r, w_uk, w_uv, scale=scale, base=base)
    for res in (ex, ab):
        np.testing.assert_allclose(res["out"], bo, rtol=0, atol=1e-13 * np.abs(bo).max())
        np.testing.assert_allclose(res["o_lat"], bl, rtol=0, atol=1e-13 * np.abs(bl).max())
        np.testing.assert_allclose(res["lse"], bs, rtol=0, atol=1e-13 * max(1, np.abs(bs).max()))


# ---------------------------------------------------------------------------
# Sliding window (keybo.xyz, "所以 cache 逻辑到底哪里要重写": eviction such as a
# sliding window works as before over the latent rows)
# ---------------------------------------------------------------------------
def _window_case(seed, n_h=2, d_h=3, d_c=4, d_r=4, L=7):
    rng = np.random.default_rng(200 + seed)
    return (rng.standard_normal((n_h, d_h)), rng.standard_normal((n_h, d_r)), rng.standard_normal((L, d_c)),
            rng.standard_normal((L, d_r)), rng.standard_normal((n_h, d_h, d_c)),
            rng.standard_normal((n_h, d_h, d_c)))


@pytest.mark.parametrize("start", [0, 1, 3, 6])
def test_window_matches_brute_force(start):
    args = _window_case(start)
    scale, base = 1 / math.sqrt(3 + 4), 50.0
    bo, bl, bs = _bf_decode(*[a.tolist() for a in args], scale, base, start=start)
    res = O.window_decode(*args, start=start, scale=scale, base=base)
    np.testing.assert_allclose(res["out"], bo, rtol=0, atol=1e-13 * np.abs(bo).max())
    np.testing.assert_allclose(res["o_lat"], bl, rtol=0, atol=1e-13 * np.abs(bl).max())
    np.testing.assert_allclose(res["lse"], bs, rtol=0, atol=1e-13 * max(1, np.abs(bs).max()))


def test_window_and_its_complement_recombine_to_the_whole():
    """Attention over rows [0, s) and over [s, L) merged by log-sum-exp equals
    attention over all L rows (the softmax sum splits exactly)."""
    args = _window_case(9, n_h=3, d_h=5, d_c=6, d_r=4, L=23)
    q_c, q_r, c_kv, k_r, w_uk, w_uv = args
    kw = dict(scale=0.3, base=1000.0)
    full = O.explicit_decode(*args, **kw)
    for s in (1, 10, 22):
        a = O.explicit_decode(q_c, q_r, c_kv[:s], k_r[:s], w_uk, w_uv, q_pos=22, **kw)
        b = O.window_decode(*args, start=s, **kw)
        m = np.maximum(a["lse"], b["lse"])
        wa, wb = np.exp(a["lse"] - m), np.exp(b["lse"] - m)
        lse = m + np.log(wa + wb)
        out = (wa[:, None] * a["out"] + wb[:, None] * b["out"]) / (wa + wb)[:, None]
        np.testing.assert_allclose(lse, full["lse"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(out, full["out"], rtol=0, atol=1e-12 * np.abs(full["out"]).max())


def test_window_ignores_rows_before_it_and_empty_window():
    args = list(_window_case(4, L=9))
    kw = dict(scale=0.5, base=100.0)
    ref = O.window_decode(*args, start=5, **kw)
    args[2] = args[2].copy(); args[3] = args[3].copy()
    args[2][:5] = 1e6
    args[3][:5] = -1e6
    got = O.window_decode(*args, start=5, **kw)
    for k in ("out", "o_lat", "lse"):
        np.testing.assert_array_equal(got[k], ref[k])
    e = O.window_decode(*args, start=9, **kw)
    assert np.all(e["o_lat"] == 0) and np.all(e["out"] == 0) and np.all(np.isneginf(e["lse"]))


# ---------------------------------------------------------------------------
# Several new tokens per sequence, each attending causally (algomooc.com
# "先区分 KV Cache 与 MLA"; keybo.xyz "第一步，训练时")
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("q,start", [(1, 0), (3, 0), (3, 2), (4, 5)])
def test_multi_query_matches_brute_force(q, start):
    rng = np.random.default_rng(300 + q + start)
    n_h, d_h, d_c, d_r, L = 2, 3, 4, 4, 7
    q_c, q_r = rng.standard_normal((q, n_h, d_h)), rng.standard_normal((q, n_h, d_r))
    c_kv, k_r = rng.standard_normal((L, d_c)), rng.standard_normal((L, d_r))
    w_uk, w_uv = rng.standard_normal((n_h, d_h, d_c)), rng.standard_normal((n_h, d_h, d_c))
    scale, base = 0.4, 50.0
    res = O.multi_query_decode(q_c, q_r, c_kv, k_r, w_uk, w_uv, scale=scale, base=base, start=start)
    for i in range(q):
        p = L - q + i
        if p < start:
            assert np.all(res["o_lat"][i] == 0) and np.all(np.isneginf(res["lse"][i]))
            continue
        bo, bl, bs = _bf_decode(q_c[i].tolist(), q_r[i].tolist(), c_kv[:p + 1].tolist(), k_r[:p + 1].tolist(),
                                w_uk.tolist(), w_uv.tolist(), scale, base, start=start)
        np.testing.assert_allclose(res["out"][i], bo, rtol=0, atol=1e-13 * np.abs(bo).max())
        np.testing.assert_allclose(res["o_lat"][i], bl, rtol=0, atol=1e-13 * np.abs(bl).max())
        np.testing.assert_allclose(res["lse"][i], bs, rtol=0, atol=1e-13 * max(1, np.abs(bs).max()))


def test_multi_query_is_causal():
    """Changing the rows after a query's own position leaves it unchanged;
    the last query sees everything."""
    rng = np.random.default_rng(17)
    n_h, d_h, d_c, d_r, L, q = 2, 4, 6, 4, 12, 4
    args = [rng.standard_normal((q, n_h, d_h)), rng.standard_normal((q, n_h, d_r)),
            rng.standard_normal((L, d_c)), rng.standard_normal((L, d_r)),
            rng.standard_normal((n_h, d_h, d_c)), rng.standard_normal((n_h, d_h, d_c))]
    kw = dict(scale=0.3, base=100.0)
    a = O.multi_query_decode(*args, **kw)
    args[2] = args[2].copy(); args[3] = args[3].copy()
    args[2][L - 1] += 5.0
    args[3][L - 1] -= 3.0
    b = O.multi_query_decode(*args, **kw)
    for k in ("out", "o_lat", "lse"):
        np.testing.assert_array_equal(a[k][:q - 1], b[k][:q - 1])
        assert not np.allclose(a[k][q - 1], b[k][q - 1])
    full = O.explicit_decode(args[0][q - 1], args[1][q - 1], args[2], args[3], args[4], args[5], **kw)
    np.testing.assert_allclose(b["out"][q - 1], full["out"], rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# Rows straight from hidden states (keybo.xyz "第一步，训练时" and "RoPE 为什么必须解耦")
# ---------------------------------------------------------------------------
def test_projected_rows_of_unit_hidden_states_are_weight_columns():
    """h = e_k (exact in bf16): the latent is column k of W_DKV and the RoPE
    part is column k of W_KR rotated by the token's position (scalar RoPE)."""
    rng = np.random.default_rng(12)
    dm, d_c, d_r = 24, 8, 6
    w_dkv = O.to_bf16(rng.standard_normal((d_c, dm))).astype(float)
    w_kr = O.to_bf16(rng.standard_normal((d_r, dm))).astype(float)
    ks = [0, 5, 23]
    pos = np.array([0, 7, 130])
    h = np.zeros((3, dm))
    h[np.arange(3), ks] = 1.0
    rows = O.projected_rows(h, w_dkv, w_kr, pos, 500.0, "bf16")
    for i, k in enumerate(ks):
        np.testing.assert_array_equal(rows[i, :d_c], w_dkv[:, k])
        np.testing.assert_allclose(rows[i, d_c:], _bf_rope(list(w_kr[:, k]), int(pos[i]), 500.0), rtol=0, atol=1e-12)


def test_projected_rows_round_each_projection_once():
    """2 h gives exactly twice the bf16 latent of h (scaling by 2 commutes with
    rounding), and an f32 latent differs from the exact product by at most
    half an f32 ulp."""
    rng = np.random.default_rng(13)
    dm = 40
    h = rng.standard_normal((4, dm))
    w_dkv, w_kr = rng.standard_normal((16, dm)), rng.standard_normal((4, dm))
    pos = np.arange(4)
    a = O.projected_rows(h, w_dkv, w_kr, pos, 100.0, "bf16")
    b = O.projected_rows(2 * h, w_dkv, w_kr, pos, 100.0, "bf16")
    np.testing.assert_array_equal(b[:, :16], 2 * a[:, :16])
    f = O.projected_rows(h, w_dkv, w_kr, pos, 100.0, "f32")[:, :16]
    exact = h @ w_dkv.T
    assert np.all(np.abs(f - exact) <= np.abs(exact) * 2.0 ** -24)


# ---------------------------------------------------------------------------
# Absorption identity (keybo.xyz, "第二步，推理时的吸收")
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_absorbed_equals_explicit(seed):
    rng = np.random.default_rng(seed)
    n_h, d_h, d_c, d_r, L = 3, 8, 16, 8, 37 + seed * 50
    args = (rng.standard_normal((n_h, d_h)), rng.standard_normal((n_h, d_r)),
            rng.standard_normal((L, d_c)), rng.standard_normal((L, d_r)),
            rng.standard_normal((n_h, d_h, d_c)) / 4, rng.standard_normal((n_h, d_h, d_c)) / 4)
    kw = dict(scale=1 / math.sqrt(d_h + d_r), base=10000.0)
    ex = O.explicit_decode(*args, **kw, chunk=16)
    ab = O.absorbed_decode(*args, **kw)
    for key in ("out", "o_lat", "lse"):
        ref = ex[key]
        assert np.abs(ab[key] - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_absorbed_batch_query_matches_per_sequence():
    rng = np.random.default_rng(5)
    B, n_h, d_h, d_c, d_r = 3, 2, 4, 6, 4
    q_c, q_r = rng.standard_normal((B, n_h, d_h)), rng.standard_normal((B, n_h, d_r))
    w_uk = rng.standard_normal((n_h, d_h, d_c))
    pos = np.array([0, 5, 17])
    q_abs = O.absorb_q(q_c, q_r, w_uk, pos, 10000.0)
    for b in range(B):
        for h in range(n_h):
            np.testing.assert_allclose(q_abs[b, h, :d_c], w_uk[h].T @ q_c[b, h], rtol=1e-14)
            np.testing.assert_allclose(q_abs[b, h, d_c:], _bf_rope(q_r[b, h].tolist(), pos[b], 10000.0),
                                       rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# RoPE (keybo.xyz, "RoPE 为什么必须解耦")
# ---------------------------------------------------------------------------
def test_rope_closed_forms():
    x = np.array([0.3, -1.7])
    assert np.array_equal(O.rope(x, 0, 10000.0), x)          # p = 0 is the identity
    for p in (1.0, 2.5, 1000.0):                                # d = 2: plain rotation by p
        c, s = math.cos(p), math.sin(p)
        np.testing.assert_allclose(O.rope(x, p, 10000.0), [0.3 * c + 1.7 * s, 0.3 * s - 1.7 * c],
                                   rtol=0, atol=1e-15)
    # d = 4, base 100: frequencies 1 and 100^(-1/2) = 0.1
    np.testing.assert_allclose(O.rope_inv_freq(4, 100.0), [1.0, 0.1], rtol=1e-15)
    p = 3.0
    np.testing.assert_allclose(O.rope(np.array([1.0, 0.0, 1.0, 0.0]), p, 100.0),
                               [math.cos(p), math.sin(p), math.cos(0.1 * p), math.sin(0.1 * p)],
                               rtol=0, atol=1e-15)


def test_rope_norm_and_relative_position():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for i, j in ((0, 0), (3, 11), (4000, 131071)):
        np.testing.assert_allclose(np.linalg.norm(O.rope(q, i, 1e4)), np.linalg.norm(q), rtol=1e-14)
        lhs = O.rope(q, i, 1e4) @ O.rope(k, j, 1e4)
        # (R_i q)^T (R_j k) = q^T R_(j-i) k
        assert abs(lhs - q @ O.rope(k, j - i, 1e4)) < 1e-9


def test_decode_is_shift_invariant():
    rng = np.random.default_rng(4)
    n_h, d_h, d_c, d_r, L = 2, 4, 8, 8, 20
    args = (rng.standard_normal((n_h, d_h)), rng.standard_normal((n_h, d_r)),
            rng.standard_normal((L, d_c)), rng.standard_normal((L, d_r)),
            rng.standard_normal((n_h, d_h, d_c)), rng.standard_normal((n_h, d_h, d_c)))
    kw = dict(scale=0.3, base=10000.0)
    a = O.explicit_decode(*args, **kw)
    for delta in (1, 777, 100000):
        b = O.explicit_decode(*args, **kw, q_pos=L - 1 + delta, k_pos=np.arange(L) + delta)
        np.testing.assert_allclose(b["out"], a["out"], rtol=0, atol=1e-9)
        np.testing.assert_allclose(b["lse"], a["lse"], rtol=0, atol=1e-9)


# ---------------------------------------------------------------------------
# Softmax and weighted sum
# ---------------------------------------------------------------------------
def test_softmax_rows_sum_to_one_and_two_token_closed_form():
    rng = np.random.default_rng(6)
    n_h, d_h, d_c, d_r = 3, 4, 6, 2
    w_uk, w_uv = rng.standard_normal((2, n_h, d_h, d_c))
    q_c, q_r = rng.standard_normal((n_h, d_h)), rng.standard_normal((n_h, d_r))
    c_kv, k_r = rng.standard_normal((40, d_c)), rng.standard_normal((40, d_r))
    res = O.explicit_decode(q_c, q_r, c_kv, k_r, w_uk, w_uv, scale=0.5, base=10000.0,
                            return_weights=True)
    assert np.abs(res["weights"].sum(axis=1) - 1).max() < 1e-14
    # two tokens: a_1 = sigmoid(s_1 - s_0)
    res2 = O.explicit_decode(q_c, q_r, c_kv[:2], k_r[:2], w_uk, w_uv, scale=0.5, base=10000.0,
                             return_weights=True)
    for h in range(n_h):
        qr = O.rope(q_r[h], 1, 10000.0)
        s = [(q_c[h] @ (w_uk[h] @ c_kv[j]) + qr @ O.rope(k_r[j], j, 10000.0)) * 0.5 for j in (0, 1)]
        assert abs(res2["weights"][h, 1] - 1 / (1 + math.exp(s[0] - s[1]))) < 1e-14


def test_identical_latents_give_projected_value():
    rng = np.random.default_rng(7)
    n_h, d_h, d_c, d_r, L = 2, 5, 6, 4, 9
    c = rng.standard_normal(d_c)
    w_uk, w_uv = rng.standard_normal((2, n_h, d_h, d_c))
    res = O.explicit_decode(rng.standard_normal((n_h, d_h)), rng.standard_normal((n_h, d_r)),
                            np.tile(c, (L, 1)), rng.standard_normal((L, d_r)), w_uk, w_uv,
                            scale=1.0, base=10000.0)
    for h in range(n_h):
        np.testing.assert_allclose(res["out"][h], w_uv[h] @ c, rtol=1e-13)


def test_empty_sequence():
    res = O.explicit_decode(np.ones((2, 3)), np.ones((2, 2)), np.zeros((0, 4)), np.zeros((0, 2)),
                            np.ones((2, 3, 4)), np.ones((2, 3, 4)), scale=1.0, base=1e4)
    assert np.all(res["out"] == 0) and np.all(res["o_lat"] == 0) and np.all(res["lse"] == -np.inf)
    lat = O.latent_decode(np.ones((2, 6)), np.zeros((0, 6)), 4, 1.0)
    assert np.all(lat["o_lat"] == 0) and np.all(lat["lse"] == -np.inf)


# ---------------------------------------------------------------------------
# Paging (keybo.xyz, "所以 cache 逻辑到底哪里要重写": paged by token latent)
# ---------------------------------------------------------------------------
def test_slot_of_hand_computed_table():
    """Block-table row [2, 0, 1] with 4-token pages: logical token j lives in
    physical page row[j // 4] at offset j % 4, so its slot is
    4 * row[j // 4] + j % 4.  The table below is written out by hand."""
    row = [2, 0, 1]
    expected = {0: 8, 1: 9, 3: 11, 4: 0, 5: 1, 7: 3, 8: 4, 9: 5, 11: 7}
    for j, slot in expected.items():
        assert O.slot_of(row, j, 4) == slot


def test_gather_pages_hand_computed_rows():
    """A pool whose entry (page p, offset o) holds the value 10 p + o: reading
    row [2, 0, 1] for 6 tokens gives pages 2 then 0, offsets 0..3 then 0..1."""
    pool = np.array([[[10.0 * p + o] for o in range(4)] for p in range(3)])
    got = O.gather_pages(pool, [2, 0, 1], 6)[:, 0].tolist()
    assert got == [20.0, 21.0, 22.0, 23.0, 0.0, 1.0]
    got = O.gather_pages(pool, [1, 2, 0], 9)[:, 0].tolist()
    assert got == [10.0, 11.0, 12.0, 13.0, 20.0, 21.0, 22.0, 23.0, 0.0]


def test_paged_gather_is_exact_under_any_page_table():
    rng = np.random.default_rng(8)
    bs, D, L = 4, 6, 13
    rows = rng.standard_normal((L, D))
    n_pages = (L + bs - 1) // bs
    for perm in (np.arange(n_pages), rng.permutation(n_pages + 3)[:n_pages]):
        pool = np.full((n_pages + 3, bs, D), np.nan)
        for j in range(L):
            s = O.slot_of(perm, j, bs)
            pool[s // bs, s % bs] = rows[j]
        assert np.array_equal(O.gather_pages(pool, perm, L), rows)


# ---------------------------------------------------------------------------
# Rounding of expected values: against independent implementations
# ---------------------------------------------------------------------------
def test_bf16_rounding_matches_torch_and_definition():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.standard_normal(10000) * 10.0 ** rng.integers(-20, 20, 10000),
                        [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 0.0, -0.0]])
    ours = O.to_bf16(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
    # ties to even at 1 + 2^-8 (down to 1) and 1 + 3*2^-8 (up to 1 + 2^-6)
    assert ours[-5] == 1.0 and ours[-4] == 1.0 + 2.0 ** -6


# ---------------------------------------------------------------------------
# Planted mistakes: a pin above must fail for each
# ---------------------------------------------------------------------------
def _mutant_rope_half_split(x, pos, base):
    x = np.asarray(x, float)
    d = x.shape[-1]
    if d == 0:
        return x.copy()
    ang = np.asarray(pos, float)[..., None] * O.rope_inv_freq(d, base)
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x0 * c - x1 * s, x0 * s + x1 * c], axis=-1)


def _mutant_up_project_transposed(c_kv, w_h):
    w = np.asarray(w_h, float)
    return np.asarray(c_kv, float) @ w[:, ::-1].T  # wrong column order of W


def _mutant_window_off_by_one(q_c, q_r, c_kv, k_r, w_uk, w_uv, *, start, scale, base, **kw):
    # (Counting positions from the window start instead of from 0 would not
    # be a mistake: RoPE scores depend only on q_pos - k_pos.)
    c_kv, k_r = np.asarray(c_kv, float), np.asarray(k_r, float)
    L = c_kv.shape[0]
    return O.explicit_decode(q_c, q_r, c_kv[start + 1:], k_r[start + 1:], w_uk, w_uv, scale=scale, base=base,
                             q_pos=L - 1, k_pos=np.arange(start + 1, L), **kw)


def _mutant_slot_of_swapped(block_table_row, j, block_size):
    # page and offset exchanged: the offset scaled, the page added
    return (j % block_size) * block_size + int(block_table_row[j // block_size])


def _mutant_gather_pages_logical(pool, block_table_row, L):
    pool = np.asarray(pool)
    bs = pool.shape[1]
    idx = np.arange(L)
    return pool[idx // bs, idx % bs]          # block table ignored


def _mutant_project_split_swapped(h, w_dkv, w_kr, w_q, n_heads, d_head, d_rope):
    h = np.asarray(h, float)
    c_kv = h @ np.asarray(w_dkv, float).T
    k_r_raw = h @ np.asarray(w_kr, float).T if d_rope else np.zeros((h.shape[0], 0))
    q = (np.asarray(w_q, float) @ h[-1]).reshape(n_heads, d_head + d_rope)
    return c_kv, k_r_raw, q[:, d_rope:].copy(), q[:, :d_rope].copy()   # RoPE part taken first


def _mutant_project_kr_first_token(h, w_dkv, w_kr, w_q, n_heads, d_head, d_rope):
    h = np.asarray(h, float)
    c_kv = h @ np.asarray(w_dkv, float).T
    k_r_raw = np.repeat(h[:1] @ np.asarray(w_kr, float).T, h.shape[0], axis=0)   # every row from token 0
    q = (np.asarray(w_q, float) @ h[-1]).reshape(n_heads, d_head + d_rope)
    return c_kv, k_r_raw, q[:, :d_head].copy(), q[:, d_head:].copy()


@pytest.mark.parametrize("name,mutant", [("rope", _mutant_rope_half_split),
                                         ("up_project", _mutant_up_project_transposed),
                                         ("window_decode", _mutant_window_off_by_one),
                                         ("slot_of", _mutant_slot_of_swapped),
                                         ("gather_pages", _mutant_gather_pages_logical),
                                         ("project", _mutant_project_split_swapped),
                                         ("project", _mutant_project_kr_first_token)])
def test_pins_catch_planted_mistakes(monkeypatch, name, mutant):
    monkeypatch.setattr(O, name, mutant)
    with pytest.raises(AssertionError):
        if name == "window_decode":
            test_window_matches_brute_force(3)
        elif name == "rope":
            test_rope_closed_forms()
            test_brute_force_matches_oracle(2, 3, 4, 4, 6)
        elif name == "slot_of":
            test_slot_of_hand_computed_table()
        elif name == "gather_pages":
            test_gather_pages_hand_computed_rows()
        elif name == "project":
            test_project_unit_hidden_states_pick_weight_columns()
        else:
            test_worked_example_projection()
