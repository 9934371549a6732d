"""GPU parity of mla_decode_multi (several new query tokens per sequence,
each attending causally over its sequence's rows) against the float64
oracle's ``multi_query_decode`` on the same seeded inputs.

Source: algomooc.com MLA interview page, section "先区分 KV Cache 与 MLA" (new
tokens are appended, then attend over history plus current) and keybo.xyz
page, section "第一步，训练时" (a token attends over the tokens up to itself).

Cases cover the bf16 MFMA kernel (64-head groups), the E4M3 kernel (16-head
groups) and the generic kernel (16 heads, bf16 cache), with 1, 4 and 5
query tokens, a sequence shorter than its query chunk, windows, and several
split counts.  Tolerances as in the other parity tests."""
import numpy as np
import pytest
import torch

import mla_inputs as W
import mla_latent_kv_38_amd as mla
from oracle import mla_oracle as O

import chain as C

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(name, lens, q, n_h=None, seed=0):
    w = W.make(name, B=len(lens), lens=lens, n_h=n_h, seed=seed)
    rng = np.random.default_rng(seed + 1000)
    qc = W.round_to(rng.standard_normal((w.B, q, w.n_h, w.d_h)), w.act)
    qr = W.round_to(rng.standard_normal((w.B, q, w.n_h, w.d_R)), w.act)
    qpos = np.array([[max(int(w.lens[b]) - q + i, 0) for i in range(q)] for b in range(w.B)], np.int32)
    return w, qc, qr, qpos


def _run(w, qc, qr, qpos, q, splits=0, starts=None):
    d = C.dims_of(w)
    at = torch.bfloat16
    cache, scale = C.new_cache(w)
    c_all = np.concatenate([w.c_kv[b] for b in range(w.B)])
    k_all = np.concatenate([w.k_r[b] for b in range(w.B)])
    pos = np.concatenate([np.arange(w.lens[b]) for b in range(w.B)]).astype(np.int32)
    slots = np.concatenate([w.slots(b) for b in range(w.B)])
    mla.cache_append(d, C.to_dev(c_all, at), C.to_dev(k_all, at), C.to_dev(pos, torch.int32),
                     C.to_dev(slots, torch.int64), cache, scale)
    B = w.B
    q_abs = mla.absorb_q(d, C.to_dev(qc.reshape(B * q, w.n_h, w.d_h), at),
                         C.to_dev(qr.reshape(B * q, w.n_h, w.d_R), at), C.to_dev(qpos.reshape(-1), torch.int32),
                         C.to_dev(w.w_uk, at))
    st = None if starts is None else C.to_dev(np.asarray(starts, np.int32), torch.int32)
    o_lat, lse = mla.decode_multi(d, q_abs.view(B, q, w.n_h, w.D), cache, C.to_dev(w.block_table, torch.int32),
                                  C.to_dev(w.lens, torch.int32), kv_scale=scale, num_splits=splits, seq_starts=st)
    out = mla.up_v(d, o_lat.view(B * q, w.n_h, w.d_c), C.to_dev(w.w_uv, at)).view(B, q, w.n_h, w.d_h)
    torch.cuda.synchronize()
    return dict(o_lat=o_lat, lse=lse, out=out)


def _check(w, res, qc, qr, q, starts=None, heads=None):
    tol = C.TOL[w.kv if w.kv == "e4m3" else w.act]
    for b in range(w.B):
        st = 0 if starts is None else int(starts[b])
        if w.kv == "e4m3":
            rows = C.oracle_rows(w, b)["stored"]
            c, k, rot = rows[:, :w.d_c], rows[:, w.d_c:], True
        else:
            c, k, rot = w.c_kv[b], w.k_r[b], False
        ref = O.multi_query_decode(qc[b], qr[b], c, k, w.w_uk, w.w_uv, scale=w.scale, base=w.rope_base,
                                   start=st, k_r_rotated=rot, heads=heads)
        hs = ref["heads"]
        for i in range(q):
            if np.all(np.isneginf(ref["lse"][i])):
                assert np.all(C.f64(res["o_lat"][b, i]) == 0), f"b={b} i={i}"
                assert np.all(np.isneginf(C.f64(res["lse"][b, i]))), f"b={b} i={i}"
                continue
            assert C.rel_err(C.f64(res["out"][b, i, hs]), ref["out"][i]) <= tol, f"out b={b} i={i}"
            assert C.rel_err(C.f64(res["o_lat"][b, i, hs]), ref["o_lat"][i]) <= tol, f"o_lat b={b} i={i}"
            assert C.lse_err(C.f64(res["lse"][b, i, hs]), ref["lse"][i]) <= tol, f"lse b={b} i={i}"


@pytest.mark.parametrize("q,splits", [(1, 0), (4, 0), (4, 7), (5, 64)])
def test_multi_bf16_mfma(q, splits):
    w, qc, qr, qpos = _case("v2_b16_4k", [300, 64, 130, 3], q, seed=q)
    res = _run(w, qc, qr, qpos, q, splits)
    _check(w, res, qc, qr, q, heads=[0, 1, 64, 127])


def test_multi_bf16_mfma_window():
    starts = [100, 0, 129, 1]
    w, qc, qr, qpos = _case("v2_b16_4k", [300, 64, 130, 3], 4, seed=9)
    res = _run(w, qc, qr, qpos, 4, 5, starts)
    _check(w, res, qc, qr, 4, starts, heads=[0, 33, 100])


@pytest.mark.parametrize("q,splits", [(4, 0), (3, 9)])
def test_multi_fp8(q, splits):
    w, qc, qr, qpos = _case("fp8_h16_b128", [513, 64, 700], q, seed=20 + q)
    res = _run(w, qc, qr, qpos, q, splits)
    _check(w, res, qc, qr, q)


def test_multi_fp8_64_heads():
    w, qc, qr, qpos = _case("v2_b16_4k_e4m3", [513, 64, 700], 4, n_h=64, seed=27)
    res = _run(w, qc, qr, qpos, 4, 7)
    _check(w, res, qc, qr, 4)


def test_multi_generic():
    w, qc, qr, qpos = _case("v2_b16_4k", [200, 65], 3, n_h=16, seed=31)
    res = _run(w, qc, qr, qpos, 3, 4)
    _check(w, res, qc, qr, 3)
