"""mla_decode_noalloc (the decode whose split-KV partials live in the
library's built-in device scratch) against mla_decode_window with a caller
workspace, through the C ABI, on two calls in a row, the second with a
smaller batch; plus the oracle on sampled heads (bf16 tolerance 1e-2, E4M3
3e-2 on the oracle's dequantised rows)."""
import numpy as np
import pytest
import torch

import mla_inputs as W
import mla_latent_kv_38_amd as mla

import chain as C

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(kind, lens, seed, starts=None):
    w = W.make(kind, B=len(lens), lens=lens, shuffle=True, seed=seed)
    res = C.run_chain(w)                       # fills the cache; decode with a workspace
    d = C.dims_of(w)
    at = C._DT[w.act]
    q_abs = res["q_abs"]
    bt = C.to_dev(w.block_table, torch.int32)
    sl = C.to_dev(w.lens, torch.int32)
    st = None if starts is None else C.to_dev(np.asarray(starts, np.int32), torch.int32)
    return w, d, at, res, q_abs, bt, sl, st


def _compare(w, d, res, q_abs, bt, sl, st, splits):
    ref_o, ref_l = mla.decode(d, q_abs, res["cache"], bt, sl, kv_scale=res["scale"], num_splits=splits,
                              seq_starts=st)
    got_o = torch.full_like(ref_o, float("nan"))
    got_l = torch.full_like(ref_l, float("nan"))
    mla.decode_noalloc(d, q_abs, res["cache"], bt, sl, kv_scale=res["scale"], num_splits=splits,
                       o_lat=got_o, lse=got_l, seq_starts=st)
    torch.cuda.synchronize()
    # the same kernels on the same inputs: identical bits
    assert torch.equal(got_o.view(torch.int16), ref_o.view(torch.int16))
    assert torch.equal(got_l.view(torch.int32), ref_l.view(torch.int32))
    if st is None:                              # and the oracle on sampled heads
        tol = C.TOL[w.kv if w.kv == "e4m3" else w.act]
        heads = [0, 63, 64, 127]
        for b in range(w.B):
            ref = C.oracle_decode(w, b, heads=heads)
            assert C.rel_err(C.f64(got_o[b, heads]), ref["o_lat"]) <= tol, f"o_lat b={b}"
            assert C.lse_err(C.f64(got_l[b, heads]), ref["lse"]) <= tol, f"lse b={b}"


@pytest.mark.parametrize("kind", ["v2_b16_4k", "v2_b16_4k_e4m3"])
def test_noalloc_matches_workspace_decode_twice_second_smaller(kind):
    big = _case(kind, [3000, 1, 700, 4096, 130, 0, 2048], seed=3)
    w, d, at, res, q_abs, bt, sl, st = big
    _compare(w, d, res, q_abs, bt, sl, st, splits=0)
    small = _case(kind, [257, 64], seed=4)
    w, d, at, res, q_abs, bt, sl, st = small
    _compare(w, d, res, q_abs, bt, sl, st, splits=0)


def test_noalloc_windows_and_explicit_splits():
    w, d, at, res, q_abs, bt, sl, st = _case("v2_b16_4k", [900, 4096, 65], seed=5, starts=[100, 4000, 64])
    _compare(w, d, res, q_abs, bt, sl, st, splits=37)
    w, d, at, res, q_abs, bt, sl, _ = _case("v2_b16_4k", [129], seed=6)
    _compare(w, d, res, q_abs, bt, sl, None, splits=1)


def test_noalloc_generic_kernel_fp32():
    w = C.tiny_inputs(W.make("tiny_f32"))
    res = C.run_chain(w)
    d = C.dims_of(w)
    bt = C.to_dev(w.block_table, torch.int32)
    sl = C.to_dev(w.lens, torch.int32)
    ref_o, ref_l = mla.decode(d, res["q_abs"], res["cache"], bt, sl, num_splits=3)
    got_o, got_l = mla.decode_noalloc(d, res["q_abs"], res["cache"], bt, sl, num_splits=3)
    torch.cuda.synchronize()
    assert torch.equal(got_o, ref_o) and torch.equal(got_l, ref_l)
