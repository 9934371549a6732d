"""GPU parity of decode over a window of each sequence's rows
(mla_decode_window) and over block tables whose sequences share prefix
pages, against the float64 oracle on the same seeded inputs.

Source: keybo.xyz page, section "所以 cache 逻辑到底哪里要重写": requests that
share a prefix share its latent pages, and eviction such as a sliding window
works as before.

Each window test makes every read the kernels must not weigh visible: the
rows of a window's first page that lie before the window are never written
(they hold NaN, or E4M3 NaN codes and NaN scales), and the block-table entries
of pages wholly before the window name a page nobody writes (NaN again).  Any
weight on them turns the output into NaN.  The windows cover a start of 0, a
start inside a page, a start one row before a page boundary, a start on a
boundary, a one-row window and an empty one.  Tolerances as in the other
parity tests (1e-2 of max|ref| for bf16, 3e-2 for the E4M3 cache)."""
import numpy as np
import pytest
import torch

import mla_inputs as W
import mla_latent_kv_38_amd as mla
from oracle import e4m3 as E
from oracle import mla_oracle as O

import chain as C

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _window_run(w, starts, num_splits=0, misalign_out=False):
    """Append only the rows inside each window, decode with seq_starts and
    up-project; returns the GPU results (o_lat, lse, out)."""
    d = C.dims_of(w)
    bs = w.block_size
    poison = w.num_pages                                   # an extra page nobody writes
    shape = (w.num_pages + 1, bs, w.D)
    if w.kv == "e4m3":
        cache = torch.full(shape, 0x7F, dtype=torch.uint8, device="cuda")
        scale = torch.full(shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    else:
        cache = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        scale = None
    bt = w.block_table.copy()
    cs, ks, ps, ss = [], [], [], []
    for b in range(w.B):
        st, L = int(starts[b]), int(w.lens[b])
        if st < L:
            cs.append(w.c_kv[b][st:]); ks.append(w.k_r[b][st:])
            ps.append(np.arange(st, L, dtype=np.int32)); ss.append(w.slots(b)[st:])
        bt[b, :min(st, L) // bs] = poison
    at = torch.bfloat16
    if cs:
        mla.cache_append(d, C.to_dev(np.concatenate(cs), at), C.to_dev(np.concatenate(ks), at),
                         C.to_dev(np.concatenate(ps), torch.int32), C.to_dev(np.concatenate(ss), torch.int64),
                         cache, scale)
    q_abs = mla.absorb_q(d, C.to_dev(w.q_c, at), C.to_dev(w.q_r, at), C.to_dev(w.q_pos, torch.int32),
                         C.to_dev(w.w_uk, at))
    o_lat = None
    if misalign_out:                                       # a 2-byte offset routes to the generic kernel
        o_lat = torch.empty(w.B * w.n_h * w.d_c + 1, dtype=at, device="cuda")[1:].view(w.B, w.n_h, w.d_c)
    o_lat, lse = mla.decode(d, q_abs, cache, C.to_dev(bt, torch.int32), C.to_dev(w.lens, torch.int32),
                            kv_scale=scale, num_splits=num_splits, o_lat=o_lat,
                            seq_starts=C.to_dev(np.asarray(starts, np.int32), torch.int32))
    out = mla.up_v(d, o_lat.contiguous(), C.to_dev(w.w_uv, at))
    torch.cuda.synchronize()
    return dict(o_lat=o_lat, lse=lse, out=out)


def _window_ref(w, b, start, heads=None):
    kw = dict(start=start, scale=w.scale, base=w.rope_base, heads=heads)
    if w.kv == "e4m3":
        rows = C.oracle_rows(w, b)["stored"]
        return O.window_decode(w.q_c[b], w.q_r[b], rows[:, :w.d_c], rows[:, w.d_c:], w.w_uk, w.w_uv,
                               k_r_rotated=True, **kw)
    return O.window_decode(w.q_c[b], w.q_r[b], w.c_kv[b], w.k_r[b], w.w_uk, w.w_uv, **kw)


def _check(w, res, starts, heads=None):
    tol = C.TOL[w.kv if w.kv == "e4m3" else w.act]
    for b in range(w.B):
        ref = _window_ref(w, b, starts[b], heads)
        hs = ref["heads"]
        if starts[b] >= w.lens[b]:                         # empty window
            assert np.all(C.f64(res["o_lat"][b]) == 0) and np.all(np.isneginf(C.f64(res["lse"][b])))
            continue
        assert C.rel_err(C.f64(res["out"][b, hs]), ref["out"]) <= tol, f"out b={b}"
        assert C.rel_err(C.f64(res["o_lat"][b, hs]), ref["o_lat"]) <= tol, f"o_lat b={b}"
        assert C.lse_err(C.f64(res["lse"][b, hs]), ref["lse"]) <= tol, f"lse b={b}"


LENS = [700, 130, 300, 64, 129, 1000]
STARTS = [0, 65, 299, 63, 128, 1000]        # from 0; inside a page; one row; row 63; a boundary; empty


@pytest.mark.parametrize("splits", [0, 3, 40])
def test_window_bf16_mfma(splits):
    w = W.make("v2_b16_4k", B=len(LENS), lens=LENS, shuffle=True)
    res = _window_run(w, STARTS, splits)
    _check(w, res, STARTS)


@pytest.mark.parametrize("splits", [0, 7])
def test_window_bf16_generic(splits):
    w = W.make("v2_b16_4k", B=len(LENS), lens=LENS, n_h=16, shuffle=True)
    res = _window_run(w, STARTS, splits, misalign_out=True)
    _check(w, res, STARTS)


@pytest.mark.parametrize("splits", [0, 9])
def test_window_fp8(splits):
    lens = [513, 64, 1000, 300]
    starts = [200, 0, 640, 299]
    w = W.make("fp8_h16_b128", B=len(lens), lens=lens)
    res = _window_run(w, starts, splits)
    _check(w, res, starts)


@pytest.mark.parametrize("splits", [0, 7])
def test_window_fp8_64_heads(splits):
    w = W.make("v2_b16_4k_e4m3", B=len(LENS), lens=LENS, n_h=64, shuffle=True)
    res = _window_run(w, STARTS, splits)
    _check(w, res, STARTS)


def test_window_all_starts_zero_equals_plain_decode():
    w = W.make("ragged_b64", B=3, lens=[200, 450, 130])
    plain = C.run_chain(w, num_splits=4)
    d = C.dims_of(w)
    o, l = mla.decode(d, plain["q_abs"], plain["cache"], C.to_dev(w.block_table, torch.int32),
                      C.to_dev(w.lens, torch.int32), num_splits=4,
                      seq_starts=torch.zeros(w.B, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(o, plain["o_lat"]) and torch.equal(l, plain["lse"])


@pytest.mark.parametrize("splits", [0, 5])
def test_shared_prefix_pages(splits):
    """Sequences 1 and 2 reuse sequence 0's first 6 and 3 pages (same latent
    rows, same positions); only their own suffixes are appended."""
    w = W.make("v2_b16_4k", B=3, lens=[700, 584, 292], shuffle=True)
    shared = [0, 6, 3]
    for b in (1, 2):
        n = shared[b] * w.block_size
        w.c_kv[b][:n] = w.c_kv[0][:n]
        w.k_r[b][:n] = w.k_r[0][:n]
        w.block_table[b, :shared[b]] = w.block_table[0, :shared[b]]
    d = C.dims_of(w)
    cache, scale = C.new_cache(w)
    cs, ks, ps, ss = [], [], [], []
    for b in range(w.B):
        j0 = shared[b] * w.block_size
        cs.append(w.c_kv[b][j0:]); ks.append(w.k_r[b][j0:])
        ps.append(np.arange(j0, w.lens[b], dtype=np.int32)); ss.append(w.slots(b)[j0:])
    at = torch.bfloat16
    mla.cache_append(d, C.to_dev(np.concatenate(cs), at), C.to_dev(np.concatenate(ks), at),
                     C.to_dev(np.concatenate(ps), torch.int32), C.to_dev(np.concatenate(ss), torch.int64),
                     cache, scale)
    res = C.run_chain(w, num_splits=splits, cache=(cache, scale), append=False)
    for b in range(w.B):
        ref = C.oracle_decode(w, b)
        assert C.rel_err(C.f64(res["out"][b]), ref["out"]) <= C.TOL["bf16"], f"out b={b}"
        assert C.rel_err(C.f64(res["o_lat"][b]), ref["o_lat"]) <= C.TOL["bf16"], f"o_lat b={b}"
        assert C.lse_err(C.f64(res["lse"][b]), ref["lse"]) <= C.TOL["bf16"], f"lse b={b}"
