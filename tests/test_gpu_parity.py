"""GPU parity: every call of the decode chain against the float64 oracle on
identical seeded inputs, through the C ABI.  Tolerances: max|gpu - ref| <=
tol * max|ref| with tol = 1e-5 (fp32), 1e-2 (bf16), 3e-2 (e4m3 cache, against
the oracle on its own dequantised rows); lse uses tol * max(1, |lse|)."""
import numpy as np
import pytest
import torch

import mla_inputs as W
from oracle import mla_oracle as O

import chain as C

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check_all(w, res, heads=None, seqs=None, tol=None):
    tol = tol or C.TOL[w.kv if w.kv == "e4m3" else w.act]
    seqs = range(w.B) if seqs is None else seqs
    # absorb_q
    q_ref = O.absorb_q(w.q_c, w.q_r, w.w_uk, w.q_pos, w.rope_base)
    assert C.rel_err(C.f64(res["q_abs"]), q_ref) <= C.TOL[w.act]
    for b in seqs:
        ref = C.oracle_decode(w, b, heads=heads)
        hs = ref["heads"]
        assert C.rel_err(C.f64(res["out"][b, hs]), ref["out"]) <= tol, f"out b={b}"
        assert C.rel_err(C.f64(res["o_lat"][b, hs]), ref["o_lat"]) <= tol, f"o_lat b={b}"
        assert C.lse_err(C.f64(res["lse"][b, hs]), ref["lse"]) <= tol, f"lse b={b}"


def test_tiny_fp32_chain():
    w = C.tiny_inputs(W.make("tiny_f32"))
    res = C.run_chain(w)
    _check_all(w, res)
    rows = C.gather_rows(w, res, 0)["stored"]
    assert C.rel_err(rows, C.oracle_rows(w, 0)["stored"]) <= 1e-6


@pytest.mark.parametrize("splits", [0, 1, 2, 5])
def test_tiny_fp32_splits(splits):
    w = C.tiny_inputs(W.make("tiny_f32"))
    res = C.run_chain(w, num_splits=splits)
    _check_all(w, res)


def test_bf16_cache_rows_are_rounded_rows():
    w = W.make("v2_b16_4k", B=3, lens=[1, 130, 257])
    res = C.run_chain(w)
    for b in range(w.B):
        got = C.gather_rows(w, res, b)["stored"]
        exp = C.oracle_rows(w, b)["stored"]
        assert np.array_equal(got[:, :w.d_c], exp[:, :w.d_c])           # latent copied exactly
        ulp = np.abs(got[:, w.d_c:] - exp[:, w.d_c:]) / np.maximum(np.abs(exp[:, w.d_c:]), 1e-30)
        assert (ulp <= 2.0 ** -8).all()                                  # RoPE part: <= 1 bf16 ulp


@pytest.mark.parametrize("lens,splits", [([1, 130, 257], 0), ([64, 65, 63], 3), ([300], 64),
                                         ([700, 1, 129, 64], 7)])
def test_bf16_v2_shapes(lens, splits):
    w = W.make("v2_b16_4k", B=len(lens), lens=lens)
    res = C.run_chain(w, num_splits=splits)
    _check_all(w, res)


@pytest.mark.parametrize("splits", [200, 640])
def test_bf16_more_parts_than_cus_and_pages(splits):
    """More parts than CUs (several workgroup waves) and than pages (empty
    parts inside a sequence's range, which the merge must skip)."""
    w = W.make("v2_b16_4k", B=5, lens=[4096, 1, 700, 3000, 64], shuffle=True)
    res = C.run_chain(w, num_splits=splits)
    _check_all(w, res)


def test_empty_sequence_in_batch():
    w = W.make("v2_b16_4k", B=3, lens=[70, 0, 5])
    res = C.run_chain(w, num_splits=4)
    o = C.f64(res["o_lat"][1])
    assert np.all(o == 0) and np.all(C.f64(res["out"][1]) == 0)
    assert np.all(np.isneginf(C.f64(res["lse"][1])))
    _check_all(w, res, seqs=[0, 2])


@pytest.mark.parametrize("splits", [1, 2, 8, 32, 64])
def test_ragged_shuffled_pages_any_split(splits):
    w = W.make("ragged_b64", B=4, lens=[1000, 65, 333, 1024], n_h=128)
    res = C.run_chain(w, num_splits=splits)
    _check_all(w, res, heads=[0, 1, 63, 127])


@pytest.mark.parametrize("name", ["ragged_b64", "v2_b16_4k_e4m3"])
def test_merge_every_batch_width(name):
    """One page per part (num_splits = total pages), so each sequence has as
    many parts as pages: 1 (written whole), 2 (merged two at a time), 3 and
    4 (four at a time, one dead slot for 3), 7 and 17 (eight at a time, 17
    over three batches with dead slots), on the 64-head bf16 and E4M3 merges."""
    pages = [1, 2, 3, 4, 7, 17]
    lens = [64 * p - (13 if p > 1 else 0) for p in pages]      # ragged last pages
    w = W.make(name, B=len(lens), lens=lens, n_h=128, shuffle=True)
    assert int(w.num_pages) == sum(pages)
    res = C.run_chain(w, num_splits=sum(pages))
    _check_all(w, res, heads=[0, 31, 64, 127])


def test_page_permutation_is_bitwise_invariant():
    import copy
    a = W.make("ragged_b64", B=3, lens=[200, 450, 130], shuffle=False)
    b = copy.copy(a)
    perm = np.random.default_rng(11).permutation(a.num_pages).astype(np.int32)
    b.block_table = np.where(a.block_table >= 0, perm[np.maximum(a.block_table, 0)], -1).astype(np.int32)
    assert not np.array_equal(a.block_table, b.block_table)
    ra, rb = C.run_chain(a, num_splits=4), C.run_chain(b, num_splits=4)
    for k in ("o_lat", "lse", "out"):
        assert torch.equal(ra[k], rb[k]), k


@pytest.mark.parametrize("name,n_h", [("ragged_b64", None), ("v2_b16_4k_e4m3", 128), ("fp8_h16_b128", None)])
def test_run_to_run_deterministic(name, n_h):
    w = W.make(name, B=2, lens=[900, 77], n_h=n_h)
    r1 = C.run_chain(w, num_splits=6)
    r2 = C.run_chain(w, num_splits=6)
    for k in ("o_lat", "lse", "out", "q_abs"):
        assert torch.equal(r1[k], r2[k]), k


def test_fp8_cache_bytes_match_oracle_quantiser():
    w = W.make("fp8_h16_b128", B=3, lens=[513, 64, 1000])
    res = C.run_chain(w)
    for b in range(w.B):
        got, exp = C.gather_rows(w, res, b), C.oracle_rows(w, b)
        mism = (got["codes"] != exp["codes"])
        assert mism.mean() <= 1e-6, f"b={b}: {mism.sum()} codes differ"
        assert np.all(np.abs(got["scales"] - exp["scales"]) <= 2.0 ** -23 * np.abs(exp["scales"]))


@pytest.mark.parametrize("lens,splits", [([513, 64, 1000], 0), ([4096, 1, 700], 9)])
def test_fp8_chain(lens, splits):
    w = W.make("fp8_h16_b128", B=len(lens), lens=lens)
    res = C.run_chain(w, num_splits=splits)
    _check_all(w, res)


@pytest.mark.parametrize("n_h,lens,splits", [(128, [513, 64, 1000], 0), (64, [4096, 1, 700], 9),
                                             (128, [130, 4000, 63, 700], 150)])
def test_fp8_64_head_groups(n_h, lens, splits):
    """The E4M3 cache at head counts that are multiples of 64: the 64-head
    kernel (codes converted to bf16 in LDS, per-token scales on the scores and
    on P), with ragged last pages, a one-row sequence and more parts than
    pages."""
    w = W.make("v2_b16_4k_e4m3", B=len(lens), lens=lens, n_h=n_h, shuffle=True)
    res = C.run_chain(w, num_splits=splits)
    _check_all(w, res)


@pytest.mark.parametrize("name", ["v2_b16_4k", "v2_b16_4k_e4m3"])
@pytest.mark.parametrize("n_h,splits", [(192, 0), (256, 11)])
def test_64_head_kernel_three_and_four_head_groups(name, n_h, splits):
    """Head counts of 3 and 4 x 64: the parts then carry 3 or 4 workgroups
    each, on both caches; ragged lengths, automatic and forced splits."""
    w = W.make(name, B=3, lens=[300, 1, 777], n_h=n_h, shuffle=True)
    res = C.run_chain(w, num_splits=splits)
    _check_all(w, res, heads=[0, 63, 64, n_h - 1])


def test_fp8_64_head_long_sequence_many_parts():
    """One 8192-token E4M3 sequence (128 pages) cut into 96 parts, next to a
    short one: most parts hold a page or two of the long sequence."""
    w = W.make("v2_b16_4k_e4m3", B=2, lens=[8192, 70], n_h=64, shuffle=True)
    res = C.run_chain(w, num_splits=96)
    _check_all(w, res, heads=[0, 31, 32, 63])


@pytest.mark.parametrize("name", ["v2_b16_4k", "v2_b16_4k_e4m3"])
@pytest.mark.parametrize("splits", [0, 7])
def test_score_jumps_on_later_pages(name, splits):
    """Rows of later pages scaled by 4 (exact in bf16): their scores exceed
    the running maximum by far more than the lazy-rescale threshold, so the
    accumulators must be rescaled mid-segment; E4M3 also gets rows that are
    all zero (scale 0) and rows 64 times smaller than the rest (row scales
    then span 256x).  Rows much larger than the rest are not used: with
    scores in the hundreds the bf16 rounding of q_abs alone moves o_lat by
    several percent (8 % for rows x64 here, float64 oracle on both sides),
    outside what the tolerance is derived for."""
    w = W.make(name, B=2, lens=[1000, 640], n_h=64, shuffle=True)
    for b, (lo, hi) in enumerate([(600, 700), (500, 640)]):
        w.c_kv[b][lo:hi] *= 4.0
        w.k_r[b][lo:hi] *= 4.0
    if w.kv == "e4m3":
        w.c_kv[0][100:130] = 0.0
        w.k_r[0][100:130] = 0.0
        w.c_kv[1][10:12] *= 1.0 / 64.0
        w.k_r[1][10:12] *= 1.0 / 64.0
    res = C.run_chain(w, num_splits=splits)
    _check_all(w, res)


def test_fp8_64_head_page_permutation_is_bitwise_invariant():
    import copy
    a = W.make("v2_b16_4k_e4m3", B=2, lens=[700, 300], n_h=64, shuffle=False)
    b = copy.copy(a)
    perm = np.random.default_rng(12).permutation(a.num_pages).astype(np.int32)
    b.block_table = np.where(a.block_table >= 0, perm[np.maximum(a.block_table, 0)], -1).astype(np.int32)
    assert not np.array_equal(a.block_table, b.block_table)
    ra, rb = C.run_chain(a, num_splits=5), C.run_chain(b, num_splits=5)
    for k in ("o_lat", "lse", "out"):
        assert torch.equal(ra[k], rb[k]), k


@pytest.mark.parametrize("splits", [40, 150])
def test_generic_merge_few_and_many_parts(splits):
    """The generic kernel's merge (16 heads, bf16 cache) with a sequence
    spread over fewer than 64 parts (one part per lane) and over more (the
    general loop, with empty parts inside the range)."""
    w = W.make("v2_b16_4k", B=2, lens=[4096, 700], n_h=16, shuffle=True)
    res = C.run_chain(w, num_splits=splits)
    _check_all(w, res)


@pytest.mark.parametrize("name,n_h,splits", [("v2_b16_4k", 64, 0), ("v2_b16_4k", 64, 37), ("v2_b16_4k", 16, 0),
                                             ("v2_b16_4k_e4m3", 64, 0)])
def test_batch_larger_than_a_workgroup(name, n_h, splits):
    """More sequences than threads in a workgroup (the part locators then sum
    several sequences per thread), with empty and one-token sequences among
    them; a sample of sequences is checked."""
    rng = np.random.default_rng(77)
    lens = rng.integers(0, 200, size=300)
    lens[[5, 6, 150]] = 0
    lens[[7, 299]] = 1
    w = W.make(name, B=300, lens=lens, n_h=n_h, shuffle=True)
    res = C.run_chain(w, num_splits=splits)
    seqs = [0, 5, 7, 8, 149, 150, 151, 298, 299]
    for b in seqs:
        if w.lens[b] == 0:
            assert np.all(C.f64(res["o_lat"][b]) == 0) and np.all(np.isneginf(C.f64(res["lse"][b])))
    _check_all(w, res, heads=[0, n_h - 1], seqs=[b for b in seqs if w.lens[b] > 0])
