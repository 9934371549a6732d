"""GPU parity at the full workload sizes, in the launch configuration that
bench.py times (automatic split count, every call on the whole batch).

The oracle cannot run every (sequence, head) of these workloads in a test, so
it checks sampled outputs it computes one by one: chosen sequences (first,
last and, for ragged batches, one in the middle) and heads, for out, o_lat
and lse, with the same tolerances as the small cases
(max|gpu - ref| <= tol * max|ref| over the sampled rows; tol = 1e-2 for bf16,
3e-2 for the E4M3 cache against the oracle on its own dequantised rows).
Cache rows of the sampled sequences are checked too: latent bits exact and
the RoPE part within one bf16 ulp (bf16 cache), codes and scales equal to the
oracle quantiser's up to a last-bit RoPE difference (E4M3 cache).  q_abs is
checked on the whole batch."""
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


CASES = {
    "v2_b16_4k": dict(seqs=[0, 15], heads=[0, 65, 127]),
    "ragged_b64": dict(seqs=[0, 37, 63], heads=[1, 100]),
    "long_b4_128k": dict(seqs=[0, 3], heads=[0, 77]),
    "fp8_h16_b128": dict(seqs=[0, 64, 127], heads=[0, 9, 15]),
    "v2_b16_4k_e4m3": dict(seqs=[0, 15], heads=[0, 64, 127]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_full_size_sampled(name):
    w = W.make(name)
    print(f"[fullsize] {name}: B={w.B} n_h={w.n_h} tokens={w.total_tokens()} kv={w.kv}", flush=True)
    res = C.run_chain(w)
    tol = C.TOL["e4m3" if w.kv == "e4m3" else w.act]

    q_ref = O.absorb_q(w.q_c, w.q_r, w.w_uk, w.q_pos, w.rope_base)
    assert C.rel_err(C.f64(res["q_abs"]), q_ref) <= C.TOL[w.act]

    heads = CASES[name]["heads"]
    for b in CASES[name]["seqs"]:
        ref = C.oracle_decode(w, b, heads=heads)
        assert C.rel_err(C.f64(res["out"][b, heads]), ref["out"]) <= tol, f"out b={b}"
        assert C.rel_err(C.f64(res["o_lat"][b, heads]), ref["o_lat"]) <= tol, f"o_lat b={b}"
        assert C.lse_err(C.f64(res["lse"][b, heads]), ref["lse"]) <= tol, f"lse b={b}"

        got = C.gather_rows(w, res, b)
        exp = C.oracle_rows(w, b)
        if w.kv == "e4m3":
            # the rotated row is float64 RoPE rounded to float32 on both sides; a
            # last-bit difference in a device cosine may move one code, never more
            mism = got["codes"] != exp["codes"]
            assert mism.mean() <= 1e-6, f"b={b}: {mism.sum()} codes differ"
            assert np.all(np.abs(got["scales"] - exp["scales"]) <= 2.0 ** -23 * np.abs(exp["scales"]))
        else:
            g, e = got["stored"], exp["stored"]
            assert np.array_equal(g[:, :w.d_c], e[:, :w.d_c]), f"latent b={b}"
            ulp = np.abs(g[:, w.d_c:] - e[:, w.d_c:]) / np.maximum(np.abs(e[:, w.d_c:]), 1e-30)
            assert (ulp <= 2.0 ** -8).all(), f"rope b={b}"
