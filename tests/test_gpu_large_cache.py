"""Cache pools larger than 4 GiB: pages whose byte offset does not fit in 32
bits.  Every odd physical page of the workload moves past the 4 GiB mark,
so each sequence reads pages from both ends of the pool; the append writes
the rows there through 64-bit slots and each decode kernel (the 64-head
bf16 and E4M3 kernels, the 16-head E4M3 kernel and the general float32
kernel) reads them back.  Outputs are compared with the oracle's
latent-space decode (keybo.xyz page, section "第二步，推理时的吸收") on the
rows as stored, to the tolerances of the small cases; the rows of the moved
pages are compared with the oracle's rows (latent bits exact for bf16,
codes equal for E4M3)."""
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


_ELEM = {"f32": 4, "bf16": 2, "e4m3": 1}


def _move_odd_pages_past_4gib(w):
    page_bytes = w.block_size * w.D * _ELEM[w.kv]
    off = (2 ** 32 + page_bytes - 1) // page_bytes + 1000
    bt = w.block_table.copy()
    odd = (bt >= 0) & (bt % 2 == 1)
    bt[odd] += off
    w.block_table = bt
    w.num_pages = int(w.num_pages + off)
    assert w.num_pages * page_bytes > 2 ** 32 and (bt[odd].astype(np.int64) * page_bytes >= 2 ** 32).all()
    return w


def _workload(case):
    if case == "bf16_64_heads":
        return W.make("v2_b16_4k", B=3, lens=[1000, 4096, 300], shuffle=True)
    if case == "e4m3_64_heads":
        return W.make("v2_b16_4k_e4m3", B=3, lens=[1000, 4096, 300], shuffle=True)
    if case == "e4m3_16_heads":
        return W.make("fp8_h16_b128", B=4)
    w = W.make("v2_b16_4k", B=2, lens=[700, 1500], n_h=8, shuffle=True)
    w.act = w.kv = "f32"                       # the inputs are bf16 values, exact in float32
    return w


@pytest.mark.parametrize("case", ["bf16_64_heads", "e4m3_64_heads", "e4m3_16_heads", "f32_general"])
def test_pages_past_4_gib(case):
    w = _move_odd_pages_past_4gib(_workload(case))
    print(f"[large cache] {case}: B={w.B} n_h={w.n_h} kv={w.kv} num_pages={w.num_pages}", flush=True)
    res = C.run_chain(w)
    try:
        tol = C.TOL["e4m3" if w.kv == "e4m3" else w.act]
        q_ref = O.absorb_q(w.q_c, w.q_r, w.w_uk, w.q_pos, w.rope_base)
        o_all, l_all = C.f64(res["o_lat"]), C.f64(res["lse"])
        for b in range(w.B):
            exp = C.oracle_rows(w, b)
            ref = O.latent_decode(q_ref[b], exp["stored"], w.d_c, w.scale)
            assert C.rel_err(o_all[b], ref["o_lat"]) <= tol, f"o_lat b={b}"
            assert C.lse_err(l_all[b], ref["lse"]) <= tol, f"lse b={b}"

            # the rows, gathered on the device so that only they are copied back
            L = int(w.lens[b])
            j = np.arange(L)
            pages = torch.from_numpy(w.block_table[b, j // w.block_size].astype(np.int64)).cuda()
            offs = torch.from_numpy((j % w.block_size).astype(np.int64)).cuda()
            got = res["cache"][pages, offs].cpu()
            if w.kv == "e4m3":
                mism = got.numpy() != exp["codes"]
                assert mism.mean() <= 1e-6, f"b={b}: {mism.sum()} codes differ"
            else:
                g = got.to(torch.float64).numpy()
                assert np.array_equal(g[:, :w.d_c], exp["stored"][:, :w.d_c]), f"latent b={b}"
    finally:
        del res
        torch.cuda.empty_cache()
