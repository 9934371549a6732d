"""GPU parity of mla_cache_append on DeepSeek-V2 rows (d_c = 512, d_R = 64,
bf16 activations), for a bf16 and an E4M3 cache.

The library writes such rows with a vectorised kernel when every buffer is
16-byte aligned and with the per-element kernel otherwise; both compute the
same float32 values (latent copied, RoPE of the page's rotation rule in
float64 rounded once, per-row scale amax / 448), so the two must leave
identical bytes in the cache.  Against the float64 oracle: latent bits exact,
RoPE within one bf16 ulp, E4M3 codes equal except where the scaled value
sits on a rounding tie that float32 and float64 resolve differently."""
import numpy as np
import pytest
import torch

import mla_inputs as W
import mla_latent_kv_38_amd as mla
from oracle import e4m3 as E
from oracle import mla_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _dev(a, dtype, offset=False):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(dtype)
    if not offset:
        return t.to("cuda")
    flat = torch.empty(t.numel() + 1, dtype=dtype, device="cuda")
    view = flat[1:].view(t.shape)
    view.copy_(t.to("cuda"))
    return view


def _append(kv, T, seed, offset):
    rng = np.random.default_rng(seed)
    d_c, d_R, bs = 512, 64, 64
    c_kv = W.round_to(rng.standard_normal((T, d_c)) * 0.7, "bf16")
    k_r = W.round_to(rng.standard_normal((T, d_R)) * 1.3, "bf16")
    pos = rng.integers(0, 1 << 17, size=T).astype(np.int32)
    pages = max(1, (T + bs - 1) // bs + 2)
    slots = rng.permutation(pages * bs)[:T].astype(np.int64)
    d = mla.make_dims(16, 128, d_c, d_R, bs, act="bf16", kv=kv, softmax_scale=192 ** -0.5, rope_base=10000.0)
    if kv == "e4m3":
        cache = torch.zeros((pages, bs, d_c + d_R), dtype=torch.uint8, device="cuda")
        scale = torch.zeros((pages, bs), dtype=torch.float32, device="cuda")
    else:
        cache = torch.zeros((pages, bs, d_c + d_R), dtype=torch.bfloat16, device="cuda")
        scale = None
    mla.cache_append(d, _dev(c_kv, torch.bfloat16, offset), _dev(k_r, torch.bfloat16, offset),
                     _dev(pos, torch.int32), _dev(slots, torch.int64), cache, scale)
    torch.cuda.synchronize()
    return dict(c_kv=c_kv, k_r=k_r, pos=pos, slots=slots, cache=cache, scale=scale)


@pytest.mark.parametrize("T", [1, 16, 333])
@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
def test_vector_and_generic_append_write_identical_bytes(kv, T):
    a = _append(kv, T, seed=T, offset=False)
    b = _append(kv, T, seed=T, offset=True)
    assert torch.equal(a["cache"].view(torch.uint8), b["cache"].view(torch.uint8))
    if kv == "e4m3":
        assert torch.equal(a["scale"], b["scale"])


@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
def test_vector_append_matches_oracle(kv):
    r = _append(kv, 333, seed=5, offset=False)
    rows = O.cache_rows(r["c_kv"], r["k_r"], r["pos"], 10000.0)
    flat = r["cache"].view(-1, 576)[torch.from_numpy(r["slots"]).cuda()]
    if kv == "bf16":
        got = flat.float().cpu().numpy().astype(np.float64)
        exp = O.to_bf16(rows).astype(np.float64)
        assert np.array_equal(got[:, :512], exp[:, :512])
        ulp = np.abs(got[:, 512:] - exp[:, 512:]) / np.maximum(np.abs(exp[:, 512:]), 1e-30)
        assert (ulp <= 2.0 ** -8).all()
    else:
        codes, s = E.quantize_rows(O.to_f32(rows))
        got = flat.cpu().numpy()
        gs = r["scale"].view(-1)[torch.from_numpy(r["slots"]).cuda()].cpu().numpy()
        assert (got != codes).mean() <= 1e-5
        assert np.all(np.abs(gs - s) <= 2.0 ** -23 * np.abs(s))


@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
@pytest.mark.parametrize("T,misalign", [(0, False), (16, False), (37, False), (16, True)])
def test_absorb_q_append_equals_the_two_calls(kv, T, misalign):
    """mla_absorb_q_append (one launch when the shapes allow; the two launches
    otherwise, here forced by a misaligned latent buffer) leaves the same bytes
    in q_abs and in the cache as mla_absorb_q followed by mla_cache_append."""
    w = W.make("v2_b16_4k", B=16, lens=[1] * 16, seed=8)
    rng = np.random.default_rng(T + 3)
    d = mla.make_dims(w.n_h, w.d_h, w.d_c, w.d_R, w.block_size, act="bf16", kv=kv,
                      softmax_scale=w.scale, rope_base=w.rope_base)
    c = W.round_to(rng.standard_normal((max(T, 1), 512)), "bf16")[:T]
    k = W.round_to(rng.standard_normal((max(T, 1), 64)), "bf16")[:T]
    pos = rng.integers(0, 1 << 16, size=T).astype(np.int32)
    pages = 3
    slots = rng.permutation(pages * 64)[:T].astype(np.int64)
    qpos = rng.integers(0, 1 << 16, size=16).astype(np.int32)
    args_q = (_dev(w.q_c, torch.bfloat16), _dev(w.q_r, torch.bfloat16), _dev(qpos, torch.int32),
              _dev(w.w_uk, torch.bfloat16))
    args_a = (_dev(c, torch.bfloat16, misalign), _dev(k, torch.bfloat16), _dev(pos, torch.int32),
              _dev(slots, torch.int64))

    def cache():
        if kv == "e4m3":
            return (torch.zeros((pages, 64, 576), dtype=torch.uint8, device="cuda"),
                    torch.zeros((pages, 64), dtype=torch.float32, device="cuda"))
        return torch.zeros((pages, 64, 576), dtype=torch.bfloat16, device="cuda"), None

    c1, s1 = cache()
    q1 = mla.absorb_q(d, *args_q)
    if T:
        mla.cache_append(d, *args_a, c1, s1)
    c2, s2 = cache()
    q2 = mla.absorb_q_append(d, *args_q, *args_a, c2, s2)
    torch.cuda.synchronize()
    assert torch.equal(q1.view(torch.int16), q2.view(torch.int16))
    assert torch.equal(c1.view(torch.uint8), c2.view(torch.uint8))
    if kv == "e4m3":
        assert torch.equal(s1, s2)
