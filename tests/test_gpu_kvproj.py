"""GPU parity of mla_kv_project_append (down-projection of new tokens fused
with their append) against the float64 oracle's ``projected_rows``.

Source: keybo.xyz page, sections "第一步，训练时" (c_kv = W_DKV x) and "RoPE 为什么
必须解耦" (k_R = RoPE(W_KR x), rotated before caching).

The library sums d_model products in float32 (in slices, then the slices)
and rounds each projection once to the activation type; the oracle rounds the
exact sum.  The two roundings agree except where the float32 sum lands on the
other side of a rounding boundary, which moves a bf16 value by one unit in
the last place, so every element must satisfy |got - ref| <= 2^-7 |ref| plus
a small absolute term (1e-6 max|ref| for the latent; for the RoPE part, where
a one-ulp change of k_R is rotated into both elements of its pair,
2^-7 max|pair| + 1e-6 max|ref|).  E4M3 cache: the stored values (code times
scale) against the oracle quantiser's on its own rows, within one E4M3 step
(2^-3 relative) plus 2^-9 of the row's maximum (subnormal codes).  Cases: the
DeepSeek-V2 shapes with d_model = 5120 on the MFMA path (1, 16 and 33
tokens: one, one and three 16-token blocks), the same shapes through the
general kernel (a hidden-state buffer offset by one element), and a float32
case of other widths."""
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


def _run(T, dm, d_c, d_r, act, kv, seed, offset=False):
    rng = np.random.default_rng(seed)
    h = W.round_to(rng.standard_normal((T, dm)), act)
    w_dkv = W.round_to(rng.standard_normal((d_c, dm)) / np.sqrt(dm), act)
    w_kr = W.round_to(rng.standard_normal((d_r, dm)) / np.sqrt(dm), act)
    pos = rng.integers(0, 1 << 16, size=T).astype(np.int32)
    bs = 64
    pages = (T + bs - 1) // bs + 2
    slots = rng.permutation(pages * bs)[:T].astype(np.int64)
    d = mla.make_dims(16, 128, d_c, d_r, bs, act=act, kv=kv, softmax_scale=0.1, rope_base=10000.0)
    tdt = torch.bfloat16 if act == "bf16" else torch.float32
    if kv == "e4m3":
        cache = torch.zeros((pages, bs, d_c + d_r), dtype=torch.uint8, device="cuda")
        scale = torch.zeros((pages, bs), dtype=torch.float32, device="cuda")
    else:
        cache = torch.zeros((pages, bs, d_c + d_r), dtype=tdt, device="cuda")
        scale = None
    mla.kv_project_append(d, _dev(h, tdt, offset), _dev(w_dkv, tdt), _dev(w_kr, tdt), _dev(pos, torch.int32),
                          _dev(slots, torch.int64), cache, scale)
    torch.cuda.synchronize()
    idx = torch.from_numpy(slots).cuda()
    flat = cache.view(-1, d_c + d_r)[idx]
    ref = O.projected_rows(h, w_dkv, w_kr, pos, 10000.0, act)
    if kv == "e4m3":
        codes, s = E.quantize_rows(O.to_f32(ref))
        want = E.dequantize_rows(codes, s)
        got = E.dequantize_rows(flat.cpu().numpy(), scale.view(-1)[idx].cpu().numpy())
        return got, want, d_c, True
    stored = O.to_bf16(ref) if (kv == "bf16") else O.to_f32(ref)
    return flat.double().cpu().numpy(), stored.astype(np.float64), d_c, False


def _check(got, ref, d_c, e4m3):
    if e4m3:
        amax = np.abs(ref).max(axis=1, keepdims=True)
        bad = np.abs(got - ref) > 2.0 ** -3 * np.abs(ref) + 2.0 ** -9 * amax
        assert not bad.any(), f"{bad.sum()} values outside one E4M3 step"
        return
    big = np.abs(ref).max()
    lat = np.abs(got[:, :d_c] - ref[:, :d_c]) > 2.0 ** -7 * np.abs(ref[:, :d_c]) + 1e-6 * big
    assert not lat.any(), f"{lat.sum()} latent values off by more than one bf16 ulp"
    r = ref[:, d_c:].reshape(ref.shape[0], -1, 2)
    pair = np.repeat(np.abs(r).max(axis=2), 2, axis=1)
    rot = np.abs(got[:, d_c:] - ref[:, d_c:]) > 2.0 ** -7 * pair + 1e-6 * big
    assert not rot.any(), f"{rot.sum()} RoPE values outside the bound"


@pytest.mark.parametrize("T", [1, 16, 33])
@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
def test_v2_rows_mfma(T, kv):
    _check(*_run(T, 5120, 512, 64, "bf16", kv, seed=T))


@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
def test_v2_rows_general_kernel(kv):
    _check(*_run(17, 5120, 512, 64, "bf16", kv, seed=40, offset=True))


def test_f32_other_widths():
    _check(*_run(5, 96, 32, 16, "f32", "f32", seed=41))
