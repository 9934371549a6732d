"""GPU parity of the two projections around latent attention, element by
element against the float64 oracle on the same bf16 inputs:

  absorb_q   q_abs = [W_UK^T q_C || RoPE(q_R)]     (keybo.xyz page, sections "第二步，推理时的吸收"
                                                    and "RoPE 为什么必须解耦"; dgblog.top page,
                                                    section "3. 一个聪明的优化")
  up_v       out   = W_UV o_lat                     (keybo.xyz page, "第二步，推理时的吸收":
                                                    one W_UV after the latent sum)

A bf16 output is the exact value rounded once, after float32 accumulation of
d_h (or d_c) products, so every element must satisfy
    |got - ref| <= 2^-8 |ref| + 2^-14 max|ref|
(one bf16 rounding, relative 2^-9, with a factor of two of slack, plus the
accumulation term: float32 partial sums of at most 512 terms stay within
512 * 2^-24 of the row scale).  Both the MFMA kernels (aligned buffers) and
the generic kernels (buffers offset by one element, which the library routes
to the generic path) are checked, at batch sizes that leave ragged 16-row
blocks."""
import numpy as np
import pytest
import torch

import mla_inputs as W
import mla_latent_kv_38_amd as mla
from oracle import mla_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _dev(a, dtype=torch.bfloat16, offset=False):
    """Device copy; with offset the data starts one element into its buffer
    (2-byte aligned only)."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if not offset:
        return t.to("cuda").to(dtype)
    flat = torch.empty(t.numel() + 1, dtype=dtype, device="cuda")
    view = flat[1:].view(t.shape)
    view.copy_(t.to(dtype).to("cuda"))
    return view


def _elementwise_ok(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -14 * np.abs(ref).max()
    bad = np.abs(got - ref) > bound
    return int(bad.sum()), float((np.abs(got - ref) / np.maximum(bound, 1e-300)).max())


def _f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


CASES = [(128, 1), (128, 16), (128, 17), (128, 40), (128, 100), (16, 128), (16, 33), (16, 300)]


@pytest.mark.parametrize("n_h,B", CASES)
@pytest.mark.parametrize("offset", [False, True], ids=["mfma", "generic"])
def test_absorb_q_elementwise(n_h, B, offset):
    w = W.make("v2_b16_4k", seed=3, B=B, lens=[1] * B, n_h=n_h)
    d = mla.make_dims(w.n_h, w.d_h, w.d_c, w.d_R, w.block_size, act="bf16", kv="bf16",
                      softmax_scale=w.scale, rope_base=w.rope_base)
    pos = np.random.default_rng(B).integers(0, 1 << 17, size=B).astype(np.int32)
    q_abs = torch.empty((B, n_h, w.D + (1 if offset else 0)), dtype=torch.bfloat16, device="cuda")
    q_abs = q_abs.view(-1)[1:1 + B * n_h * w.D].view(B, n_h, w.D) if offset else q_abs
    mla.absorb_q(d, _dev(w.q_c, offset=offset), _dev(w.q_r, offset=offset), _dev(pos, torch.int32),
                 _dev(w.w_uk, offset=offset), q_abs)
    torch.cuda.synchronize()
    ref = O.absorb_q(w.q_c, w.q_r, w.w_uk, pos, w.rope_base)
    nbad, worst = _elementwise_ok(_f64(q_abs), ref)
    assert nbad == 0, f"{nbad} elements outside the bound (worst ratio {worst:.2f})"


@pytest.mark.parametrize("n_h,B", CASES)
@pytest.mark.parametrize("offset", [False, True], ids=["mfma", "generic"])
def test_up_v_elementwise(n_h, B, offset):
    w = W.make("v2_b16_4k", seed=4, B=B, lens=[1] * B, n_h=n_h)
    d = mla.make_dims(w.n_h, w.d_h, w.d_c, w.d_R, w.block_size, act="bf16", kv="bf16",
                      softmax_scale=w.scale, rope_base=w.rope_base)
    o_lat = W.round_to(np.random.default_rng(B + 7).standard_normal((B, n_h, w.d_c)), "bf16")
    out = mla.up_v(d, _dev(o_lat, offset=offset), _dev(w.w_uv, offset=offset))
    torch.cuda.synchronize()
    ref = O.up_v(o_lat, w.w_uv)
    nbad, worst = _elementwise_ok(_f64(out), ref)
    assert nbad == 0, f"{nbad} elements outside the bound (worst ratio {worst:.2f})"

