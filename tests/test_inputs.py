"""Host-side checks of the seeded input recipe (no attention arithmetic)."""
import numpy as np

import mla_inputs as W
from oracle import mla_oracle as O


def test_rounding_agrees_with_oracle_rounding():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000) * 10.0 ** rng.integers(-10, 10, 100000)
    assert np.array_equal(W.round_to(x, "bf16").view(np.uint32), O.to_bf16(x).view(np.uint32))
    assert np.array_equal(W.round_to(x, "f32"), O.to_f32(x))


def test_workloads_are_seeded_and_shaped():
    a = W.make("ragged_b64", B=5, n_h=16)
    b = W.make("ragged_b64", B=5, n_h=16)
    assert np.array_equal(a.lens, b.lens) and np.array_equal(a.block_table, b.block_table)
    assert all(np.array_equal(x, y) for x, y in zip(a.c_kv, b.c_kv))
    assert a.lens.min() >= 1024 and a.lens.max() <= 8192
    pages = [a.block_table[i, : (a.lens[i] + 63) // 64] for i in range(5)]
    allp = np.concatenate(pages)
    assert sorted(allp.tolist()) == list(range(a.num_pages))        # a permutation
    assert a.c_kv[2].shape == (a.lens[2], 512) and a.q_c.shape == (5, 16, 128)
    # bf16 values round-trip exactly through bf16
    assert np.array_equal(W.round_to(a.c_kv[0], "bf16"), a.c_kv[0])
    s = a.slots(1)
    assert len(np.unique(s)) == a.lens[1]


def test_v2_shapes_and_cache_bytes():
    """576 cached values per token per layer at DeepSeek-V2 shapes (1152 B in bf16)."""
    w = W.make("v2_b16_4k", B=2, lens=[130, 64])
    assert w.D == 576 and w.D * 2 == 1152
    assert w.block_table[0, :3].tolist() == [0, 1, 2] and w.block_table[1, 0] == 3
    assert abs(w.scale - 1 / np.sqrt(192)) < 1e-15
