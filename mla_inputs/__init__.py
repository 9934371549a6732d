"""Seeded synthetic inputs for MLA decode workloads.

This module only draws random numbers, rounds them to storage types and lays
out page tables.  It holds none of the attention arithmetic: the float64
oracle (``oracle/``) and the HIP library (``mla_latent_kv_38_amd``) both
receive what it produces, and neither imports the other.

Recipe (every workload):
* ``numpy.random.default_rng(seed)`` (PCG64) and float64 ``standard_normal``.
* The workload-level stream draws, in this order: the cache lengths (when they
  are random), the physical page permutation (when pages are shuffled), then
  W_UK and W_UV, each N(0,1)/sqrt(d_c), shaped [n_h, d_h, d_c].
* Sequence b has its own stream ``default_rng([seed, b])`` drawing c_KV
  [L_b, d_c], k_R [L_b, d_R] (not rotated), q_C [n_h, d_h], q_R [n_h, d_R],
  all N(0,1).
* Values are rounded float64 -> float32 -> bfloat16 (each nearest-even) when
  the activation type is bf16, float64 -> float32 when it is f32.
* The tiny workload draws h [L, d_model] ~ N(0,1), then W_DKV, W_UK, W_UV,
  W_KR, W_Q, each N(0,1)/sqrt(fan_in); its projections are computed by whoever
  consumes it.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# name -> workload description (shapes and value recipe); sizes follow the
# DeepSeek-V2 configuration table (n_h = 128, d_h = 128, d_c = 512, d_R = 64).
WORKLOADS = {
    "tiny_f32": dict(kind="tiny", B=1, n_h=4, d_h=16, d_c=32, d_R=16, d_model=64,
                     lens=("const", 64), act="f32", kv="f32", shuffle=False),
    "v2_b16_4k": dict(kind="latent", B=16, n_h=128, d_h=128, d_c=512, d_R=64,
                      lens=("const", 4096), act="bf16", kv="bf16", shuffle=False),
    "ragged_b64": dict(kind="latent", B=64, n_h=128, d_h=128, d_c=512, d_R=64,
                       lens=("uniform", 1024, 8192), act="bf16", kv="bf16", shuffle=True),
    "long_b4_128k": dict(kind="latent", B=4, n_h=128, d_h=128, d_c=512, d_R=64,
                         lens=("const", 131072), act="bf16", kv="bf16", shuffle=False),
    "fp8_h16_b128": dict(kind="latent", B=128, n_h=16, d_h=128, d_c=512, d_R=64,
                         lens=("uniform", 512, 4096), act="bf16", kv="e4m3", shuffle=True),
    # the headline shapes with an E4M3 cache (all 128 heads on one GPU)
    "v2_b16_4k_e4m3": dict(kind="latent", B=16, n_h=128, d_h=128, d_c=512, d_R=64,
                           lens=("const", 4096), act="bf16", kv="e4m3", shuffle=False),
}

BLOCK_SIZE = 64
ROPE_BASE = 10000.0


def round_to(x, dtype: str) -> np.ndarray:
    """Round float64 values to a storage type; returns float32 holding them.

    'f32': nearest-even float32.  'bf16': nearest-even float32, then
    nearest-even bfloat16 (add 0x7FFF plus the kept LSB, truncate).
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return f
    if dtype != "bf16":
        raise ValueError(dtype)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    n_h: int
    d_h: int
    d_c: int
    d_R: int
    act: str
    kv: str
    block_size: int
    rope_base: float
    scale: float
    lens: np.ndarray            # [B] int32
    block_table: np.ndarray     # [B, max_pages] int32, -1 past the end
    num_pages: int
    w_uk: np.ndarray            # [n_h, d_h, d_c] float32 (rounded)
    w_uv: np.ndarray            # [n_h, d_h, d_c]
    q_c: np.ndarray             # [B, n_h, d_h]
    q_r: np.ndarray             # [B, n_h, d_R] (not rotated)
    c_kv: list                  # per sequence [L_b, d_c]
    k_r: list                   # per sequence [L_b, d_R] (not rotated)
    raw: dict | None = None     # tiny workload: h and the projection matrices

    @property
    def D(self) -> int:
        return self.d_c + self.d_R

    @property
    def max_pages(self) -> int:
        return self.block_table.shape[1]

    @property
    def q_pos(self) -> np.ndarray:
        """Position of each sequence's query token: its last cached token."""
        return (self.lens - 1).astype(np.int32)

    def slots(self, b: int, j0: int = 0, j1: int | None = None) -> np.ndarray:
        """Physical slots (page * block_size + offset) of tokens j0..j1 of b."""
        j1 = int(self.lens[b]) if j1 is None else j1
        j = np.arange(j0, j1)
        return (self.block_table[b, j // self.block_size].astype(np.int64)
                * self.block_size + j % self.block_size)

    def total_tokens(self) -> int:
        return int(self.lens.sum())


def _page_table(lens, block_size, shuffle, rng):
    pages_per = [(int(L) + block_size - 1) // block_size for L in lens]
    max_pages = max(1, max(pages_per) if len(pages_per) else 1)
    total = int(sum(pages_per))
    bt = np.full((len(lens), max_pages), -1, dtype=np.int32)
    phys = rng.permutation(total) if shuffle else np.arange(total)
    k = 0
    for b, n in enumerate(pages_per):
        bt[b, :n] = phys[k:k + n]
        k += n
    return bt, max(total, 1)


def make(name: str, seed: int = 0, B: int | None = None, lens=None,
         n_h: int | None = None, shuffle: bool | None = None) -> Workload:
    """Build a workload by name; B, lens, n_h and shuffle may be overridden
    (smaller cases of the same recipe for tests)."""
    cfg = dict(WORKLOADS[name])
    if B is not None:
        cfg["B"] = B
    if n_h is not None:
        cfg["n_h"] = n_h
    if shuffle is not None:
        cfg["shuffle"] = shuffle
    act = cfg["act"]
    rng = np.random.default_rng(seed)
    Bn, nh, dh, dc, dR = cfg["B"], cfg["n_h"], cfg["d_h"], cfg["d_c"], cfg["d_R"]
    scale = 1.0 / math.sqrt(dh + dR)

    if cfg["kind"] == "tiny":
        L = cfg["lens"][1] if lens is None else int(np.asarray(lens).reshape(-1)[0])
        dm = cfg["d_model"]
        h = rng.standard_normal((L, dm))
        w_dkv = rng.standard_normal((dc, dm)) / math.sqrt(dm)
        w_uk = rng.standard_normal((nh, dh, dc)) / math.sqrt(dc)
        w_uv = rng.standard_normal((nh, dh, dc)) / math.sqrt(dc)
        w_kr = rng.standard_normal((dR, dm)) / math.sqrt(dm)
        w_q = rng.standard_normal((nh * (dh + dR), dm)) / math.sqrt(dm)
        lens_arr = np.array([L], dtype=np.int32)
        bt, npages = _page_table(lens_arr, BLOCK_SIZE, False, rng)
        raw = dict(h=h, w_dkv=w_dkv, w_uk=w_uk, w_uv=w_uv, w_kr=w_kr, w_q=w_q)
        # The projected inputs are filled in by the consumer (they need the
        # down-projection, which is method arithmetic).
        return Workload(name, 1, nh, dh, dc, dR, act, cfg["kv"], BLOCK_SIZE, ROPE_BASE,
                        scale, lens_arr, bt, npages, round_to(w_uk, act),
                        round_to(w_uv, act), None, None, None, None, raw)

    if lens is not None:
        lens_arr = np.asarray(lens, dtype=np.int32).reshape(-1)
        Bn = len(lens_arr)
    elif cfg["lens"][0] == "const":
        lens_arr = np.full(Bn, cfg["lens"][1], dtype=np.int32)
    else:
        lo, hi = cfg["lens"][1], cfg["lens"][2]
        lens_arr = rng.integers(lo, hi + 1, size=Bn).astype(np.int32)
    bt, npages = _page_table(lens_arr, BLOCK_SIZE, cfg["shuffle"], rng)
    w_uk = round_to(rng.standard_normal((nh, dh, dc)) / math.sqrt(dc), act)
    w_uv = round_to(rng.standard_normal((nh, dh, dc)) / math.sqrt(dc), act)
    q_c = np.empty((Bn, nh, dh), np.float32)
    q_r = np.empty((Bn, nh, dR), np.float32)
    c_kv, k_r = [], []
    for b in range(Bn):
        r = np.random.default_rng([seed, b])
        L = int(lens_arr[b])
        c_kv.append(round_to(r.standard_normal((L, dc)), act))
        k_r.append(round_to(r.standard_normal((L, dR)), act))
        q_c[b] = round_to(r.standard_normal((nh, dh)), act)
        q_r[b] = round_to(r.standard_normal((nh, dR)), act)
    return Workload(name, Bn, nh, dh, dc, dR, act, cfg["kv"], BLOCK_SIZE, ROPE_BASE, scale,
                    lens_arr, bt, npages, w_uk, w_uv, q_c, q_r, c_kv, k_r)
