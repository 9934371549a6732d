"""Host-only checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects invalid requests before touching the GPU (all
pointers below are fake; validation fails before any HIP call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

L = pytest.importorskip("mla_latent_kv_38_amd._lib")


def _lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("library not built")
    return L.lib()


def _header_functions():
    inc = os.path.join(ROOT, "include")
    src = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = _lib()
    names = _header_functions()
    assert set(names) == set(L.SIGNATURES), names
    for n in names:
        assert hasattr(lib, n), n


def test_dims_struct_layout():
    assert ctypes.sizeof(L.Dims) == 40
    assert L.Dims.rope_base.offset == 32


def _dims(**kw):
    d = dict(n_heads=128, d_head=128, d_latent=512, d_rope=64, block_size=64,
             act_dtype=L.MLA_BF16, kv_dtype=L.MLA_BF16, softmax_scale=1 / 192 ** 0.5, rope_base=1e4)
    d.update(kw)
    return L.Dims(**d)


FAKE = ctypes.c_void_p(0x1000)
NULL = ctypes.c_void_p(0)


def test_status_strings_and_version():
    lib = _lib()
    assert lib.mla_status_string(0) == b"ok"
    assert lib.mla_status_string(-4).startswith(b"workspace")
    assert lib.mla_abi_version() == 1
    assert lib.mla_last_hip_error() == 0


def test_validation_errors_launch_nothing():
    lib = _lib()
    d = _dims()
    ref = ctypes.byref
    # absorb_q
    assert lib.mla_absorb_q(None, 1, FAKE, FAKE, FAKE, FAKE, FAKE, NULL) == -1
    assert lib.mla_absorb_q(ref(d), 0, FAKE, FAKE, FAKE, FAKE, FAKE, NULL) == -2
    assert lib.mla_absorb_q(ref(d), 4, NULL, FAKE, FAKE, FAKE, FAKE, NULL) == -1
    bad = _dims(d_rope=63)
    assert lib.mla_absorb_q(ref(bad), 4, FAKE, FAKE, FAKE, FAKE, FAKE, NULL) == -2
    bad = _dims(act_dtype=L.MLA_E4M3)
    assert lib.mla_absorb_q(ref(bad), 4, FAKE, FAKE, FAKE, FAKE, FAKE, NULL) == -3
    bad = _dims(kv_dtype=7)
    assert lib.mla_absorb_q(ref(bad), 4, FAKE, FAKE, FAKE, FAKE, FAKE, NULL) == -3
    bad = _dims(d_latent=2048)
    assert lib.mla_absorb_q(ref(bad), 4, FAKE, FAKE, FAKE, FAKE, FAKE, NULL) == -2
    bad = _dims(rope_base=0.0)
    assert lib.mla_absorb_q(ref(bad), 4, FAKE, FAKE, FAKE, FAKE, FAKE, NULL) == -2
    for sc in (0.0, -0.125, float("inf"), float("nan")):       # softmax_scale must be finite and > 0
        bad = _dims(softmax_scale=sc)
        assert lib.mla_absorb_q(ref(bad), 4, FAKE, FAKE, FAKE, FAKE, FAKE, NULL) == -2
        assert lib.mla_decode_workspace_bytes(ref(bad), 16, 0) == 0
        assert lib.mla_decode(ref(bad), 16, FAKE, FAKE, NULL, FAKE, 64, FAKE, 0, ctypes.c_void_p(0x10000),
                              1 << 40, FAKE, NULL, NULL) == -2
    # cache_append
    assert lib.mla_cache_append(ref(d), 0, NULL, NULL, NULL, NULL, 1, NULL, NULL, NULL) == 0  # no-op
    assert lib.mla_cache_append(ref(d), -1, FAKE, FAKE, FAKE, FAKE, 1, FAKE, NULL, NULL) == -2
    assert lib.mla_cache_append(ref(d), 3, FAKE, FAKE, FAKE, FAKE, 0, FAKE, NULL, NULL) == -2
    assert lib.mla_cache_append(ref(d), 3, FAKE, FAKE, FAKE, NULL, 1, FAKE, NULL, NULL) == -1
    d8 = _dims(kv_dtype=L.MLA_E4M3)
    assert lib.mla_cache_append(ref(d8), 3, FAKE, FAKE, FAKE, FAKE, 1, FAKE, NULL, NULL) == -1
    # decode
    need = lib.mla_decode_workspace_bytes(ref(d), 16, 0)
    assert need > 0
    assert lib.mla_decode_workspace_bytes(ref(d), 0, 0) == 0
    assert lib.mla_decode_workspace_bytes(ref(d), 16, -1) == 0
    args = [FAKE, FAKE, NULL, FAKE, 64, FAKE, 0]
    ws = ctypes.c_void_p(0x10000)
    assert lib.mla_decode(ref(d), 16, *args, ws, need - 1, FAKE, NULL, NULL) == -4
    assert lib.mla_decode(ref(d), 16, *args, ctypes.c_void_p(0x10010), need, FAKE, NULL, NULL) == -4
    assert lib.mla_decode(ref(d), 16, *args, NULL, need, FAKE, NULL, NULL) == -1
    assert lib.mla_decode(ref(d), 0, *args, ws, need, FAKE, NULL, NULL) == -2
    assert lib.mla_decode(ref(d8), 16, *args, ws, 1 << 40, FAKE, NULL, NULL) == -1   # no kv_scale
    args_bad_split = [FAKE, FAKE, NULL, FAKE, 64, FAKE, 70000]
    assert lib.mla_decode(ref(d), 16, *args_bad_split, ws, 1 << 40, FAKE, NULL, NULL) == -2
    # decode_window: same validation as decode; seq_starts may be NULL
    assert lib.mla_decode_window(ref(d), 16, FAKE, FAKE, NULL, FAKE, 64, FAKE, FAKE, 0, ws, need - 1,
                                 FAKE, NULL, NULL) == -4
    assert lib.mla_decode_window(ref(d), 16, FAKE, FAKE, NULL, FAKE, 64, NULL, FAKE, 0, ws, need,
                                 FAKE, NULL, NULL) == -1
    assert lib.mla_decode_window(ref(d), 16, FAKE, FAKE, NULL, FAKE, 0, FAKE, NULL, 0, ws, need,
                                 FAKE, NULL, NULL) == -2
    # decode_noalloc: same validation as decode_window; a plan beyond the built-in scratch is refused
    nargs = [FAKE, FAKE, NULL, FAKE, 64, FAKE, NULL, 0]
    assert lib.mla_decode_noalloc(ref(d), 0, *nargs, FAKE, NULL, NULL) == -2
    assert lib.mla_decode_noalloc(ref(d), 16, *nargs, NULL, NULL, NULL) == -1
    assert lib.mla_decode_noalloc(ref(d8), 16, *nargs, FAKE, NULL, NULL) == -1        # no kv_scale
    big = 1
    while lib.mla_decode_workspace_bytes(ref(d), big, 0) <= L.NOALLOC_SCRATCH_BYTES:
        big *= 2
    assert lib.mla_decode_noalloc(ref(d), big, *nargs, FAKE, NULL, NULL) == -4
    assert lib.mla_decode_workspace_bytes(ref(d), 96, 0) <= L.NOALLOC_SCRATCH_BYTES   # the header's stated cover
    # kv_project_append
    pw = lib.mla_kv_project_workspace_bytes(ref(d), 16, 5120)
    assert pw >= 16 * 576 * 4
    assert lib.mla_kv_project_workspace_bytes(ref(d), 16, 0) == 0
    assert lib.mla_kv_project_workspace_bytes(ref(d), -1, 5120) == 0
    pargs = [FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE, NULL]
    assert lib.mla_kv_project_append(ref(d), 0, 5120, *[NULL] * 5, 1, NULL, NULL, NULL, 0, NULL) == 0  # no-op
    assert lib.mla_kv_project_append(ref(d), 16, 5120, *pargs, ws, pw - 1, NULL) == -4
    assert lib.mla_kv_project_append(ref(d), 16, 5120, *pargs, ctypes.c_void_p(0x10010), pw, NULL) == -4
    assert lib.mla_kv_project_append(ref(d), 16, 0, *pargs, ws, pw, NULL) == -2
    assert lib.mla_kv_project_append(ref(d), 16, 5120, FAKE, FAKE, NULL, FAKE, FAKE, 1, FAKE, NULL, ws, pw,
                                     NULL) == -1                                   # no W_KR with d_R > 0
    assert lib.mla_kv_project_append(ref(d8), 16, 5120, *pargs, ws, 1 << 40, NULL) == -1   # no kv_scale
    # up_v
    assert lib.mla_up_v(ref(d), 16, FAKE, NULL, FAKE, NULL) == -1
    assert lib.mla_up_v(ref(d), -3, FAKE, FAKE, FAKE, NULL) == -2
    assert lib.mla_last_hip_error() == 0


def test_workspace_grows_with_splits_and_batch():
    lib = _lib()
    d = _dims()
    ref = ctypes.byref
    a = lib.mla_decode_workspace_bytes(ref(d), 16, 8)
    b = lib.mla_decode_workspace_bytes(ref(d), 16, 64)
    c = lib.mla_decode_workspace_bytes(ref(d), 64, 64)
    assert a < b < c
    # one float32 partial (d_latent values + lse) per head per slot, slots = splits + batch
    assert b >= (64 + 16) * 128 * (512 + 1) * 4


def test_probes_reject_bad_arguments_before_launching():
    lib = _lib()
    assert lib.mla_probe_stream_read(NULL, 1024, FAKE, NULL) == -1
    assert lib.mla_probe_stream_read(FAKE, 1024, NULL, NULL) == -1
    assert lib.mla_probe_stream_read(FAKE, 0, FAKE, NULL) == -2
    assert lib.mla_probe_stream_read(FAKE, 1000, FAKE, NULL) == -2
    assert lib.mla_probe_stream_read(ctypes.c_void_p(0x1008), 1024, FAKE, NULL) == -2
    assert lib.mla_probe_mfma_bf16(100, 256, NULL, NULL) == -1
    assert lib.mla_probe_mfma_bf16(0, 256, FAKE, NULL) == -2
    assert lib.mla_probe_mfma_bf16(100, 0, FAKE, NULL) == -2
