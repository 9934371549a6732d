"""MI355X (gfx950) absorbed-MLA decode over a paged latent KV cache.

The library is the C ABI in include/mla.h (built into libmla_gfx950.so);
``ops`` binds it for torch tensors with the same call names.
"""
from .ops import (absorb_q, absorb_q_append, cache_append, decode, decode_multi, decode_noalloc, decode_workspace_bytes,  # noqa: F401
                  kv_project_append,
                  kv_project_workspace_bytes, make_dims, up_v)
from ._lib import MLAError, Dims  # noqa: F401
