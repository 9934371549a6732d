"""Float64 CPU oracle for absorbed-weight MLA decode (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The library under
``mla_latent_kv_38_amd`` never imports it and shares no code with it.
"""
from . import mla_oracle, e4m3  # noqa: F401
