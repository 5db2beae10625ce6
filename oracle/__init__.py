"""CPU oracle for the UltraQuant FP4 KV-cache hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library under
``bit_kv_cache_wht_amd/csrc``; both sides implement the cache format from its
written definition.

Everything is plain numpy in float64, written to be checked against the pages
by eye rather than to be fast.  Parity is pinned by ``tests/test_oracle_*.py``;
every function below has at least one pin that does not re-derive it.
"""
from .uq_oracle import *  # noqa: F401,F403
from .uq_oracle import __all__  # noqa: F401
