"""CPU oracle for the KPool-DSA sparse-attention layer (GLM-5.3-Flash).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything here.  The product path (the HIP library and its Python binding) never
does, and this package shares no code with it: plain numpy, float64, one step at a time, no blocking, fusion or
reordering beyond what the definitions state.

Parity pins (see ``tests/test_oracle_pins.py``): every function below is checked against brute force, closed
forms, limits, invariants or a library routine that does not share this code.  Readings of points the pages
leave open are listed with each function.
"""
from .kpool_dsa import (  # noqa: F401
    bf16_round,
    store_round,
    fp8_e4m3_decode,
    pool_compress,
    pool_mean,
    pool_geometry,
    indexer_scores,
    select_pools,
    attended_tokens,
    shared_attended_tokens,
    sparse_mla,
    LayerOracle,
)
from .projections import (  # noqa: F401
    linear,
    indexer_project,
    mla_absorb_q,
    mla_unabsorb_o,
)
