"""Plain CPU oracle for TriAttention's KV-cache compression step (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may
import this package.  The product path (the HIP library and its Python binding) never
imports, links or calls anything here, and nothing here imports the product path.
"""

from .triattention import (  # noqa: F401
    rope_theta,
    rope_apply,
    decode_fp8_e4m3,
    decode_bf16,
    decode_stored,
    split_bands,
    concentration,
    score_keys,
    score_magnitude_bound,
    select_top_b,
    compact_dense,
    compact_paged_sequence,
    calibrate,
    unit_heads,
    decode_attention,
)
