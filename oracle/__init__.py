"""Float64 CPU oracle of the DSA hot path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It is independent of the HIP library.
"""
from .dsa_oracle import (  # noqa: F401
    append_rows,
    attention_row,
    attention_target,
    decode_bf16,
    decode_e4m3fn,
    dsa_row,
    encode_bf16,
    encode_e4m3fn,
    indexer_backward,
    indexer_kl,
    indexer_row,
    indexer_scores,
    mha_attention,
    mha_decompress,
    paged_append,
    paged_view,
    pow2_scale,
    project,
    project_tokens,
    quantize_e4m3fn,
    select_topk,
    sparse_attention,
)
