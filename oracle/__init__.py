"""Float64 CPU oracle of causal scaled dot-product attention (prefill, chunked
prefill against a cache, decode, cache append, the backward pass, rotary
position embedding and key-padding masks).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the package's smoke
check and the benchmark's CPU-baseline leg, never by the GPU library.  It is
plain NumPy, materialises full score matrices, and shares no code with the
HIP path.  Every function is pinned by the CPU tests against values printed on
the source pages, closed forms, brute force and an independent library routine.
"""

from .attention import (
    allowed_mask,
    append_ref,
    attention_ref,
    attention_rows_ref,
    backward_ref,
    backward_rows_ref,
    chunk_ref,
    decode_ref,
    head_attention,
    kv_head_of,
    softmax_rows,
    softmax_vjp,
)
from .rope import append_rope_ref, rope_angles, rope_ref, rope_table_ref

__all__ = [
    "allowed_mask",
    "append_ref",
    "append_rope_ref",
    "attention_ref",
    "attention_rows_ref",
    "backward_ref",
    "backward_rows_ref",
    "chunk_ref",
    "decode_ref",
    "head_attention",
    "kv_head_of",
    "rope_angles",
    "rope_ref",
    "rope_table_ref",
    "softmax_rows",
    "softmax_vjp",
]
