"""CPU oracle for the DSA layer (test infrastructure only).

Only the tests, the smoke check and the bench's CPU-baseline leg may import this package.
The product path never does; it shares no code with the HIP library.  See dsa_oracle.cpp
for what each function computes and which passage of the pages it follows.
"""

from .oracle import (  # noqa: F401
    build,
    decode_bf16,
    decode_e4m3,
    index_scores,
    library_path,
    pool_keys,
    round_bf16,
    sparse_attn_bwd,
    sparse_attn_fwd,
    topk,
    visible,
)
