"""CPU fp64 oracle for partial causal GQA attention and its LSE merge.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports, links or calls this
package; only the test suite, the smoke check and the CPU-baseline leg of the
benchmark do. It shares no code with the HIP path.
"""
from .cpattn_oracle import (  # noqa: F401
    zigzag_chunk_sizes,
    zigzag_partition,
    rr_rank,
    rr_local_index,
    rr_global_index,
    rr_local_len,
    rr_placement,
    attend,
    full_causal_attn,
    partial_attn,
    lse_merge,
    visible_pairs,
    choose_pass,
    pass_cost,
)
