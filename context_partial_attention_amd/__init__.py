"""Partial causal GQA attention and exact LSE merge for context parallelism,
on AMD MI355X (gfx950).

This package is a thin ctypes binding over libcpattn.so (C ABI declared in
include/cpattn.h). Every step of the computation runs in the library's HIP
kernels or host C++; Python only passes pointers, sizes and the current torch
stream, and allocates outputs with torch when the caller gives none. If the
library is not built, every call raises.
"""
from .binding import (  # noqa: F401
    BF16,
    F32,
    MASK_CAUSAL,
    MASK_NONE,
    CpaError,
    choose_pass,
    cp_partition,
    library_path,
    load_library,
    lse_merge,
    partial_attn,
    partial_attn_accumulate,
    partial_attn_merged,
    partial_attn_multi,
    partial_attn_multi_noalloc,
    partial_attn_multi_workspace,
    partial_attn_paged,
    partial_attn_paged_merged,
    partial_attn_paged_workspace,
    pass_cost,
    rr_placement,
)
