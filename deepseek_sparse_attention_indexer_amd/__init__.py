"""MI355X (gfx950) DeepSeek Sparse Attention layer hot path.

Thin Python binding over the C ABI of ``libdsa.so`` (declared in include/dsa.h): the
functions below carry the C entry points' names and only marshal torch tensors (device
memory, current HIP stream) into pointers and sizes. Every step of the layer runs in the
library's HIP kernels; there is no Python or CPU fallback, and importing this package
without the built library raises.
"""
from ._binding import (  # noqa: F401
    DSAError, KeyCache, KVCache, Rows, lib_path,
    dsa_index_scores, dsa_topk, dsa_sparse_mla_decode, dsa_sparse_mla_prefill, dsa_decode,
    dsa_decode_static, STATIC_SCRATCH_BYTES, DSA_ERR_SCRATCH_LIMIT,
    dsa_sparse_mla_backward,
    dsa_workspace_size, dsa_workspace_init, dsa_status_string, dsa_abi_version,
    dsa_profile_enable, dsa_profile_collect, dsa_launch_override, dsa_kv_cache_write, dsa_key_cache_write,
    Workspace, ENTRY_TOPK, ENTRY_MLA_DECODE, ENTRY_MLA_PREFILL, ENTRY_DECODE, ENTRY_MLA_BACKWARD,
)
