"""Seeded synthetic inputs for the DSA layer hot path.

This package only draws tensors, stores them in the cache formats the kernels and the
oracle read (bf16 bit patterns, fp8 e4m3 bytes with their scales, paged tables), and
describes each workload. It holds none of the method's arithmetic: no scoring, no
selection, no attention, no dequantisation. Both the oracle and the HIP path consume it.
"""
from .gen import (  # noqa: F401
    KeyPool, KVPool, DSAProblem,
    tiny_decode, glm_decode, causal_prefill, dsv4_fp8_decode, long_decode,
    attention_case, WORKLOADS, make_workload,
)
