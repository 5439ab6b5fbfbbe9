"""Plain fp64 CPU oracle of the DSA layer hot path. TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this
package. The HIP library and its binding never import, call or link it, and it shares no
code, table or constant generator with them.
"""
from . import compare  # noqa: F401
from .dsa_oracle import (  # noqa: F401
    bf16_to_f64, FP8_E4M3FN, ue8m0_to_f64, slots_of, key_rows, kv_rows,
    index_scores_row, topk_row, attention_row, layer_row, order_key,
    attention_math, attention_backward_math, attention_backward_row,
)
