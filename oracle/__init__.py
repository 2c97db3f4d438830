"""fp64 CPU oracle (test infrastructure only; never imported by the product path)."""

from .attention import (  # noqa: F401
    causal_attention,
    causal_attention_backward,
    causal_attention_bruteforce,
    causal_attention_range,
    causal_flops,
    kv_head_of,
    merge_partials,
    softmax_scale,
    unmasked_pairs,
    visible,
    zigzag_positions,
)
from . import ulysses  # noqa: F401,E402
from . import tsp_layer  # noqa: F401,E402
