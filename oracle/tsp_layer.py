"""Plain CPU oracle of one rank's TSP attention layer forward.

TEST INFRASTRUCTURE ONLY: used by tests/, never by the product path; shares no code with
the HIP library.

"Folding Tensor and Sequence Parallelism for Memory-Efficient Transformer Training &
Inference", section 2 (Methodology), attention layers: each rank holds 1/D of the tokens
(the zigzag chunks) and 1/D of the weights; the ranks iterate over the packed W_Q, W_K,
W_V, W_O shards, each broadcast by its owner; every rank projects its own tokens with the
shard, the K/V of all ranks are gathered along the sequence, attention runs on the local
queries, and the output projection is accumulated. The result for the rank's tokens is
the standard causal multi-head (grouped-query) attention layer:
    y = Attention(x W_Q^T, K, V) W_O^T,
where K, V hold every token's projections at its global position (the rank's own rows
x W_K^T, x W_V^T; the other rows those of the other ranks).

Readings: weights in the [out_features, in_features] layout;
w_qkv stacks the rows of W_Q (query heads in order), W_K and W_V; shard i holds query
heads i*Hq/D .. and KV heads i*Hkv/D .. (whole heads per shard, so Hq and Hkv divide by
D); no bias; the attention is this package's oracle attention (zigzag positions, GQA,
scale 1/sqrt(dh)).
"""

from __future__ import annotations

import numpy as np

from .attention import _as_f64, causal_attention, zigzag_positions


def attention_layer(x_local, w_qkv, w_o, k_gathered, v_gathered, D: int, rank: int, Hq: int, Hkv: int, dh: int):
    """Returns (y_local [B, 2C, d_model], K, V) in float64; K, V are the gathered buffers
    with the rank's rows replaced by its own projections."""
    x = _as_f64(x_local)
    W = _as_f64(w_qkv)
    Wo = _as_f64(w_o)
    B, S_local, d_model = x.shape
    K = _as_f64(k_gathered).copy()
    V = _as_f64(v_gathered).copy()
    S_total = K.shape[1]
    q = (x @ W[:Hq * dh].T).reshape(B, S_local, Hq, dh)
    k_loc = (x @ W[Hq * dh:(Hq + Hkv) * dh].T).reshape(B, S_local, Hkv, dh)
    v_loc = (x @ W[(Hq + Hkv) * dh:].T).reshape(B, S_local, Hkv, dh)
    pos = zigzag_positions(S_total, D, rank)
    K[:, pos] = k_loc
    V[:, pos] = v_loc
    o, _ = causal_attention(q, K, V, D, rank)
    y = o.reshape(B, S_local, Hq * dh) @ Wo.T
    return y, K, V
