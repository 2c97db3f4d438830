"""Plain CPU fp64 oracle for the causal attention one sequence-parallel rank computes.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or run this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it. It shares no code, table or constant with the HIP library.

What it computes (the plain definition, written out step by step):

* "Folding Tensor and Sequence Parallelism for Memory-Efficient Transformer Training &
  Inference", section 2 (Methodology), attention layers: every rank projects its own
  share of the sequence, an all-gather rebuilds the whole key/value context along the
  sequence, and the rank runs causal attention of its local queries against that full
  context. The local queries are a zigzag share of the sequence, chosen so that causal
  work is balanced across ranks.
* "AutoSP: Unlocking Long-Context LLM Training Via Compiler-Based Sequence
  Parallelism", section 2.A (automated SP pass), index recomputation: the causal mask
  must be recomputed for the distributed layout, so visibility is decided by global
  token positions, not by local row numbers.
* "Tensor, pipeline e sequence parallelism", section 01 (Conceito), grouped-query
  attention paragraph: several query heads share one key/value head (24 query heads
  over 4 KV heads; at degree 4 a rank holding 6 query heads holds exactly 1 KV head),
  and the sequence-parallel paragraph: Ulysses gives each rank full attention over a
  subset of heads, which is the one-rank (D = 1) case here.

Readings taken where the pages are silent:

* zigzag map: the sequence is cut into 2D equal chunks of C = S_total / (2D) tokens and
  rank r holds chunk r followed by chunk 2D-1-r (local rows [0, C) then [C, 2C));
* keys/values are indexed by global position (row j of k_full is token j);
* the causal diagonal is inclusive: key j is visible to a query at position p iff j <= p;
* softmax scale 1/sqrt(dh); query head h uses KV head h // (Hq / Hkv);
* lse is the natural-log log-sum-exp of the scaled scores of visible keys.

Inputs are upcast exactly to float64 (bf16 and fp32 values are exactly representable).

Parity is pinned by the ``-m "not gpu"`` tests in tests/test_oracle_pins.py (brute force,
a library routine for the one-rank case, closed forms, the concatenation identity, the
equal-pair-count identity and the lesson page's GQA head ownership; for the backward,
central finite differences of the forward, PyTorch autograd through its causal SDPA,
the rank-partition identity and closed-form sums); none of the functions below is
"parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np


# --------------------------------------------------------------------------------------
# Step 1 -- the zigzag map from local query row to global position.
# "Folding Tensor and Sequence Parallelism ...", section 2 (Methodology), attention
# layers: zigzag partitioning balances causal attention work across ranks. The page
# gives no formula; the reading used is "2D equal chunks, rank r owns chunks r and
# 2D-1-r, in ascending order".
# --------------------------------------------------------------------------------------
def zigzag_positions(S_total: int, D: int, rank: int) -> np.ndarray:
    """Global token position of every local query row of ``rank`` (int64, length 2C)."""
    if D < 1 or not (0 <= rank < D) or S_total % (2 * D) != 0:
        raise ValueError("need D >= 1, 0 <= rank < D and S_total divisible by 2D")
    C = S_total // (2 * D)
    low_chunk = rank
    high_chunk = 2 * D - 1 - rank
    low = np.arange(low_chunk * C, (low_chunk + 1) * C, dtype=np.int64)
    high = np.arange(high_chunk * C, (high_chunk + 1) * C, dtype=np.int64)
    return np.concatenate([low, high])


# --------------------------------------------------------------------------------------
# Step 2 -- which KV head a query head reads.
# "Tensor, pipeline e sequence parallelism", section 01, GQA paragraph: query heads are
# grouped over the KV heads; a rank holding 6 consecutive query heads of 24 holds one of
# the 4 KV heads, which only contiguous grouping gives.
# --------------------------------------------------------------------------------------
def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (Hq // Hkv)


# --------------------------------------------------------------------------------------
# Step 3 -- causal visibility by global position.
# "AutoSP ...", section 2.A, item 4 (index recomputation): masks are recomputed for the
# distributed layout. Reading: key j is visible to the query at global position p iff
# j <= p (inclusive diagonal, as in causal language-model attention).
# --------------------------------------------------------------------------------------
def visible(key_index: np.ndarray, query_pos: np.ndarray) -> np.ndarray:
    """Boolean mask [len(query_pos), len(key_index)]: True where the key is visible."""
    return key_index[None, :] <= query_pos[:, None]


def softmax_scale(dh: int) -> float:
    return 1.0 / math.sqrt(dh)


def _as_f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch tensor: its stored values, upcast exactly
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------------------
# The attention itself, materialised-scores form.
# "Folding Tensor and Sequence Parallelism ...", section 2, attention layers: local
# queries attend to the gathered full-sequence keys/values. For every (batch, query
# head, local row): scores over the visible keys, max-subtracted exponentials, their
# sum, the weighted mean of the values, and lse = max + ln(sum).
# --------------------------------------------------------------------------------------
def causal_attention(q, k, v, D: int, rank: int, rows=None, heads=None, block: int = 256):
    """Oracle forward for one rank.

    q: [B, S_local, Hq, dh]; k, v: [B, S_total, Hkv, dh] (global position order).
    rows / heads: optional subsets of local rows / query heads to compute.
    Returns (out [B, len(rows), len(heads), dh] float64, lse [B, len(heads), len(rows)]).
    """
    q = _as_f64(q)
    B, S_local, Hq, dh = q.shape
    S_total, Hkv = k.shape[1], k.shape[2]
    pos_all = zigzag_positions(S_total, D, rank)
    if S_local != pos_all.shape[0]:
        raise ValueError("q_local must hold 2 * S_total / (2D) rows")
    rows = np.arange(S_local) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = list(range(Hq)) if heads is None else list(heads)
    scale = softmax_scale(dh)
    out = np.zeros((B, len(rows), len(heads), dh))
    lse = np.zeros((B, len(heads), len(rows)))
    for b in range(B):
        kv_cache = {}
        for hi, h in enumerate(heads):
            hk = kv_head_of(h, Hq, Hkv)
            if hk not in kv_cache:
                kv_cache = {hk: (_as_f64(k[b, :, hk, :]), _as_f64(v[b, :, hk, :]))}
            kb, vb = kv_cache[hk]
            for start in range(0, len(rows), block):
                r = rows[start:start + block]
                p = pos_all[r]
                nkeys = int(p.max()) + 1
                keys = np.arange(nkeys, dtype=np.int64)
                s = scale * (q[b, r, h, :] @ kb[:nkeys].T)
                s = np.where(visible(keys, p), s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                w = np.exp(s - m)
                l = w.sum(axis=1, keepdims=True)
                out[b, start:start + len(r), hi, :] = (w @ vb[:nkeys]) / l
                lse[b, hi, start:start + len(r)] = (m + np.log(l))[:, 0]
    return out, lse


def causal_attention_bruteforce(q, k, v, D: int, rank: int, kv_begin: int = 0, kv_end=None):
    """Same definition as ``causal_attention`` (keys restricted to [kv_begin, kv_end)) as
    plain scalar loops (tiny inputs only). A row without a visible key gets out = 0 and
    lse = -inf."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, S_local, Hq, dh = q.shape
    S_total, Hkv = k.shape[1], k.shape[2]
    pos = zigzag_positions(S_total, D, rank)
    scale = softmax_scale(dh)
    kv_end = S_total if kv_end is None else kv_end
    out = np.zeros((B, S_local, Hq, dh))
    lse = np.full((B, Hq, S_local), -np.inf)
    for b in range(B):
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            for i in range(S_local):
                p = int(pos[i])
                scores = []
                for j in range(kv_begin, kv_end):
                    if visible(np.array([j]), np.array([p]))[0, 0]:
                        dot = 0.0
                        for d in range(dh):
                            dot += q[b, i, h, d] * k[b, j, hk, d]
                        scores.append((j, scale * dot))
                if not scores:
                    continue
                m = max(s for _, s in scores)
                weights = [(j, math.exp(s - m)) for j, s in scores]
                l = sum(w for _, w in weights)
                for d in range(dh):
                    acc = 0.0
                    for j, w in weights:
                        acc += w * v[b, j, hk, d]
                    out[b, i, h, d] = acc / l
                lse[b, h, i] = m + math.log(l)
    return out, lse


# --------------------------------------------------------------------------------------
# Work accounting.
# "Folding Tensor and Sequence Parallelism ...", section 2: the zigzag split exists to
# balance causal work. The count of visible (query, key) pairs of a rank, per (batch,
# query head), is the sum over its local rows of (position + 1).
# --------------------------------------------------------------------------------------
def unmasked_pairs(S_total: int, D: int, rank: int) -> int:
    pos = zigzag_positions(S_total, D, rank)
    return int(np.sum(pos + 1))


def causal_flops(B: int, Hq: int, dh: int, S_total: int, D: int, rank: int) -> int:
    """Algorithmic FLOPs: two products of 2*dh FLOP per visible pair per query head."""
    return 4 * B * Hq * dh * unmasked_pairs(S_total, D, rank)


# --------------------------------------------------------------------------------------
# Attention over a key range, and the merge of partial results.
# "Folding Tensor and Sequence Parallelism ...", section 2 (Methodology): the K/V
# all-gather is overlapped with computation (section 3, item 3: communication hidden
# behind compute). Reading: a rank may attend to each gathered chunk of keys as it
# arrives and combine the partial results. Each partial is the same definition with the
# keys restricted to [kv_begin, kv_end); a row with no visible key in the range has the
# empty sum: out = 0 and lse = -inf. Merging two partials over disjoint key sets is the
# log-sum-exp combination of their softmax denominators, which reproduces the attention
# over the union of the keys exactly.
# --------------------------------------------------------------------------------------
def causal_attention_range(q, k, v, D: int, rank: int, kv_begin: int, kv_end: int, rows=None, block: int = 256):
    """Oracle forward restricted to keys j in [kv_begin, kv_end) (and j <= position)."""
    q = _as_f64(q)
    B, S_local, Hq, dh = q.shape
    S_total, Hkv = k.shape[1], k.shape[2]
    if not (0 <= kv_begin <= kv_end <= S_total):
        raise ValueError("need 0 <= kv_begin <= kv_end <= S_total")
    pos_all = zigzag_positions(S_total, D, rank)
    rows = np.arange(S_local) if rows is None else np.asarray(rows, dtype=np.int64)
    scale = softmax_scale(dh)
    out = np.zeros((B, len(rows), Hq, dh))
    lse = np.full((B, Hq, len(rows)), -np.inf)
    for b in range(B):
        kv_cache = {}
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            if hk not in kv_cache:
                kv_cache = {hk: (_as_f64(k[b, :, hk, :]), _as_f64(v[b, :, hk, :]))}
            kb, vb = kv_cache[hk]
            for start in range(0, len(rows), block):
                r = rows[start:start + block]
                p = pos_all[r]
                hi = min(kv_end, int(p.max()) + 1)
                if hi <= kv_begin:
                    continue  # no row of the block sees a key of the range
                keys = np.arange(kv_begin, hi, dtype=np.int64)
                s = scale * (q[b, r, h, :] @ kb[kv_begin:hi].T)
                vis = visible(keys, p)
                s = np.where(vis, s, -np.inf)
                any_vis = vis.any(axis=1)
                m = np.where(any_vis, s.max(axis=1), 0.0)[:, None]
                w = np.where(vis, np.exp(s - m), 0.0)
                l = w.sum(axis=1, keepdims=True)
                o = np.where(any_vis[:, None], (w @ vb[kv_begin:hi]) / np.where(l > 0, l, 1.0), 0.0)
                out[b, start:start + len(r), h, :] = o
                lse[b, h, start:start + len(r)] = np.where(any_vis, (m + np.log(np.where(l > 0, l, 1.0)))[:, 0], -np.inf)
    return out, lse


def merge_partials(out_a, lse_a, out_b, lse_b):
    """Combine two partial results over disjoint key sets (log-sum-exp weights).

    out: [B, rows, Hq, dh]; lse: [B, Hq, rows]. A partial with lse = -inf contributes
    nothing; if both are empty the result is out = 0, lse = -inf.
    """
    out_a, out_b = _as_f64(out_a), _as_f64(out_b)
    lse_a, lse_b = _as_f64(lse_a), _as_f64(lse_b)
    m = np.maximum(lse_a, lse_b)
    finite = np.isfinite(m)
    m0 = np.where(finite, m, 0.0)
    wa = np.where(np.isfinite(lse_a), np.exp(lse_a - m0), 0.0)
    wb = np.where(np.isfinite(lse_b), np.exp(lse_b - m0), 0.0)
    tot = wa + wb
    lse = np.where(finite, m0 + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    ta = np.where(tot > 0, wa / np.where(tot > 0, tot, 1.0), 0.0)
    tb = np.where(tot > 0, wb / np.where(tot > 0, tot, 1.0), 0.0)
    # weights are [B, Hq, rows]; outputs are [B, rows, Hq, dh]
    out = out_a * ta.transpose(0, 2, 1)[..., None] + out_b * tb.transpose(0, 2, 1)[..., None]
    return out, lse


# --------------------------------------------------------------------------------------
# The backward pass of the per-rank attention.
# Both systems the pages describe train models ("Folding Tensor and Sequence Parallelism
# for Memory-Efficient Transformer Training & Inference"; "AutoSP: Unlocking
# Long-Context LLM Training ...", section 2.B: attention activations are recomputed in
# the backward pass rather than kept). The backward of the forward above is its
# gradient, by the chain rule through the softmax. With s_ij = scale * q_i . k_j on
# visible pairs and P_ij = softmax_j(s_ij) (0 on masked pairs), for an upstream
# gradient dO of out:
#   dV_j  = sum_i P_ij dO_i
#   dP_ij = dO_i . v_j
#   dS_ij = P_ij (dP_ij - sum_l P_il dP_il)
#   dQ_i  = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i
# dK and dV are this rank's partial gradients of the gathered full K/V: the all-gather's
# adjoint is a reduce-scatter that adds up the partials of all ranks ("Tensor, pipeline
# e sequence parallelism", section 01: row-parallel pieces sum partial results). The
# query heads that share a KV head add their contributions to it.
# --------------------------------------------------------------------------------------
def causal_attention_backward(q, k, v, dout, D: int, rank: int, kv_heads=None, block: int = 256, rows=None):
    """Oracle backward for one rank.

    q, dout: [B, S_local, Hq, dh]; k, v: [B, S_total, Hkv, dh].
    kv_heads: optional subset of KV heads; the query heads of their groups are included.
    rows: optional local row indices; only their terms are computed (dq of the other rows
    stays 0, and dk / dv hold these rows' contributions, which add up over the rows, so the
    results of a partition of the rows sum to the full result).
    Returns (dq [B, S_local, n_q, dh], dk [B, S_total, n_kv, dh], dv [B, S_total, n_kv, dh])
    in float64, n_kv = len(kv_heads), n_q = n_kv * Hq / Hkv (query heads in group order).
    Keys that no local row sees get dk = dv = 0.
    """
    q, dout = _as_f64(q), _as_f64(dout)
    B, S_local, Hq, dh = q.shape
    S_total, Hkv = k.shape[1], k.shape[2]
    pos_all = zigzag_positions(S_total, D, rank)
    if S_local != pos_all.shape[0] or dout.shape != q.shape:
        raise ValueError("q_local and dout must hold 2 * S_total / (2D) rows")
    kv_heads = list(range(Hkv)) if kv_heads is None else list(kv_heads)
    sel = np.arange(S_local) if rows is None else np.asarray(rows, dtype=np.int64)
    if sel.size and (sel.min() < 0 or sel.max() >= S_local):
        raise ValueError("rows outside the local rows")
    grp = Hq // Hkv
    scale = softmax_scale(dh)
    dq = np.zeros((B, S_local, len(kv_heads) * grp, dh))
    dk = np.zeros((B, S_total, len(kv_heads), dh))
    dv = np.zeros((B, S_total, len(kv_heads), dh))
    for b in range(B):
        for ki, hk in enumerate(kv_heads):
            kb, vb = _as_f64(k[b, :, hk, :]), _as_f64(v[b, :, hk, :])
            for g in range(grp):
                h = hk * grp + g
                if kv_head_of(h, Hq, Hkv) != hk:
                    raise ValueError("query head outside the KV head's group")
                for start in range(0, len(sel), block):
                    r = sel[start:start + block]
                    p = pos_all[r]
                    nkeys = int(p.max()) + 1
                    keys = np.arange(nkeys, dtype=np.int64)
                    vis = visible(keys, p)
                    s = np.where(vis, scale * (q[b, r, h, :] @ kb[:nkeys].T), -np.inf)
                    e = np.exp(s - s.max(axis=1, keepdims=True))
                    P = e / e.sum(axis=1, keepdims=True)  # softmax over the visible keys
                    dO = dout[b, r, h, :]
                    dP = dO @ vb[:nkeys].T
                    dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
                    dq[b, r, ki * grp + g, :] = scale * (dS @ kb[:nkeys])
                    dk[b, :nkeys, ki, :] += scale * (dS.T @ q[b, r, h, :])
                    dv[b, :nkeys, ki, :] += P.T @ dO
    return dq, dk, dv
