"""Pins for the fp64 oracle: checks against what the pages and the mathematics fix.

Each ``pin_*`` takes an oracle namespace ``o`` (attributes ``causal_attention``,
``causal_attention_bruteforce``, ``zigzag_positions``, ``unmasked_pairs``, ``causal_flops``,
``kv_head_of``, ``causal_attention_range``, ``merge_partials``,
``causal_attention_backward``, ``ulysses``, ``tsp_layer``) and raises AssertionError when the
implementation breaks the pin. The
same pins run against deliberately broken copies in test_oracle_mutants.py, which
shows that a plausible mistake anywhere in the oracle trips at least one of them.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# -- the zigzag map ----------------------------------------------------------------------

def pin_zigzag_golden(o):
    """Chunk ownership of the workloads' shards (zigzag_ownership.json)."""
    for c in _load("zigzag_ownership.json")["cases"]:
        S, D, r = c["S_total"], c["D"], c["rank"]
        C = S // (2 * D)
        lo, hi = c["chunks"]
        pos = np.asarray(o.zigzag_positions(S, D, r))
        assert pos.shape == (2 * C,), (c, pos.shape)
        assert np.array_equal(pos[:C], np.arange(lo * C, (lo + 1) * C)), c
        assert np.array_equal(pos[C:], np.arange(hi * C, (hi + 1) * C)), c


def pin_zigzag_permutation(o):
    """Over all ranks the map is a permutation of [0, S_total); D = 1 is the identity."""
    for S, D in [(8, 1), (24, 2), (48, 3), (64, 4), (512, 4), (4096, 8), (1040, 8)]:
        allpos = np.concatenate([np.asarray(o.zigzag_positions(S, D, r)) for r in range(D)])
        assert np.array_equal(np.sort(allpos), np.arange(S)), (S, D)
        for r in range(D):
            pos = np.asarray(o.zigzag_positions(S, D, r))
            assert np.all(np.diff(pos) > 0), (S, D, r)
    assert np.array_equal(np.asarray(o.zigzag_positions(96, 1, 0)), np.arange(96))


def pin_pairs_closed_form(o):
    """Every rank sees C * (S_total + 1) visible (query, key) pairs per (batch, head).

    Closed form: chunks c and 2D-1-c contribute (c*C^2 + C(C+1)/2) and
    ((2D-1-c)*C^2 + C(C+1)/2); their sum is (2D-1)*C^2 + C^2 + C = C*(S_total + 1).
    """
    for S, D in [(512, 4), (32768, 8), (65536, 4), (131072, 1), (262144, 8), (120, 3), (14, 7)]:
        C = S // (2 * D)
        for r in range(D):
            assert int(o.unmasked_pairs(S, D, r)) == C * (S + 1), (S, D, r)


def pin_causal_flops(o):
    """The algorithmic FLOP count: per visible (query, key) pair and query head, one dot
    product of length dh for the score (dh multiplies, dh adds) and one scaled row of V
    added into the output (dh multiplies, dh adds).

    Checked by counting those operations pair by pair with scalar loops on tiny shards
    (positions built here from the chunk definition: chunk r, then chunk 2D-1-r), and
    against the per-workload counts of the five measured shapes as printed to 4-5
    significant digits (3.362e7, 1.0995e12, 1.3194e13, 1.7592e13, 1.0555e14).
    """
    for B, S, D, r, Hq, dh in [(1, 8, 1, 0, 1, 4), (2, 24, 3, 1, 3, 8), (1, 40, 4, 3, 2, 16), (3, 28, 7, 6, 5, 2)]:
        C = S // (2 * D)
        positions = list(range(r * C, (r + 1) * C)) + list(range((2 * D - 1 - r) * C, (2 * D - r) * C))
        ops = 0
        for _b in range(B):
            for _h in range(Hq):
                for p in positions:
                    for j in range(S):
                        if j <= p:
                            ops += dh + dh  # score: multiplies and adds of the dot product
                            ops += dh + dh  # output: weight times value row, added in
        assert int(o.causal_flops(B, Hq, dh, S, D, r)) == ops, (B, S, D, r, Hq, dh)
    printed = [((1, 4, 64, 512, 4, 1), 3.362e7), ((1, 32, 128, 32768, 8, 3), 1.0995e12),
               ((1, 24, 256, 65536, 4, 2), 1.3194e13), ((1, 4, 128, 131072, 1, 0), 1.7592e13),
               ((1, 24, 256, 262144, 8, 0), 1.0555e14), ((1, 24, 256, 262144, 8, 7), 1.0555e14)]
    for args, want in printed:
        got = float(o.causal_flops(*args))
        digits = 10 ** (math.floor(math.log10(want)) - 3)  # the last printed digit
        assert abs(got - want) <= digits, (args, got, want)


def pin_gqa_ownership(o):
    """The lesson page's degree-4 split of 24 query heads over 4 KV heads."""
    g = _load("gqa_head_ownership.json")
    Hq, Hkv, deg = g["Hq"], g["Hkv"], g["degree"]
    per = Hq // deg
    assert per == g["query_heads_per_rank"]
    assert Hkv * g["dh"] == g["kv_proj_width"]
    for r in range(deg):
        owned = {o.kv_head_of(h, Hq, Hkv) for h in range(r * per, (r + 1) * per)}
        assert len(owned) == g["kv_heads_per_rank"], (r, owned)
    used = [o.kv_head_of(h, Hq, Hkv) for h in range(Hq)]
    assert sorted(set(used)) == list(range(Hkv))


# -- the attention ---------------------------------------------------------------------

TINY = [  # (B, S_total, D, rank, Hq, Hkv, dh)
    (1, 8, 1, 0, 1, 1, 4),
    (1, 16, 2, 1, 2, 1, 4),
    (2, 24, 3, 0, 3, 3, 3),
    (1, 24, 3, 2, 4, 2, 5),
    (1, 32, 4, 1, 4, 1, 8),
]


def _tiny_inputs(case, seed):
    B, S, D, r, Hq, Hkv, dh = case
    q = _rand((B, S // D, Hq, dh), seed)
    k = _rand((B, S, Hkv, dh), seed + 1)
    v = _rand((B, S, Hkv, dh), seed + 2)
    return q, k, v


def pin_bruteforce(o):
    """Blocked matrix form == scalar triple loop, with blocks smaller than a chunk."""
    for n, case in enumerate(TINY):
        q, k, v = _tiny_inputs(case, 10 + n)
        D, r = case[2], case[3]
        out_b, lse_b = o.causal_attention(q, k, v, D, r, block=3)
        out_r, lse_r = o.causal_attention_bruteforce(q, k, v, D, r)
        assert np.allclose(out_b, out_r, rtol=0, atol=1e-12), case
        assert np.allclose(lse_b, lse_r, rtol=0, atol=1e-12), case


def pin_sdpa_one_rank(o):
    """D = 1 (Ulysses head subset) equals PyTorch's causal SDPA in fp64 on the CPU."""
    for B, S, Hq, Hkv, dh, seed in [(1, 40, 2, 2, 8, 1), (2, 33 * 2, 6, 2, 16, 2), (1, 128, 4, 1, 32, 3)]:
        q = _rand((B, S, Hq, dh), seed)
        k = _rand((B, S, Hkv, dh), seed + 1)
        v = _rand((B, S, Hkv, dh), seed + 2)
        out, lse = o.causal_attention(q, k, v, 1, 0)
        grp = Hq // Hkv
        tq = torch.from_numpy(q).permute(0, 2, 1, 3)
        tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(grp, dim=1)
        tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(grp, dim=1)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
        ref = ref.permute(0, 2, 1, 3).numpy()
        assert np.allclose(out, ref, rtol=0, atol=1e-12), (B, S, Hq, Hkv, dh)
        s = torch.einsum("bhid,bhjd->bhij", tq, tk) / math.sqrt(dh)
        s = s.masked_fill(torch.triu(torch.ones(S, S, dtype=torch.bool), 1), float("-inf"))
        assert np.allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


def pin_concatenation(o):
    """Scattering every rank's rows by global position rebuilds the unsharded result."""
    for B, S, D, Hq, Hkv, dh, seed in [(1, 48, 3, 2, 1, 4, 5), (1, 64, 4, 4, 2, 8, 6), (2, 32, 2, 1, 1, 4, 7)]:
        qf = _rand((B, S, Hq, dh), seed)
        k = _rand((B, S, Hkv, dh), seed + 1)
        v = _rand((B, S, Hkv, dh), seed + 2)
        full_out, full_lse = o.causal_attention(qf, k, v, 1, 0)
        got_out = np.full_like(full_out, np.nan)
        got_lse = np.full_like(full_lse, np.nan)
        for r in range(D):
            pos = np.asarray(o.zigzag_positions(S, D, r))
            out, lse = o.causal_attention(qf[:, pos], k, v, D, r)
            got_out[:, pos] = out
            got_lse[:, :, pos] = lse
        assert np.allclose(got_out, full_out, rtol=0, atol=1e-12), (S, D)
        assert np.allclose(got_lse, full_lse, rtol=0, atol=1e-12), (S, D)


def pin_probabilities(o):
    """One-hot values expose the softmax matrix: rows sum to 1, zero exactly past the
    query's global position, positive up to it, and equal exp(score - lse)."""
    B, S, D, Hq, Hkv = 1, 24, 3, 2, 1
    dh = S  # value row j = e_j, so out[i, j] is the weight of key j
    for r in range(D):
        q = _rand((B, S // D, Hq, dh), 20 + r)
        k = _rand((B, S, Hkv, dh), 30)
        v = np.eye(S).reshape(1, S, 1, S)
        out, lse = o.causal_attention(q, k, v, D, r)
        pos = np.arange(r * (S // (2 * D)), (r + 1) * (S // (2 * D)))
        pos = np.concatenate([pos, np.arange((2 * D - 1 - r) * (S // (2 * D)), (2 * D - r) * (S // (2 * D)))])
        for h in range(Hq):
            P = out[0, :, h, :]
            assert np.allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-12)
            for i, p in enumerate(pos):
                assert np.all(P[i, p + 1:] == 0.0), (r, h, i)
                assert np.all(P[i, :p + 1] > 0.0), (r, h, i)
                s = (q[0, i, h] @ k[0, :p + 1, 0].T) / math.sqrt(dh)
                assert np.allclose(P[i, :p + 1], np.exp(s - lse[0, h, i]), rtol=1e-12, atol=0)


def pin_values_ones(o):
    """v = 1 everywhere gives out = 1 (weights are normalised)."""
    q, k, _ = _tiny_inputs((1, 32, 4, 2, 4, 2, 8), 40)
    out, _ = o.causal_attention(q, k, np.ones_like(k), 4, 2)
    assert np.allclose(out, 1.0, rtol=0, atol=1e-13)


def pin_zero_queries(o):
    """q = 0: every visible key weighs the same, so out is the prefix mean of v and
    lse = ln(position + 1)."""
    B, S, D, Hq, Hkv, dh = 1, 64, 4, 4, 2, 8
    k = _rand((B, S, Hkv, dh), 50)
    v = _rand((B, S, Hkv, dh), 51)
    for r in range(D):
        q = np.zeros((B, S // D, Hq, dh))
        out, lse = o.causal_attention(q, k, v, D, r)
        C = S // (2 * D)
        pos = np.concatenate([np.arange(r * C, (r + 1) * C), np.arange((2 * D - 1 - r) * C, (2 * D - r) * C)])
        for h in range(Hq):
            hk = h // (Hq // Hkv)
            prefix_mean = np.cumsum(v[0, :, hk, :], axis=0) / np.arange(1, S + 1)[:, None]
            assert np.allclose(out[0, :, h, :], prefix_mean[pos], rtol=0, atol=1e-13), (r, h)
            assert np.allclose(lse[0, h, :], np.log(pos + 1.0), rtol=0, atol=1e-13), (r, h)


def pin_first_position(o):
    """The query at global position 0 sees only key 0: out = v_0, lse = q.k_0 / sqrt(dh)."""
    for dh in (4, 16, 64):
        q, k, v = _tiny_inputs((1, 32, 4, 0, 2, 1, dh), 60 + dh)
        out, lse = o.causal_attention(q, k, v, 4, 0)
        for h in range(2):
            assert np.allclose(out[0, 0, h], v[0, 0, 0], rtol=0, atol=1e-14)
            assert abs(lse[0, h, 0] - q[0, 0, h] @ k[0, 0, 0] / math.sqrt(dh)) < 1e-13


def pin_gqa_equivalence(o):
    """Grouped-query attention == multi-head attention on repeated K/V heads."""
    B, S, D, r, Hq, Hkv, dh = 1, 48, 3, 1, 6, 2, 8
    q, k, v = _tiny_inputs((B, S, D, r, Hq, Hkv, dh), 70)
    out_g, lse_g = o.causal_attention(q, k, v, D, r)
    grp = Hq // Hkv
    out_m, lse_m = o.causal_attention(q, np.repeat(k, grp, axis=2), np.repeat(v, grp, axis=2), D, r)
    assert np.allclose(out_g, out_m, rtol=0, atol=1e-13)
    assert np.allclose(lse_g, lse_m, rtol=0, atol=1e-13)


def pin_shift_invariance(o):
    """Adding c to every key leaves out unchanged and shifts lse by q.c / sqrt(dh)."""
    B, S, D, r, Hq, Hkv, dh = 1, 32, 2, 1, 2, 1, 8
    q, k, v = _tiny_inputs((B, S, D, r, Hq, Hkv, dh), 80)
    c = _rand((dh,), 81)
    out0, lse0 = o.causal_attention(q, k, v, D, r)
    out1, lse1 = o.causal_attention(q, k + c, v, D, r)
    assert np.allclose(out0, out1, rtol=0, atol=1e-12)
    shift = np.einsum("bshd,d->bhs", q, c) / math.sqrt(dh)
    assert np.allclose(lse1 - lse0, shift, rtol=0, atol=1e-12)


# -- attention over key ranges and the merge of partials -------------------------------

def pin_range_bruteforce(o):
    """Key-range partials == scalar loops restricted to the range (incl. empty rows)."""
    for n, case in enumerate(TINY):
        q, k, v = _tiny_inputs(case, 90 + n)
        S, D, r = case[1], case[2], case[3]
        for lo, hi in [(0, S), (0, S // 3), (S // 3, S), (S // 4, S // 2 + 1), (S - 1, S), (5, 5)]:
            out_b, lse_b = o.causal_attention_range(q, k, v, D, r, lo, hi, block=3)
            out_r, lse_r = o.causal_attention_bruteforce(q, k, v, D, r, lo, hi)
            assert np.allclose(out_b, out_r, rtol=0, atol=1e-12), (case, lo, hi)
            assert np.array_equal(np.isinf(lse_b), np.isinf(lse_r)), (case, lo, hi)
            fin = np.isfinite(lse_r)
            assert np.allclose(lse_b[fin], lse_r[fin], rtol=0, atol=1e-12), (case, lo, hi)


def pin_range_partition(o):
    """Merging the partials of any split of [0, S_total) reproduces the full attention
    (the softmax denominator is a sum over keys, split by the log-sum-exp combination)."""
    for n, (B, S, D, r, Hq, Hkv, dh) in enumerate([(1, 32, 4, 1, 2, 1, 8), (2, 48, 3, 2, 4, 2, 4),
                                                    (1, 64, 1, 0, 2, 2, 8)]):
        q, k, v = _tiny_inputs((B, S, D, r, Hq, Hkv, dh), 100 + n)
        full_out, full_lse = o.causal_attention(q, k, v, D, r)
        C = S // (2 * D)
        cuts_list = [list(range(0, S + 1, C)),          # the all-gather's chunks
                     [0, 3, 3, 17, S - 2, S],           # ragged, with an empty range
                     [0, S]]
        for cuts in cuts_list:
            parts = [o.causal_attention_range(q, k, v, D, r, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
            for order in (parts, parts[::-1]):
                acc_o, acc_l = order[0]
                for po, pl in order[1:]:
                    acc_o, acc_l = o.merge_partials(acc_o, acc_l, po, pl)
                assert np.allclose(acc_o, full_out, rtol=0, atol=1e-12), (S, D, cuts)
                assert np.allclose(acc_l, full_lse, rtol=0, atol=1e-12), (S, D, cuts)


def pin_merge_identity(o):
    """An empty partial (lse = -inf) is the identity of the merge; the merge commutes."""
    rng = np.random.default_rng(110)
    out_a = rng.standard_normal((1, 5, 2, 4))
    lse_a = rng.standard_normal((1, 2, 5))
    out_e = np.zeros_like(out_a)
    lse_e = np.full_like(lse_a, -np.inf)
    mo, ml = o.merge_partials(out_a, lse_a, out_e, lse_e)
    assert np.array_equal(mo, out_a) and np.array_equal(ml, lse_a)
    mo, ml = o.merge_partials(out_e, lse_e, out_e, lse_e)
    assert np.all(mo == 0) and np.all(np.isneginf(ml))
    out_b = rng.standard_normal((1, 5, 2, 4))
    lse_b = rng.standard_normal((1, 2, 5))
    m1 = o.merge_partials(out_a, lse_a, out_b, lse_b)
    m2 = o.merge_partials(out_b, lse_b, out_a, lse_a)
    assert np.allclose(m1[0], m2[0], rtol=0, atol=1e-15) and np.allclose(m1[1], m2[1], rtol=0, atol=1e-15)


# -- the backward pass -------------------------------------------------------------------

BWD_TINY = [  # (B, S_total, D, rank, Hq, Hkv, dh)
    (1, 8, 2, 1, 2, 1, 4),    # zigzag, GQA 2:1
    (1, 12, 3, 0, 1, 1, 3),   # rank 0 of 3 (holds the first and the last chunk)
    (2, 8, 1, 0, 2, 2, 2),    # D = 1, batch of 2
]


def _bwd_inputs(case, seed):
    B, S, D, r, Hq, Hkv, dh = case
    q, k, v = _tiny_inputs(case, seed)
    dout = _rand((B, S // D, Hq, dh), seed + 3)
    return q, k, v, dout


def pin_bwd_finite_differences(o):
    """The backward is the derivative of the forward: central differences of
    L = sum(out * dout) in every input element match dq, dk, dv."""
    eps = 1e-6
    for n, case in enumerate(BWD_TINY):
        B, S, D, r, Hq, Hkv, dh = case
        q, k, v, dout = _bwd_inputs(case, 40 + n)
        dq, dk, dv = o.causal_attention_backward(q, k, v, dout, D, r, block=3)

        def loss(qq, kk, vv):
            return float(np.sum(o.causal_attention(qq, kk, vv, D, r)[0] * dout))

        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
                args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert np.allclose(g, num, rtol=0, atol=1e-7), (case, name, np.abs(g - num).max())


def pin_bwd_autograd_sdpa(o):
    """D = 1: equals PyTorch autograd through its causal SDPA in fp64 (GQA by
    repeat_interleave, whose adjoint sums the group's KV gradients)."""
    for B, S, Hq, Hkv, dh, seed in [(1, 24, 2, 2, 8, 50), (2, 40, 6, 2, 16, 51), (1, 64, 4, 1, 32, 52)]:
        q = _rand((B, S, Hq, dh), seed)
        k = _rand((B, S, Hkv, dh), seed + 1)
        v = _rand((B, S, Hkv, dh), seed + 2)
        dout = _rand((B, S, Hq, dh), seed + 3)
        dq, dk, dv = o.causal_attention_backward(q, k, v, dout, 1, 0, block=16)
        grp = Hq // Hkv
        tq = torch.from_numpy(q).requires_grad_()
        tk = torch.from_numpy(k).requires_grad_()
        tv = torch.from_numpy(v).requires_grad_()
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq.permute(0, 2, 1, 3), tk.permute(0, 2, 1, 3).repeat_interleave(grp, dim=1),
            tv.permute(0, 2, 1, 3).repeat_interleave(grp, dim=1), is_causal=True)
        ref.permute(0, 2, 1, 3).backward(torch.from_numpy(dout))
        for got, t in ((dq, tq), (dk, tk), (dv, tv)):
            assert np.allclose(got, t.grad.numpy(), rtol=0, atol=1e-10), (B, S, Hq, Hkv, dh)


def pin_bwd_rank_partition(o):
    """The ranks' partial dK/dV add up to the unsharded gradient, and their dQ rows,
    scattered by global position, rebuild the unsharded dQ."""
    for B, S, D, Hq, Hkv, dh, seed in [(1, 48, 3, 2, 1, 4, 60), (1, 64, 4, 4, 2, 8, 61), (2, 32, 2, 1, 1, 4, 62)]:
        qf = _rand((B, S, Hq, dh), seed)
        k = _rand((B, S, Hkv, dh), seed + 1)
        v = _rand((B, S, Hkv, dh), seed + 2)
        dof = _rand((B, S, Hq, dh), seed + 3)
        fq, fk, fv = o.causal_attention_backward(qf, k, v, dof, 1, 0)
        gq = np.full_like(fq, np.nan)
        gk, gv = np.zeros_like(fk), np.zeros_like(fv)
        for r in range(D):
            pos = np.asarray(o.zigzag_positions(S, D, r))
            dq, dk, dv = o.causal_attention_backward(qf[:, pos], k, v, dof[:, pos], D, r)
            gq[:, pos] = dq
            gk += dk
            gv += dv
        assert np.allclose(gq, fq, rtol=0, atol=1e-12), (S, D)
        assert np.allclose(gk, fk, rtol=0, atol=1e-12), (S, D)
        assert np.allclose(gv, fv, rtol=0, atol=1e-12), (S, D)


def pin_bwd_closed_forms(o):
    """Softmax rows sum to 1, so the dK of every KV head sums to 0 over the keys and its
    dV sums to the group's total upstream gradient; dout = 0 gives zero gradients; equal
    value rows give dq = dk = 0 (out no longer depends on the scores)."""
    B, S, D, r, Hq, Hkv, dh = 1, 64, 4, 2, 6, 2, 8
    q, k, v, dout = _bwd_inputs((B, S, D, r, Hq, Hkv, dh), 70)
    dq, dk, dv = o.causal_attention_backward(q, k, v, dout, D, r, block=7)
    assert np.allclose(dk.sum(axis=1), 0.0, rtol=0, atol=1e-12)
    grp = Hq // Hkv
    for hk in range(Hkv):
        tot = dout[:, :, hk * grp:(hk + 1) * grp, :].sum(axis=(1, 2))
        assert np.allclose(dv[:, :, hk, :].sum(axis=1), tot, rtol=0, atol=1e-12)
    # keys past the rank's last position get nothing
    last = int(np.asarray(o.zigzag_positions(S, D, r)).max())
    assert np.all(dk[:, last + 1:] == 0) and np.all(dv[:, last + 1:] == 0)
    z = o.causal_attention_backward(q, k, v, np.zeros_like(dout), D, r)
    assert all(np.all(t == 0) for t in z)
    vc = np.broadcast_to(_rand((B, 1, Hkv, dh), 71), v.shape).copy()
    dq2, dk2, _ = o.causal_attention_backward(q, k, vc, dout, D, r)
    assert np.allclose(dq2, 0.0, rtol=0, atol=1e-12) and np.allclose(dk2, 0.0, rtol=0, atol=1e-12)


def pin_bwd_gqa_and_subset(o):
    """GQA gradients equal the MHA gradients on repeated K/V with each group's dK/dV
    summed; a subset of KV heads returns exactly those heads' slices."""
    B, S, D, r, Hq, Hkv, dh = 1, 48, 3, 1, 6, 2, 4
    q, k, v, dout = _bwd_inputs((B, S, D, r, Hq, Hkv, dh), 80)
    grp = Hq // Hkv
    dq, dk, dv = o.causal_attention_backward(q, k, v, dout, D, r)
    mq, mk, mv = o.causal_attention_backward(q, np.repeat(k, grp, axis=2), np.repeat(v, grp, axis=2), dout, D, r)
    assert np.allclose(dq, mq, rtol=0, atol=1e-12)
    assert np.allclose(dk, mk.reshape(B, S, Hkv, grp, dh).sum(axis=3), rtol=0, atol=1e-12)
    assert np.allclose(dv, mv.reshape(B, S, Hkv, grp, dh).sum(axis=3), rtol=0, atol=1e-12)
    sq, sk, sv = o.causal_attention_backward(q, k, v, dout, D, r, kv_heads=[1])
    assert np.array_equal(sq, dq[:, :, grp:2 * grp]) and np.array_equal(sk, dk[:, :, 1:2])
    assert np.array_equal(sv, dv[:, :, 1:2])


def pin_bwd_row_subsets(o):
    """The backward restricted to a set of local rows: over a partition of the rows (an
    interleaved one, with a block size that splits runs), dk and dv add up to the full
    result, each part's dq equals the full dq on its rows and is 0 elsewhere."""
    B, S, D, r, Hq, Hkv, dh = 2, 40, 2, 1, 4, 2, 4
    q, k, v, dout = _bwd_inputs((B, S, D, r, Hq, Hkv, dh), 85)
    fq, fk, fv = o.causal_attention_backward(q, k, v, dout, D, r)
    rows = np.arange(q.shape[1])
    parts = [rows[rows % 3 == 0], rows[rows % 3 != 0][::-1]]
    gq, gk, gv = np.zeros_like(fq), np.zeros_like(fk), np.zeros_like(fv)
    for sel in parts:
        dq, dk, dv = o.causal_attention_backward(q, k, v, dout, D, r, block=4, rows=sel)
        rest = np.setdiff1d(rows, sel)
        assert np.allclose(dq[:, sel], fq[:, sel], rtol=0, atol=1e-12) and np.all(dq[:, rest] == 0)
        gq, gk, gv = gq + dq, gk + dk, gv + dv
    assert np.allclose(gq, fq, rtol=0, atol=1e-12)
    assert np.allclose(gk, fk, rtol=0, atol=1e-12) and np.allclose(gv, fv, rtol=0, atol=1e-12)


# -- the Ulysses layout changes ---------------------------------------------------------

def _coded(shape):
    """Every element holds its own index (a provenance code)."""
    return np.arange(int(np.prod(shape)), dtype=np.int64).reshape(shape)


def pin_ulysses_pack_elementwise(o):
    """pack_heads / gather_sequence against element-by-element loops over every index."""
    u = o.ulysses
    B, S_local, P, Hl, dh = 2, 3, 4, 2, 3
    x = _coded((B, S_local, P * Hl, dh))
    send = u.pack_heads(x, P)
    assert send.shape == (P, B, S_local, Hl, dh)
    for r in range(P):
        for b in range(B):
            for s in range(S_local):
                for hl in range(Hl):
                    for d in range(dh):
                        assert send[r, b, s, hl, d] == x[b, s, r * Hl + hl, d]
    recv = _coded((P, B, S_local, Hl, dh))
    full = u.gather_sequence(recv)
    assert full.shape == (B, P * S_local, Hl, dh)
    for p in range(P):
        for b in range(B):
            for s in range(S_local):
                assert np.array_equal(full[b, p * S_local + s], recv[p, b, s])


def pin_ulysses_round_trip_and_heads(o):
    """Simulated P ranks: pack + all-to-all + gather gives rank r the whole sequence of its
    contiguous heads (the head-subset definition, by slicing the unsharded tensor); the
    reverse path (scatter + all-to-all + unpack) returns every rank its own tokens with
    all heads. The lesson's example: 24 heads over degree 4 give 6 heads per rank."""
    u = o.ulysses
    assert list(u.heads_of_rank(24, 4, 1)) == list(range(6, 12))
    for B, S, H, dh, P in [(1, 16, 8, 4, 4), (2, 12, 6, 2, 3), (1, 8, 4, 3, 1)]:
        xf = _coded((B, S, H, dh))
        S_local, Hl = S // P, H // P
        shards = [xf[:, p * S_local:(p + 1) * S_local] for p in range(P)]
        recvs = u.all_to_all([u.pack_heads(x, P) for x in shards])
        fulls = [u.gather_sequence(rv) for rv in recvs]
        for r in range(P):
            assert np.array_equal(fulls[r], xf[:, :, r * Hl:(r + 1) * Hl]), (B, S, H, P, r)
        back = u.all_to_all([u.scatter_sequence(f, P) for f in fulls])
        for p in range(P):
            assert np.array_equal(u.unpack_heads(back[p], P), shards[p])
        for x in shards:
            assert np.array_equal(u.unpack_heads(u.pack_heads(x, P), P), x)


# -- one rank's TSP attention layer ---------------------------------------------------

def _layer_inputs(B, S, D, Hq, Hkv, dh, dm, seed):
    xf = _rand((B, S, dm), seed) / np.sqrt(dm)
    w_qkv = _rand(((Hq + 2 * Hkv) * dh, dm), seed + 1)
    w_o = _rand((dm, Hq * dh), seed + 2) / np.sqrt(Hq * dh)
    return xf, w_qkv, w_o


def pin_layer_unsharded(o):
    """Every rank's layer output equals the rows, at its zigzag positions, of the standard
    causal multi-head attention layer on the whole sequence (computed here with PyTorch's
    causal SDPA in fp64), when the gathered K/V hold the other ranks' projections; the
    gathered buffers come back with all of the sequence's projections."""
    for B, S, D, Hq, Hkv, dh, dm, seed in [(1, 32, 4, 4, 2, 8, 16, 90), (2, 24, 2, 6, 2, 4, 12, 91)]:
        xf, w_qkv, w_o = _layer_inputs(B, S, D, Hq, Hkv, dh, dm, seed)
        kf = (xf @ w_qkv[Hq * dh:(Hq + Hkv) * dh].T).reshape(B, S, Hkv, dh)
        vf = (xf @ w_qkv[(Hq + Hkv) * dh:].T).reshape(B, S, Hkv, dh)
        qf = (xf @ w_qkv[:Hq * dh].T).reshape(B, S, Hq, dh)
        grp = Hq // Hkv
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qf).permute(0, 2, 1, 3),
            torch.from_numpy(kf).permute(0, 2, 1, 3).repeat_interleave(grp, dim=1),
            torch.from_numpy(vf).permute(0, 2, 1, 3).repeat_interleave(grp, dim=1), is_causal=True)
        yf = ref.permute(0, 2, 1, 3).reshape(B, S, Hq * dh).numpy() @ w_o.T
        for r in range(D):
            pos = np.asarray(o.zigzag_positions(S, D, r))
            garbage_k = np.where(np.isin(np.arange(S), pos)[None, :, None, None], 123.0, kf)
            garbage_v = np.where(np.isin(np.arange(S), pos)[None, :, None, None], -7.0, vf)
            y, K, V = o.tsp_layer.attention_layer(xf[:, pos], w_qkv, w_o, garbage_k, garbage_v, D, r, Hq, Hkv, dh)
            assert np.allclose(y, yf[:, pos], rtol=0, atol=1e-10), (B, S, D, r)
            assert np.allclose(K, kf, rtol=0, atol=1e-12) and np.allclose(V, vf, rtol=0, atol=1e-12)


def pin_layer_shard_sum(o):
    """The shard schedule: the layer with all heads equals the sum of the layers restricted
    to each weight shard's heads (query heads i*Hq/D.., KV heads i*Hkv/D.., the matching
    columns of W_O), which is what accumulating the output projection shard by shard adds up."""
    B, S, D, Hq, Hkv, dh, dm = 1, 32, 4, 8, 4, 8, 16
    xf, w_qkv, w_o = _layer_inputs(B, S, D, Hq, Hkv, dh, dm, 92)
    r = 1
    pos = np.asarray(o.zigzag_positions(S, D, r))
    kf = _rand((B, S, Hkv, dh), 93)
    vf = _rand((B, S, Hkv, dh), 94)
    y, _, _ = o.tsp_layer.attention_layer(xf[:, pos], w_qkv, w_o, kf, vf, D, r, Hq, Hkv, dh)
    hs, hks = Hq // D, Hkv // D
    total = np.zeros_like(y)
    for i in range(D):
        wq = w_qkv[i * hs * dh:(i + 1) * hs * dh]
        wk = w_qkv[Hq * dh + i * hks * dh:Hq * dh + (i + 1) * hks * dh]
        wv = w_qkv[(Hq + Hkv) * dh + i * hks * dh:(Hq + Hkv) * dh + (i + 1) * hks * dh]
        wo = w_o[:, i * hs * dh:(i + 1) * hs * dh]
        yi, _, _ = o.tsp_layer.attention_layer(xf[:, pos], np.concatenate([wq, wk, wv]), wo,
                                               kf[:, :, i * hks:(i + 1) * hks], vf[:, :, i * hks:(i + 1) * hks],
                                               D, r, hs, hks, dh)
        total += yi
    assert np.allclose(total, y, rtol=0, atol=1e-10)


ALL_PINS = [
    pin_zigzag_golden,
    pin_zigzag_permutation,
    pin_pairs_closed_form,
    pin_causal_flops,
    pin_gqa_ownership,
    pin_bruteforce,
    pin_sdpa_one_rank,
    pin_concatenation,
    pin_probabilities,
    pin_values_ones,
    pin_zero_queries,
    pin_first_position,
    pin_gqa_equivalence,
    pin_shift_invariance,
    pin_range_bruteforce,
    pin_range_partition,
    pin_merge_identity,
    pin_bwd_finite_differences,
    pin_bwd_autograd_sdpa,
    pin_bwd_rank_partition,
    pin_bwd_closed_forms,
    pin_bwd_gqa_and_subset,
    pin_bwd_row_subsets,
    pin_ulysses_pack_elementwise,
    pin_ulysses_round_trip_and_heads,
    pin_layer_unsharded,
    pin_layer_shard_sum,
]
