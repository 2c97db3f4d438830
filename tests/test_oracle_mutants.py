"""Planted mistakes in the oracle must each trip at least one pin (CPU only).

Every mutant is a copy of the oracle with one plausible error: a swapped or mirrored
chunk, a strict causal diagonal, interleaved GQA grouping, a wrong softmax scale, a
base-2 lse, a dropped normalisation, swapped K/V operands, local instead of global
positions, a block-boundary error in the blocked form, or a FLOP count with one product
per pair or without the causal mask; and, for the backward, a dropped
softmax-Jacobian term, an unscaled dQ, a wrong operand or an overwritten GQA sum in dK,
unnormalised weights in dV, a strict diagonal, or a row selection that is ignored.
"""

import types

import numpy as np
import pytest

import oracle.attention as A
import oracle.tsp_layer as L
import oracle.ulysses as U
from pins import ALL_PINS


def _zz_swapped(S, D, r):
    pos = A_orig_zigzag(S, D, r)
    C = S // (2 * D)
    return np.concatenate([pos[C:], pos[:C]])


def _zz_mirror_off_by_one(S, D, r):
    C = S // (2 * D)
    hi = (2 * D - r) % (2 * D)
    return np.concatenate([np.arange(r * C, (r + 1) * C), np.arange(hi * C, (hi + 1) * C)])


def _zz_local(S, D, r):
    return np.arange(S // D, dtype=np.int64)


A_orig_zigzag = A.zigzag_positions

PATCHES = {
    "chunk_order_swapped": ("zigzag_positions", _zz_swapped),
    "mirror_chunk_off_by_one": ("zigzag_positions", _zz_mirror_off_by_one),
    "local_positions": ("zigzag_positions", _zz_local),
    "strict_diagonal": ("visible", lambda j, p: j[None, :] < p[:, None]),
    "gqa_interleaved": ("kv_head_of", lambda h, Hq, Hkv: h % Hkv),
    "scale_one_over_dh": ("softmax_scale", lambda dh: 1.0 / dh),
    "no_scale": ("softmax_scale", lambda dh: 1.0),
    # FLOP count with one product per pair instead of two
    "flops_one_product": ("causal_flops", lambda B, Hq, dh, S, D, r: 2 * B * Hq * dh * A.unmasked_pairs(S, D, r)),
    # FLOP count over the rank's local rows times all keys (no causal mask)
    "flops_dense": ("causal_flops", lambda B, Hq, dh, S, D, r: 4 * B * Hq * dh * (S // D) * S),
}


def _lse_log2(f):
    def g(*a, **kw):
        out, lse = f(*a, **kw)
        return out, lse / np.log(2.0)
    return g


def _unnormalised(f):
    def g(*a, **kw):
        out, lse = f(*a, **kw)
        return out * np.exp(lse).transpose(0, 2, 1)[..., None], lse
    return g


def _kv_swapped(f):
    def g(q, k, v, *a, **kw):
        return f(q, v, k, *a, **kw)
    return g


def _block_drops_last_row(f):
    def g(q, k, v, D, rank, rows=None, heads=None, block=256):
        out, lse = f(q, k, v, D, rank, rows=rows, heads=heads, block=block)
        out = out.copy()
        out[:, block - 1::block] = 0.0  # last row of every block lost
        return out, lse
    g.__wrapped_blocked__ = True
    return g


WRAPS = {
    "lse_base2": _lse_log2,
    "dropped_normalisation": _unnormalised,
    "kv_swapped": _kv_swapped,
}


def _namespace():
    ns = types.SimpleNamespace()
    for n in ("causal_attention", "causal_attention_bruteforce", "zigzag_positions",
              "unmasked_pairs", "causal_flops", "kv_head_of", "causal_attention_range", "merge_partials",
              "causal_attention_backward"):
        setattr(ns, n, getattr(A, n))
    ns.ulysses = U
    ns.tsp_layer = L
    return ns


def _failures(ns):
    failed = []
    for pin in ALL_PINS:
        try:
            pin(ns)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(PATCHES))
def test_patched_mutant_is_caught(name, monkeypatch):
    attr, fn = PATCHES[name]
    monkeypatch.setattr(A, attr, fn)
    with np.errstate(all="ignore"):
        failed = _failures(_namespace())
    assert failed, f"mutant {name} passed every pin"


@pytest.mark.parametrize("name", sorted(WRAPS))
def test_wrapped_mutant_is_caught(name):
    ns = _namespace()
    ns.causal_attention = WRAPS[name](A.causal_attention)
    ns.causal_attention_bruteforce = WRAPS[name](A.causal_attention_bruteforce)
    with np.errstate(all="ignore"):
        failed = _failures(ns)
    assert failed, f"mutant {name} passed every pin"


def _merge_linear(out_a, lse_a, out_b, lse_b):
    # plausible mistake: weights from exp(lse) without the shared max, and lse summed
    wa, wb = np.exp(lse_a), np.exp(lse_b)
    t = (wa + wb).transpose(0, 2, 1)[..., None]
    return (out_a * wa.transpose(0, 2, 1)[..., None] + out_b * wb.transpose(0, 2, 1)[..., None]) / t, lse_a + lse_b


def _range_inclusive_end(f):
    def g(q, k, v, D, rank, kv_begin, kv_end, rows=None, block=256):
        return f(q, k, v, D, rank, kv_begin, min(kv_end + 1, k.shape[1]), rows=rows, block=block)
    return g


def test_merge_mistake_is_caught():
    ns = _namespace()
    ns.merge_partials = _merge_linear
    with np.errstate(all="ignore"):
        assert "pin_range_partition" in _failures(ns)


def test_range_end_mistake_is_caught():
    ns = _namespace()
    ns.causal_attention_range = _range_inclusive_end(A.causal_attention_range)
    with np.errstate(all="ignore"):
        failed = _failures(ns)
    assert "pin_range_bruteforce" in failed or "pin_range_partition" in failed


def test_blocked_form_error_is_caught():
    ns = _namespace()
    ns.causal_attention = _block_drops_last_row(A.causal_attention)
    failed = _failures(ns)
    assert "pin_bruteforce" in failed


def _bwd_mutant(kind):
    """A copy of the oracle's backward with one plausible mistake."""

    def bwd(q, k, v, dout, D, rank, kv_heads=None, block=256, rows=None):
        q, dout, k, v = (np.asarray(x, dtype=np.float64) for x in (q, dout, k, v))
        B, S_local, Hq, dh = q.shape
        S_total, Hkv = k.shape[1], k.shape[2]
        pos_all = A.zigzag_positions(S_total, D, rank)
        kv_heads = list(range(Hkv)) if kv_heads is None else list(kv_heads)
        sel = np.arange(S_local) if rows is None or kind == "rows_ignored" else np.asarray(rows)
        grp = Hq // Hkv
        scale = 1.0 / np.sqrt(dh)
        dq = np.zeros((B, S_local, len(kv_heads) * grp, dh))
        dk = np.zeros((B, S_total, len(kv_heads), dh))
        dv = np.zeros((B, S_total, len(kv_heads), dh))
        for b in range(B):
            for ki, hk in enumerate(kv_heads):
                kb, vb = k[b, :, hk, :], v[b, :, hk, :]
                for g in range(grp):
                    h = hk * grp + g
                    for start in range(0, len(sel), block):
                        r = sel[start:start + block]
                        p = pos_all[r]
                        nkeys = int(p.max()) + 1
                        keys = np.arange(nkeys)
                        vis = keys[None, :] < p[:, None] if kind == "strict_diagonal" else keys[None, :] <= p[:, None]
                        s = np.where(vis, scale * (q[b, r, h, :] @ kb[:nkeys].T), -np.inf)
                        e = np.exp(s - s.max(axis=1, keepdims=True))
                        P = e / e.sum(axis=1, keepdims=True)
                        dO = dout[b, r, h, :]
                        dP = dO @ vb[:nkeys].T
                        if kind == "no_delta":
                            dS = P * dP
                        else:
                            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
                        dq[b, r, ki * grp + g, :] = (1.0 if kind == "dq_unscaled" else scale) * (dS @ kb[:nkeys])
                        src = dO if kind == "dk_uses_dout" else q[b, r, h, :]
                        if kind == "gqa_overwrite":
                            dk[b, :nkeys, ki, :] = scale * (dS.T @ src)
                        else:
                            dk[b, :nkeys, ki, :] += scale * (dS.T @ src)
                        dv[b, :nkeys, ki, :] += (e if kind == "dv_unnormalised" else P).T @ dO
        return dq, dk, dv

    return bwd


BWD_MUTANTS = ["no_delta", "dq_unscaled", "dk_uses_dout", "gqa_overwrite", "dv_unnormalised", "strict_diagonal",
               "rows_ignored"]


@pytest.mark.parametrize("kind", BWD_MUTANTS)
def test_backward_mutant_is_caught(kind):
    ns = _namespace()
    ns.causal_attention_backward = _bwd_mutant(kind)
    with np.errstate(all="ignore"):
        failed = [f for f in _failures(ns) if f.startswith("pin_bwd")]
    assert failed, f"backward mutant {kind} passed every backward pin"


def test_backward_mutant_copy_is_faithful():
    """Without a mistake the mutant copy passes the backward pins (so each failure above
    comes from its one change)."""
    ns = _namespace()
    ns.causal_attention_backward = _bwd_mutant("none")
    assert not [f for f in _failures(ns) if f.startswith("pin_bwd")]


def _ulysses_mutant(kind):
    """A copy of the oracle's Ulysses module with one plausible mistake."""
    m = types.SimpleNamespace(**{n: getattr(U, n) for n in
                                 ("heads_of_rank", "pack_heads", "unpack_heads", "gather_sequence",
                                  "scatter_sequence", "all_to_all")})
    if kind == "interleaved_heads":  # head h to rank h % P
        def pack(x, P):
            x = np.asarray(x)
            return np.stack([x[:, :, r::P, :] for r in range(P)], axis=0)
        m.pack_heads = pack
    elif kind == "sequence_order_reversed":  # blocks stored in reverse source order
        def gather(recv):
            recv = np.asarray(recv)
            return U.gather_sequence(recv[::-1])
        m.gather_sequence = gather
    elif kind == "pack_axes_swapped":  # [B, P, ...] instead of [P, B, ...]
        def pack(x, P):
            return np.swapaxes(U.pack_heads(x, P), 0, 1).reshape(U.pack_heads(x, P).shape)
        m.pack_heads = pack
    return m


@pytest.mark.parametrize("kind", ["interleaved_heads", "sequence_order_reversed", "pack_axes_swapped"])
def test_ulysses_mutant_is_caught(kind):
    ns = _namespace()
    ns.ulysses = _ulysses_mutant(kind)
    failed = [f for f in _failures(ns) if f.startswith("pin_ulysses")]
    assert failed, f"Ulysses mutant {kind} passed every Ulysses pin"


def _layer_mutant(kind):
    """A copy of the layer oracle with one plausible mistake."""
    def layer(x_local, w_qkv, w_o, k_gathered, v_gathered, D, rank, Hq, Hkv, dh):
        x, W, Wo = (np.asarray(t, dtype=np.float64) for t in (x_local, w_qkv, w_o))
        B, S_local, dm = x.shape
        K = np.array(k_gathered, dtype=np.float64)
        V = np.array(v_gathered, dtype=np.float64)
        q = (x @ W[:Hq * dh].T).reshape(B, S_local, Hq, dh)
        k_loc = (x @ W[Hq * dh:(Hq + Hkv) * dh].T).reshape(B, S_local, Hkv, dh)
        v_loc = (x @ W[(Hq + Hkv) * dh:].T).reshape(B, S_local, Hkv, dh)
        pos = A.zigzag_positions(K.shape[1], D, rank)
        if kind == "local_rows_not_placed":
            pass
        elif kind == "placed_at_local_rows":
            K[:, :S_local] = k_loc
            V[:, :S_local] = v_loc
        else:
            K[:, pos] = k_loc
            V[:, pos] = v_loc
        if kind == "k_v_weights_swapped":
            K[:, pos], V[:, pos] = v_loc, k_loc
        o, _ = A.causal_attention(q, K, V, D, rank)
        y = o.reshape(B, S_local, Hq * dh) @ (Wo if kind == "w_o_untransposed" and Wo.shape[0] == Wo.shape[1] else Wo.T)
        return y, K, V
    return layer


@pytest.mark.parametrize("kind", ["local_rows_not_placed", "placed_at_local_rows", "k_v_weights_swapped",
                                  "w_o_untransposed"])
def test_layer_mutant_is_caught(kind):
    ns = _namespace()
    ns.tsp_layer = types.SimpleNamespace(attention_layer=_layer_mutant(kind))
    with np.errstate(all="ignore"):
        failed = [f for f in _failures(ns) if f.startswith("pin_layer")]
    assert failed, f"layer mutant {kind} passed every layer pin"
