"""Backward (tsp_attn_bwd) vs the fp64 oracle's gradients, through the C ABI, on an MI355X.

The forward's out / lse come from the HIP forward (as in training); the oracle computes
the gradients from q, k, v and dout alone. Tolerances (bf16 inputs, bf16 outputs; fp32
cases below have their own, tighter bounds):
per tensor and KV head, relative Frobenius error <= 1e-2, and max-abs error
<= 2^-6 * max|ref| + 1e-3 (the outputs are rounded to bf16, 2^-9 relative, and P / dS
are rounded to bf16 before their products, with fp32 accumulation).
"""

import numpy as np
import pytest
import torch

import oracle
import sequence_causal_attention_amd as tsp
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _note(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def check_grad(name, got, ref, axis_head):
    """Per-head relative Frobenius and scaled max-abs bounds; returns the worst errors."""
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    worst = (0.0, 0.0)
    for h in range(got.shape[axis_head]):
        g = np.take(got, h, axis=axis_head)
        r = np.take(ref, h, axis=axis_head)
        scale = np.abs(r).max()
        err = np.abs(g - r).max()
        rel = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)
        assert err <= 2.0 ** -6 * scale + 1e-3, f"{name} head {h}: max err {err:.3g} vs max|ref| {scale:.3g}"
        assert rel <= 1e-2, f"{name} head {h}: relative error {rel:.3g}"
        worst = (max(worst[0], err / max(scale, 1e-30)), max(worst[1], rel))
    return worst


def run_bwd(q, k, v, dout, D, rank):
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, dout))
    out, lse = tsp.fwd(qd, kd, vd, D=D, rank=rank)
    dq, dk, dv, delta = tsp.bwd(qd, kd, vd, out, lse, dod, D=D, rank=rank)
    torch.cuda.synchronize()
    return dq, dk, dv, delta


CASES = [  # (B, S_total, D, rank, Hq, Hkv, dh)
    (1, 2048, 8, 3, 4, 4, 128),    # 7B-style MHA shard, scaled down
    (1, 2048, 8, 0, 4, 4, 128),
    (1, 2048, 8, 7, 4, 4, 128),
    (1, 4096, 4, 2, 12, 2, 256),   # GQA 6:1, dh 256
    (1, 4096, 1, 0, 4, 4, 128),    # D = 1
    (1, 1024, 2, 1, 8, 2, 64),     # dh 64
    (1, 1200, 3, 2, 6, 2, 128),    # ragged: C = 200
    (1, 1200, 3, 0, 6, 3, 256),    # ragged, dh 256, grp 2
    (2, 1024, 4, 1, 4, 2, 128),    # batch of 2
    (1, 8, 4, 3, 2, 1, 64),        # one token per chunk
    (1, 96, 1, 0, 3, 1, 128),      # grp 3
    (1, 2, 1, 0, 1, 1, 128),       # two tokens
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_S{}_D{}_r{}_H{}x{}_d{}".format(*c))
def test_bwd_vs_oracle(case):
    B, S, D, r, Hq, Hkv, dh = case
    _note(f"bwd {case}")
    q, k, v = workloads.make_custom(B, S, D, Hq, Hkv, dh, torch.bfloat16, seed=91)
    dout = workloads.make_grad(q.shape, 95, torch.bfloat16)
    dq, dk, dv, delta = run_bwd(q, k, v, dout, D, r)
    rq, rk, rv = oracle.causal_attention_backward(q, k, v, dout, D, r)
    wq = check_grad("dq", _np(dq), rq, 2)
    wk = check_grad("dk", _np(dk), rk, 2)
    wv = check_grad("dv", _np(dv), rv, 2)
    ro, _ = oracle.causal_attention(q, k, v, D, r)
    rdelta = np.einsum("bihd,bihd->bhi", ro, _np(dout))
    assert np.abs(_np(delta) - rdelta).max() <= 2.0 ** -7 * max(1.0, np.abs(rdelta).max())
    _note(f"worst scaled max-abs / relative errors: dq {wq}, dk {wk}, dv {wv}")


def test_bwd_workload_sampled_heads():
    """The 7B shard at its full size (32K tokens, rank 3 of 8): every row and key of two
    KV heads against the oracle."""
    w = workloads.BY_NAME["tsp_7b_shard_s32k"]
    r = w.ranks[0]
    _note(f"bwd workload {w.name}")
    q, k, v = workloads.make_inputs(w, r)
    dout = workloads.make_grad(q.shape, 97, torch.bfloat16)
    dq, dk, dv, _ = run_bwd(q, k, v, dout, w.D, r)
    heads = [0, w.Hkv - 1]
    rq, rk, rv = oracle.causal_attention_backward(q, k, v, dout, w.D, r, kv_heads=heads)
    grp = w.Hq // w.Hkv
    qh = [hk * grp + g for hk in heads for g in range(grp)]
    check_grad("dq", _np(dq[:, :, qh]), rq, 2)
    check_grad("dk", _np(dk[:, :, heads]), rk, 2)
    check_grad("dv", _np(dv[:, :, heads]), rv, 2)


def test_bwd_gqa_full_size_one_query_head():
    """The GQA dh-256 shard at full size (16384 local rows, 65536 keys, rank 2 of 4), dout
    zero on every query head but head 7 (the second of KV head 1's group). Every other
    head's dS is then 0, so head 7's dq (every row) and KV head 1's dk and dv (every key)
    are the gradients of a one-head problem, which the oracle computes in full; the other
    query heads' dq and the other KV heads' dk and dv must be exactly 0."""
    w = workloads.BY_NAME["gqa_shard_s64k"]
    r = w.ranks[0]
    grp = w.Hq // w.Hkv
    h, hk = grp + 1, 1
    _note(f"bwd one query head {w.name} head {h}")
    q, k, v = workloads.make_inputs(w, r)
    dout = workloads.make_grad(q.shape, 96, torch.bfloat16)
    keep = torch.zeros(w.Hq, dtype=torch.bool)
    keep[h] = True
    dout[:, :, ~keep] = 0
    dq, dk, dv, _ = run_bwd(q, k, v, dout, w.D, r)
    others = [x for x in range(w.Hkv) if x != hk]
    assert (dq[:, :, ~keep.to(DEV)] == 0).all()
    assert (dk[:, :, others] == 0).all() and (dv[:, :, others] == 0).all()
    rq, rk, rv = oracle.causal_attention_backward(q[:, :, [h]], k[:, :, [hk]], v[:, :, [hk]], dout[:, :, [h]], w.D, r)
    wq = check_grad("dq", _np(dq[:, :, [h]]), rq, 2)
    wk = check_grad("dk", _np(dk[:, :, [hk]]), rk, 2)
    wv = check_grad("dv", _np(dv[:, :, [hk]]), rv, 2)
    _note(f"worst scaled max-abs / relative errors: dq {wq}, dk {wk}, dv {wv}")


def test_bwd_ulysses_full_size_last_rows_of_one_head():
    """The Ulysses shard at full size (D = 1, 131072 queries and keys, dh 128), dout zero
    except on the last 4096 rows of query head 1. Every other row's dS is then 0, so the
    gradients are those of the oracle restricted to those rows: dq of those rows, and dk
    and dv of KV head 1 over all 131072 keys. All other dq rows and the other KV heads'
    dk and dv must be exactly 0."""
    w = workloads.BY_NAME["ulysses_head_subset_s128k"]
    r = w.ranks[0]
    h, n_rows = 1, 4096
    hk = h // (w.Hq // w.Hkv)
    _note(f"bwd last rows {w.name} head {h}")
    q, k, v = workloads.make_inputs(w, r)
    dout = workloads.make_grad(q.shape, 94, torch.bfloat16)
    keep = torch.zeros(w.S_local, w.Hq, dtype=torch.bool)
    keep[w.S_local - n_rows:, h] = True
    dout[:, ~keep] = 0
    dq, dk, dv, _ = run_bwd(q, k, v, dout, w.D, r)
    others = [x for x in range(w.Hkv) if x != hk]
    assert (dq[:, ~keep.to(DEV)] == 0).all()
    assert (dk[:, :, others] == 0).all() and (dv[:, :, others] == 0).all()
    rows = np.arange(w.S_local - n_rows, w.S_local)
    rq, rk, rv = oracle.causal_attention_backward(q[:, :, [h]], k[:, :, [hk]], v[:, :, [hk]], dout[:, :, [h]],
                                                  w.D, r, rows=rows)
    wq = check_grad("dq", _np(dq[:, w.S_local - n_rows:, [h]]), rq[:, w.S_local - n_rows:], 2)
    wk = check_grad("dk", _np(dk[:, :, [hk]]), rk, 2)
    wv = check_grad("dv", _np(dv[:, :, [hk]]), rv, 2)
    _note(f"worst scaled max-abs / relative errors: dq {wq}, dk {wk}, dv {wv}")


@pytest.mark.parametrize("name", ["gqa_shard_s64k", "ulysses_head_subset_s128k", "tsp_7b_shard_s32k"])
def test_bwd_closed_form_sums_full_size(name):
    """At full size, for every KV head: dK sums to 0 over the keys and dV sums to the
    group's total dout (softmax rows sum to 1); keys past the rank's last position are 0.
    Covers the one-wave dh-256 kernel (GQA shard) and the two-wave one-launch dK/dV kernel
    at D = 1 (Ulysses shard, 131072 keys) and on the 7B shard."""
    w = workloads.BY_NAME[name]
    r = w.ranks[0]
    _note(f"bwd sums {w.name}")
    q, k, v = workloads.make_inputs(w, r)
    dout = workloads.make_grad(q.shape, 98, torch.bfloat16)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, dout))
    out, lse = tsp.fwd(qd, kd, vd, D=w.D, rank=r)
    dk = torch.full_like(kd, float("nan"))
    dv = torch.full_like(vd, float("nan"))
    tsp.bwd(qd, kd, vd, out, lse, dod, D=w.D, rank=r, dk=dk, dv=dv)
    torch.cuda.synchronize()
    need = (2 * w.D - r) * w.C
    assert torch.isfinite(dk).all() and torch.isfinite(dv).all()
    assert (dk[:, need:] == 0).all() and (dv[:, need:] == 0).all()
    grp = w.Hq // w.Hkv
    sk = dk.double().sum(dim=1)                       # [B, Hkv, dh]
    sv = dv.double().sum(dim=1)
    tot = dod.double().reshape(w.B, w.S_local, w.Hkv, grp, w.dh).sum(dim=(1, 3))
    absk = dk.double().abs().sum(dim=1)
    # each bf16 output carries a rounding error <= 2^-9 of its magnitude
    assert ((sk.abs() <= 2.0 ** -8 * absk + 1e-3)).all(), (sk.abs().max(), absk.max())
    assert ((sv - tot).abs() <= 2.0 ** -8 * dv.double().abs().sum(dim=1) + 1e-2).all()


def test_bwd_deterministic_and_zero_dout():
    _note("bwd determinism")
    q, k, v = workloads.make_custom(1, 2048, 8, 4, 2, 128, torch.bfloat16, seed=7)
    dout = workloads.make_grad(q.shape, 8, torch.bfloat16)
    a = run_bwd(q, k, v, dout, 8, 5)
    b = run_bwd(q, k, v, dout, 8, 5)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    z = run_bwd(q, k, v, torch.zeros_like(dout), 8, 5)
    for x in z:
        assert (x == 0).all()


def test_bwd_writes_only_its_outputs():
    _note("bwd canaries")
    q, k, v = workloads.make_custom(1, 1200, 3, 6, 2, 128, torch.bfloat16, seed=12)
    dout = workloads.make_grad(q.shape, 13, torch.bfloat16)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, dout))
    out, lse = tsp.fwd(qd, kd, vd, D=3, rank=1)
    bufs = {}
    for name, like in (("dq", qd), ("dk", kd), ("dv", vd), ("delta", lse)):
        big = torch.full((like.numel() + 256,), 3.0, dtype=like.dtype, device=DEV)
        bufs[name] = (big, big[:like.numel()].view_as(like))
    ins = [t.clone() for t in (qd, kd, vd, out, lse, dod)]
    tsp.bwd(qd, kd, vd, out, lse, dod, D=3, rank=1, dq=bufs["dq"][1], dk=bufs["dk"][1], dv=bufs["dv"][1],
            delta=bufs["delta"][1])
    torch.cuda.synchronize()
    for name, (big, view) in bufs.items():
        assert (big[view.numel():] == 3).all(), name
    for a, b in zip(ins, (qd, kd, vd, out, lse, dod)):
        assert torch.equal(a, b)


F32_CASES = [  # (B, S_total, D, rank, Hq, Hkv, dh): the tiny zigzag GQA shard and ragged fp32 shapes
    (1, 512, 4, 1, 4, 1, 64),
    (1, 512, 4, 0, 4, 1, 64),
    (1, 600, 3, 1, 2, 1, 128),
    (1, 288, 2, 1, 4, 2, 256),
    (2, 96, 1, 0, 3, 1, 128),
    (1, 8, 4, 3, 2, 1, 64),
]


@pytest.mark.parametrize("case", F32_CASES, ids=lambda c: "B{}_S{}_D{}_r{}_H{}x{}_d{}".format(*c))
def test_bwd_f32_vs_oracle(case):
    """fp32 end to end: within 1e-4 of the oracle (relative to the largest gradient, at
    least 1), and a relative Frobenius error below 1e-5."""
    B, S, D, r, Hq, Hkv, dh = case
    _note(f"bwd f32 {case}")
    q, k, v = workloads.make_custom(B, S, D, Hq, Hkv, dh, torch.float32, seed=61)
    dout = workloads.make_grad(q.shape, 62, torch.float32)
    dq, dk, dv, delta = run_bwd(q, k, v, dout, D, r)
    rq, rk, rv = oracle.causal_attention_backward(q, k, v, dout, D, r)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        g = _np(got)
        err = np.abs(g - ref).max()
        assert err <= 1e-4 * max(1.0, np.abs(ref).max()), (name, err)
        assert np.linalg.norm(g - ref) <= 1e-5 * max(np.linalg.norm(ref), 1e-30), name
    ro, _ = oracle.causal_attention(q, k, v, D, r)
    rdelta = np.einsum("bihd,bihd->bhi", ro, _np(dout))
    assert np.abs(_np(delta) - rdelta).max() <= 1e-4 * max(1.0, np.abs(rdelta).max())
