"""Key-range attention and the log-sum-exp merge (tsp_attn_fwd_range, tsp_attn_merge) vs
the fp64 oracle, through the C ABI, on an MI355X (gfx950).

A rank that overlaps the K/V all-gather with compute attends to each gathered chunk as it
arrives and merges the partials; the result must equal attention over the full K/V.
Tolerances as in the full-path parity tests: max-abs 2e-2 (bf16) / 1e-4 (fp32) on out and
lse, plus a relative Frobenius bound of 1e-2 for bf16. Rows with no visible key in the
range must come back exactly as out = 0, lse = -inf.
"""

import numpy as np
import pytest
import torch

import oracle
import sequence_causal_attention_amd as tsp
import workloads

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}
DEV = "cuda:0"


def _note(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def check_partial(out, lse, ref_out, ref_lse, dtype):
    """Exact empties, then the tolerance on every row with a visible key."""
    tol = TOL[dtype]
    empty = np.isneginf(ref_lse)  # [B, Hq, rows]
    assert np.array_equal(np.isneginf(lse), empty), "empty rows differ"
    e_rows = empty.transpose(0, 2, 1)  # [B, rows, Hq]
    assert (out[e_rows] == 0).all(), "an empty row has a nonzero output"
    assert np.isfinite(out).all()
    if (~empty).any():
        err_l = np.abs(lse[~empty] - ref_lse[~empty]).max()
        assert err_l <= tol, f"max |lse - ref| = {err_l:.3g}"
    err_o = np.abs(out - ref_out).max()
    assert err_o <= tol, f"max |out - ref| = {err_o:.3g}"
    if dtype == torch.bfloat16 and (~e_rows).any():
        d = (out - ref_out)[~e_rows]
        rel = np.linalg.norm(d) / max(np.linalg.norm(ref_out[~e_rows]), 1e-30)
        assert rel <= 1e-2, f"relative error {rel:.3g}"


RANGE_CASES = [  # (B, S_total, D, rank, Hq, Hkv, dh, dtype, kv_begin, kv_end)
    (1, 2048, 8, 3, 4, 4, 128, torch.bfloat16, 0, 2048),      # whole range
    (1, 2048, 8, 3, 4, 4, 128, torch.bfloat16, 384, 512),     # one aligned gathered chunk
    (1, 2048, 8, 3, 4, 4, 128, torch.bfloat16, 100, 1700),    # unaligned both ends
    (1, 2048, 8, 3, 4, 4, 128, torch.bfloat16, 1600, 1700),   # only the second chunk sees it
    (1, 2048, 8, 3, 4, 4, 128, torch.bfloat16, 1900, 2048),   # beyond every position: empty
    (1, 2048, 8, 3, 4, 4, 128, torch.bfloat16, 700, 700),     # empty range
    (1, 2048, 8, 3, 4, 4, 128, torch.bfloat16, 417, 418),     # a single key
    (1, 2048, 8, 0, 4, 4, 128, torch.bfloat16, 33, 95),       # inside the first chunk's diagonal
    (1, 4096, 4, 2, 12, 2, 256, torch.bfloat16, 1000, 2600),  # GQA, dh 256
    (1, 1024, 2, 1, 8, 2, 64, torch.bfloat16, 250, 777),      # dh 64
    (1, 1200, 3, 2, 6, 2, 128, torch.bfloat16, 399, 801),     # ragged chunks
    (1, 4096, 1, 0, 4, 4, 128, torch.bfloat16, 1024, 3000),   # D = 1
    (2, 1024, 4, 1, 4, 2, 128, torch.bfloat16, 128, 896),     # batch of 2
    (1, 512, 4, 1, 4, 1, 64, torch.float32, 64, 448),         # fp32
    (1, 600, 3, 1, 2, 1, 128, torch.float32, 37, 451),        # fp32 ragged, unaligned
    (1, 288, 2, 1, 4, 2, 256, torch.float32, 100, 101),       # fp32 single key
    (1, 512, 4, 1, 4, 1, 64, torch.float32, 300, 300),        # fp32 empty range
    # a wave whose rows are partly empty (row 32 sees none of keys 33..94, row 33 does):
    # the running-max update must leave the empty rows at zero
    (1, 512, 4, 0, 4, 1, 64, torch.float32, 33, 95),
    (1, 1024, 2, 0, 8, 2, 64, torch.bfloat16, 45, 46),
    # dh 128: ranges shorter than 8192 keys run the two-wave kernel, longer ones the
    # one-wave kernel; both sides of that switch, and a long unaligned range
    (1, 16384, 8, 6, 2, 2, 128, torch.bfloat16, 0, 8191),
    (1, 16384, 8, 6, 2, 2, 128, torch.bfloat16, 0, 8192),
    (1, 16384, 8, 1, 2, 2, 128, torch.bfloat16, 3000, 16000),
]


@pytest.mark.parametrize("case", RANGE_CASES,
                         ids=lambda c: "B{}_S{}_D{}_r{}_H{}x{}_d{}_{}_{}-{}".format(*c[:7], str(c[7])[6:], *c[8:]))
def test_range_vs_oracle(case):
    B, S, D, r, Hq, Hkv, dh, dtype, lo, hi = case
    _note(f"range {case}")
    q, k, v = workloads.make_custom(B, S, D, Hq, Hkv, dh, dtype, seed=11)
    out, lse = tsp.fwd(q.to(DEV), k.to(DEV), v.to(DEV), D=D, rank=r, kv_range=(lo, hi))
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.causal_attention_range(q, k, v, D, r, lo, hi)
    check_partial(_np(out), _np(lse), ref_out, ref_lse, dtype)


def test_full_range_is_bitwise_fwd():
    _note("full range == fwd")
    q, k, v = workloads.make_custom(1, 2048, 8, 4, 4, 128, torch.bfloat16, seed=5)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o1, l1 = tsp.fwd(qd, kd, vd, D=8, rank=3)
    o2, l2 = tsp.fwd(qd, kd, vd, D=8, rank=3, kv_range=(0, 2048))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def _chunk_pipeline(qd, kd, vd, D, r, bounds, fused):
    """Attend to each key chunk in turn and fold it into a running (out, lse): in the
    kernel's epilogue (fused) or with a separate merge launch."""
    acc_o = acc_l = None
    part_o, part_l = torch.empty_like(qd), None
    for lo, hi in bounds:
        if acc_o is None:
            acc_o, acc_l = tsp.fwd(qd, kd, vd, D=D, rank=r, kv_range=(lo, hi))
            part_l = torch.empty_like(acc_l)
        elif fused:
            tsp.fwd(qd, kd, vd, D=D, rank=r, kv_range=(lo, hi), out=acc_o, lse=acc_l, accumulate=True)
        else:
            tsp.fwd(qd, kd, vd, D=D, rank=r, kv_range=(lo, hi), out=part_o, lse=part_l)
            tsp.merge(acc_o, acc_l, part_o, part_l, out=acc_o, lse=acc_l)
    torch.cuda.synchronize()
    return acc_o, acc_l


PIPE_CASES = [  # (B, S_total, D, rank, Hq, Hkv, dh, dtype, order)
    (1, 2048, 8, 3, 4, 4, 128, torch.bfloat16, "ring"),     # arrival order of a ring from rank r
    (1, 2048, 8, 0, 4, 4, 128, torch.bfloat16, "natural"),
    (1, 2048, 8, 7, 4, 4, 128, torch.bfloat16, "reverse"),
    (1, 4096, 4, 2, 12, 2, 256, torch.bfloat16, "ring"),
    (1, 1024, 2, 1, 8, 2, 64, torch.bfloat16, "ring"),
    (1, 1200, 3, 2, 6, 2, 128, torch.bfloat16, "ring"),     # ragged: chunks of 200 keys
    (1, 512, 4, 1, 4, 1, 64, torch.float32, "ring"),
    (1, 600, 3, 1, 2, 1, 128, torch.float32, "reverse"),
]


def _bounds(S, D, r, order):
    C = S // (2 * D)
    chunks = list(range(2 * D))
    if order == "ring":  # own pair first, then the pair (p, 2D-1-p) of peer p = r-1, r-2, ...
        chunks = [c for p in ((r - s) % D for s in range(D)) for c in (p, 2 * D - 1 - p)]
    elif order == "reverse":
        chunks = chunks[::-1]
    return [(c * C, (c + 1) * C) for c in chunks]


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "merge"])
@pytest.mark.parametrize("case", PIPE_CASES,
                         ids=lambda c: "B{}_S{}_D{}_r{}_H{}x{}_d{}_{}_{}".format(*c[:7], str(c[7])[6:], c[8]))
def test_chunk_pipeline_merge(case, fused):
    B, S, D, r, Hq, Hkv, dh, dtype, order = case
    _note(f"pipeline {case} fused={fused}")
    q, k, v = workloads.make_custom(B, S, D, Hq, Hkv, dh, dtype, seed=23)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    bounds = _bounds(S, D, r, order)
    assert sorted(bounds) == [(c * (S // (2 * D)), (c + 1) * (S // (2 * D))) for c in range(2 * D)]
    o, l = _chunk_pipeline(qd, kd, vd, D, r, bounds, fused)
    ref_out, ref_lse = oracle.causal_attention(q, k, v, D, r)
    out, lse = _np(o), _np(l)
    assert np.isfinite(lse).all()
    check_partial(out, lse, ref_out, ref_lse, dtype)
    # and against the single-launch kernel
    of, lf = tsp.fwd(qd, kd, vd, D=D, rank=r)
    torch.cuda.synchronize()
    assert np.abs(out - _np(of)).max() <= TOL[dtype]
    # bf16: each form sums weights rounded to bf16 (relative error <= 2^-9 per weight), so
    # each lse is within 2^-9 of exact and the two within 2^-8 of each other
    assert np.abs(lse - _np(lf)).max() <= (2.0 ** -8 if dtype == torch.bfloat16 else 1e-5)


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "merge"])
def test_chunk_pipeline_workload_sampled(fused):
    """The 7B shard at its full size, gathered in 16 chunks, on sampled rows."""
    w = workloads.BY_NAME["tsp_7b_shard_s32k"]
    r = w.ranks[0]
    _note(f"pipeline workload {w.name} rank {r} fused={fused}")
    q, k, v = workloads.make_inputs(w, r)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o, l = _chunk_pipeline(qd, kd, vd, w.D, r, _bounds(w.S_total, w.D, r, "ring"), fused)
    C = w.S_total // (2 * w.D)
    rows = np.concatenate([np.arange(0, 48), np.arange(C - 16, C + 32), np.arange(2 * C - 16, 2 * C)])
    heads = [0, 17, 31]
    ref_out, ref_lse = oracle.causal_attention(q, k, v, w.D, r, rows=rows, heads=heads)
    idx = torch.as_tensor(rows, device=DEV)
    hidx = torch.as_tensor(heads, device=DEV)
    out = _np(o.index_select(1, idx).index_select(2, hidx))
    lse = _np(l.index_select(1, hidx).index_select(2, idx))
    check_partial(out, lse, ref_out, ref_lse, w.torch_dtype())


ACC_CASES = [  # (B, S_total, D, rank, Hq, Hkv, dh, dtype, first range, second range)
    (1, 2048, 8, 3, 4, 4, 128, torch.bfloat16, (0, 700), (700, 1800)),
    (1, 2048, 8, 0, 4, 4, 128, torch.bfloat16, (60, 100), (0, 60)),       # first leaves rows empty
    (1, 2048, 8, 3, 4, 4, 128, torch.bfloat16, (1900, 2048), (100, 900)),  # first is empty for all
    (1, 4096, 4, 2, 12, 2, 256, torch.bfloat16, (2000, 4096), (0, 2000)),
    (1, 1024, 2, 1, 8, 2, 64, torch.bfloat16, (300, 301), (0, 300)),
    (1, 600, 3, 1, 2, 1, 128, torch.float32, (37, 451), (451, 600)),
    (1, 512, 4, 0, 4, 1, 64, torch.float32, (33, 95), (0, 33)),
]


@pytest.mark.parametrize("case", ACC_CASES, ids=lambda c: "S{}_D{}_r{}_d{}_{}_{}_{}".format(
    c[1], c[2], c[3], c[6], str(c[7])[6:], *c[8:]))
def test_accumulate_matches_oracle_merge(case):
    """A range launch with accumulate=1 on top of another range's result equals the
    oracle's merge of the two partials (empty rows: untouched / exact)."""
    B, S, D, r, Hq, Hkv, dh, dtype, ra, rb = case
    _note(f"accumulate {case}")
    q, k, v = workloads.make_custom(B, S, D, Hq, Hkv, dh, dtype, seed=31)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o, l = tsp.fwd(qd, kd, vd, D=D, rank=r, kv_range=ra)
    tsp.fwd(qd, kd, vd, D=D, rank=r, kv_range=rb, out=o, lse=l, accumulate=True)
    torch.cuda.synchronize()
    oa, la = oracle.causal_attention_range(q, k, v, D, r, *ra)
    ob, lb = oracle.causal_attention_range(q, k, v, D, r, *rb)
    ref_o, ref_l = oracle.merge_partials(oa, la, ob, lb)
    check_partial(_np(o), _np(l), ref_o, ref_l, dtype)


def test_accumulate_needs_running_result():
    q, k, v = workloads.make_custom(1, 512, 4, 4, 1, 64, torch.bfloat16, seed=3)
    with pytest.raises(tsp.TspAttnError):
        tsp.fwd(q.to(DEV), k.to(DEV), v.to(DEV), D=4, rank=1, kv_range=(0, 64), accumulate=True)


MERGE_CASES = [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.bfloat16, 256), (torch.float32, 64),
               (torch.float32, 128), (torch.float32, 256)]


def _merge_inputs(dtype, dh, B=2, S_local=96, Hq=3, seed=7):
    g = torch.Generator().manual_seed(seed)
    oa = torch.randn(B, S_local, Hq, dh, generator=g).to(dtype)
    ob = torch.randn(B, S_local, Hq, dh, generator=g).to(dtype)
    la = torch.randn(B, Hq, S_local, generator=g) * 4
    lb = torch.randn(B, Hq, S_local, generator=g) * 4
    # empties: a alone, b alone, both; a huge lse gap
    la[0, 0, :10] = -float("inf")
    lb[0, 1, 5:15] = -float("inf")
    la[1, 2, 20:30] = -float("inf")
    lb[1, 2, 20:30] = -float("inf")
    la[1, 0, 40:50] = 80.0
    lb[1, 0, 40:50] = -80.0
    # an empty partial comes back as out = 0
    oa.permute(0, 2, 1, 3)[torch.isneginf(la)] = 0
    ob.permute(0, 2, 1, 3)[torch.isneginf(lb)] = 0
    return oa, la, ob, lb


@pytest.mark.parametrize("dtype,dh", MERGE_CASES, ids=lambda x: str(x))
@pytest.mark.parametrize("inplace", [False, True])
def test_merge_vs_oracle(dtype, dh, inplace):
    _note(f"merge {dtype} dh{dh} inplace={inplace}")
    oa, la, ob, lb = _merge_inputs(dtype, dh)
    ref_o, ref_l = oracle.merge_partials(oa, la, ob, lb)
    a_o, a_l, b_o, b_l = (t.to(DEV) for t in (oa, la, ob, lb))
    if inplace:
        o, l = tsp.merge(a_o, a_l, b_o, b_l, out=a_o, lse=a_l)
        assert o.data_ptr() == a_o.data_ptr()
    else:
        o, l = tsp.merge(a_o, a_l, b_o, b_l)
    torch.cuda.synchronize()
    out, lse = _np(o), _np(l)
    both = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(lse), both)
    assert (out[both.transpose(0, 2, 1)] == 0).all()
    assert np.abs(lse[~both] - ref_l[~both]).max() <= 1e-5
    # bf16: one rounding of a convex combination of bf16 values
    tol = 1e-5 if dtype == torch.float32 else 2 ** -8 * np.abs(ref_o).max()
    assert np.abs(out - ref_o).max() <= tol


def test_merge_inputs_untouched_and_canaries():
    _note("merge canaries")
    oa, la, ob, lb = _merge_inputs(torch.bfloat16, 128)
    a_o, a_l, b_o, b_l = (t.to(DEV) for t in (oa, la, ob, lb))
    big = torch.full((a_o.numel() + 64,), 7.0, dtype=a_o.dtype, device=DEV)
    out = big[:a_o.numel()].view_as(a_o)
    bigl = torch.full((a_l.numel() + 64,), 7.0, device=DEV)
    lse = bigl[:a_l.numel()].view_as(a_l)
    tsp.merge(a_o, a_l, b_o, b_l, out=out, lse=lse)
    torch.cuda.synchronize()
    assert (big[a_o.numel():] == 7).all() and (bigl[a_l.numel():] == 7).all()
    assert torch.equal(a_o.cpu(), oa) and torch.equal(b_l.cpu(), lb)


def test_range_invalid_arguments_write_nothing():
    _note("range invalid")
    q, k, v = workloads.make_custom(1, 512, 4, 4, 1, 64, torch.bfloat16, seed=3)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.full_like(qd, 5.0)
    lse = torch.full((1, 4, 128), 5.0, device=DEV)
    for lo, hi in [(10, 9), (-1, 5), (0, 513), (600, 700)]:
        with pytest.raises(tsp.TspAttnError) as ei:
            tsp.fwd(qd, kd, vd, D=4, rank=1, kv_range=(lo, hi), out=out, lse=lse)
        assert ei.value.status == tsp.TSP_EINVAL
    torch.cuda.synchronize()
    assert (out == 5).all() and (lse == 5).all()


RANGE2_CASES = [  # (B, S_total, D, rank, Hq, Hkv, dh, dtype, first range, second range)
    (1, 2048, 8, 3, 4, 4, 128, torch.bfloat16, (128, 256), (1792, 1920)),   # peer 1's two chunks
    (1, 2048, 8, 3, 4, 4, 128, torch.bfloat16, (384, 512), (1536, 1664)),   # own two chunks
    (1, 2048, 8, 3, 4, 4, 128, torch.bfloat16, (100, 700), (700, 1800)),    # adjacent, unaligned
    (1, 2048, 8, 3, 4, 4, 128, torch.bfloat16, (1900, 2000), (2000, 2048)),  # empty for every row
    (1, 2048, 8, 3, 4, 4, 128, torch.bfloat16, (0, 60), (1600, 1700)),      # second: 2nd chunk only
    (1, 2048, 8, 0, 4, 4, 128, torch.bfloat16, (33, 95), (95, 95)),         # empty second range
    (1, 2048, 8, 0, 4, 4, 128, torch.bfloat16, (33, 33), (60, 1000)),       # empty first range
    (1, 2048, 8, 0, 4, 4, 128, torch.bfloat16, (1, 2), (40, 41)),           # one key each
    (1, 4096, 4, 2, 12, 2, 256, torch.bfloat16, (512, 1024), (3072, 3584)),  # GQA, dh 256
    (1, 1024, 2, 1, 8, 2, 64, torch.bfloat16, (256, 512), (512, 768)),      # dh 64
    (1, 1200, 3, 2, 6, 2, 128, torch.bfloat16, (0, 200), (1000, 1200)),     # ragged chunks
    (2, 1024, 4, 1, 4, 2, 128, torch.bfloat16, (128, 256), (768, 896)),     # batch of 2
    (1, 4096, 1, 0, 4, 4, 128, torch.bfloat16, (17, 1000), (2000, 3001)),   # D = 1
    (1, 2048, 8, 3, 4, 4, 128, torch.bfloat16, (100, 650), (700, 1650)),   # unaligned, with a gap
    (1, 2048, 8, 3, 4, 4, 128, torch.bfloat16, (0, 640), (704, 1664)),     # unmasked run into the second
    (1, 2048, 8, 5, 4, 4, 128, torch.bfloat16, (320, 384), (1280, 1408)),  # peer 2's chunks
    (1, 1024, 2, 1, 8, 2, 64, torch.bfloat16, (64, 300), (400, 700)),      # dh 64, unaligned
    (1, 4096, 4, 2, 12, 2, 256, torch.bfloat16, (77, 1500), (2100, 3333)),  # dh 256, unaligned
    (1, 512, 4, 1, 4, 1, 64, torch.float32, (0, 64), (448, 512)),           # fp32
    (1, 600, 3, 1, 2, 1, 128, torch.float32, (37, 100), (451, 600)),        # fp32 ragged
]


def _base_range(S, lo, hi2):
    """Keys outside both ranges, for the running result that an accumulating call adds to."""
    return (hi2, S) if hi2 < S else (0, lo)


@pytest.mark.parametrize("accumulate", [False, True], ids=["write", "accumulate"])
@pytest.mark.parametrize("case", RANGE2_CASES, ids=lambda c: "B{}_S{}_D{}_r{}_d{}_{}_{}_{}".format(
    *c[:4], c[6], str(c[7])[6:], *c[8:]))
def test_two_ranges_match_oracle_merge(case, accumulate):
    """One call over two key ranges equals the oracle's merge of the two range partials
    (and, accumulating, of those and the running result's range)."""
    B, S, D, r, Hq, Hkv, dh, dtype, ra, rb = case
    _note(f"two ranges {case} accumulate={accumulate}")
    q, k, v = workloads.make_custom(B, S, D, Hq, Hkv, dh, dtype, seed=41)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    oa, la = oracle.causal_attention_range(q, k, v, D, r, *ra)
    ob, lb = oracle.causal_attention_range(q, k, v, D, r, *rb)
    ref_o, ref_l = oracle.merge_partials(oa, la, ob, lb)
    if accumulate:
        base = _base_range(S, ra[0], rb[1])
        o, l = tsp.fwd(qd, kd, vd, D=D, rank=r, kv_range=base)
        tsp.fwd(qd, kd, vd, D=D, rank=r, kv_range=ra, kv_range2=rb, out=o, lse=l, accumulate=True)
        oc, lc = oracle.causal_attention_range(q, k, v, D, r, *base)
        ref_o, ref_l = oracle.merge_partials(oc, lc, ref_o, ref_l)
    else:
        o, l = tsp.fwd(qd, kd, vd, D=D, rank=r, kv_range=ra, kv_range2=rb)
    torch.cuda.synchronize()
    check_partial(_np(o), _np(l), ref_o, ref_l, dtype)


def test_two_ranges_covering_all_keys_match_fwd():
    """Two ranges that split the keys give the single launch's result to rounding."""
    _note("two ranges == fwd")
    q, k, v = workloads.make_custom(1, 2048, 8, 4, 4, 128, torch.bfloat16, seed=5)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o1, l1 = tsp.fwd(qd, kd, vd, D=8, rank=3)
    o2, l2 = tsp.fwd(qd, kd, vd, D=8, rank=3, kv_range=(0, 1000), kv_range2=(1000, 2048))
    torch.cuda.synchronize()
    # the same sweep over the same keys: only the stage boundary at 1000 differs
    assert (o1.float() - o2.float()).abs().max().item() <= TOL[torch.bfloat16]
    assert (l1 - l2).abs().max().item() <= 2.0 ** -8


def _pair_pipeline(qd, kd, vd, D, r, C):
    """One call per step of a ring all-gather: the rank's own two chunks first, then the
    two chunks of each peer (r-1, r-2, ... mod D) in arrival order, accumulated."""
    acc_o = acc_l = None
    for s in range(D):
        p = (r - s) % D
        ra, rb = (p * C, (p + 1) * C), ((2 * D - 1 - p) * C, (2 * D - p) * C)
        if acc_o is None:
            acc_o, acc_l = tsp.fwd(qd, kd, vd, D=D, rank=r, kv_range=ra, kv_range2=rb)
        else:
            tsp.fwd(qd, kd, vd, D=D, rank=r, kv_range=ra, kv_range2=rb, out=acc_o, lse=acc_l, accumulate=True)
    torch.cuda.synchronize()
    return acc_o, acc_l


PAIR_CASES = [  # (B, S_total, D, rank, Hq, Hkv, dh, dtype)
    (1, 2048, 8, 3, 4, 4, 128, torch.bfloat16),
    (1, 2048, 8, 0, 4, 4, 128, torch.bfloat16),
    (1, 2048, 8, 7, 4, 4, 128, torch.bfloat16),
    (1, 4096, 4, 2, 12, 2, 256, torch.bfloat16),
    (1, 1024, 2, 1, 8, 2, 64, torch.bfloat16),
    (1, 1200, 3, 2, 6, 2, 128, torch.bfloat16),   # ragged: chunks of 200 keys
    (1, 512, 4, 1, 4, 1, 64, torch.float32),
]


@pytest.mark.parametrize("case", PAIR_CASES, ids=lambda c: "B{}_S{}_D{}_r{}_H{}x{}_d{}_{}".format(
    *c[:7], str(c[7])[6:]))
def test_ring_pair_pipeline(case):
    B, S, D, r, Hq, Hkv, dh, dtype = case
    _note(f"pair pipeline {case}")
    q, k, v = workloads.make_custom(B, S, D, Hq, Hkv, dh, dtype, seed=43)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o, l = _pair_pipeline(qd, kd, vd, D, r, S // (2 * D))
    ref_out, ref_lse = oracle.causal_attention(q, k, v, D, r)
    out, lse = _np(o), _np(l)
    assert np.isfinite(lse).all()
    check_partial(out, lse, ref_out, ref_lse, dtype)
    of, lf = tsp.fwd(qd, kd, vd, D=D, rank=r)
    torch.cuda.synchronize()
    assert np.abs(out - _np(of)).max() <= TOL[dtype]
    assert np.abs(lse - _np(lf)).max() <= (2.0 ** -8 if dtype == torch.bfloat16 else 1e-5)


def test_ring_pair_pipeline_workload_sampled():
    """The 7B shard at its full size, one call per ring step, on sampled rows."""
    w = workloads.BY_NAME["tsp_7b_shard_s32k"]
    r = w.ranks[0]
    _note(f"pair pipeline workload {w.name} rank {r}")
    q, k, v = workloads.make_inputs(w, r)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    C = w.S_total // (2 * w.D)
    o, l = _pair_pipeline(qd, kd, vd, w.D, r, C)
    rows = np.concatenate([np.arange(0, 48), np.arange(C - 16, C + 32), np.arange(2 * C - 16, 2 * C)])
    heads = [0, 17, 31]
    ref_out, ref_lse = oracle.causal_attention(q, k, v, w.D, r, rows=rows, heads=heads)
    idx = torch.as_tensor(rows, device=DEV)
    hidx = torch.as_tensor(heads, device=DEV)
    out = _np(o.index_select(1, idx).index_select(2, hidx))
    lse = _np(l.index_select(1, hidx).index_select(2, idx))
    check_partial(out, lse, ref_out, ref_lse, w.torch_dtype())


def test_two_ranges_invalid_write_nothing():
    _note("two ranges invalid")
    q, k, v = workloads.make_custom(1, 512, 4, 4, 1, 64, torch.bfloat16, seed=3)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.full_like(qd, 5.0)
    lse = torch.full((1, 4, 128), 5.0, device=DEV)
    for ra, rb in [((0, 100), (50, 200)), ((0, 100), (300, 200)), ((0, 100), (400, 513)),
                   ((100, 200), (0, 50))]:
        with pytest.raises(tsp.TspAttnError) as ei:
            tsp.fwd(qd, kd, vd, D=4, rank=1, kv_range=ra, kv_range2=rb, out=out, lse=lse)
        assert ei.value.status == tsp.TSP_EINVAL
    torch.cuda.synchronize()
    assert (out == 5).all() and (lse == 5).all()


FOLD_CASES = [  # (rank, first, second, the one range it equals); S_total 2048, D 8, C 128
    (3, (0, 128), (1920, 2048), (0, 128)),        # second past every position (peer 0 of rank 3)
    (3, (896, 1024), (1024, 1152), (896, 1152)),  # adjacent chunks 7 and 8 (peer 7 of rank 3)
    (3, (1700, 1800), (1800, 1900), (2048, 2048)),  # both past every position: nothing visible
    (0, (0, 0), (100, 300), (100, 300)),          # empty first range
]


@pytest.mark.parametrize("accumulate", [False, True], ids=["write", "accumulate"])
@pytest.mark.parametrize("case", FOLD_CASES, ids=lambda c: f"r{c[0]}_{c[1]}_{c[2]}")
def test_two_ranges_that_fold_to_one_are_bitwise_one_range(case, accumulate):
    """Ranges clipped at the rank's last position, an empty first range and adjacent ranges
    run as one range: the result is the one-range call's, bit for bit."""
    r, ra, rb, one = case
    _note(f"fold {case} accumulate={accumulate}")
    q, k, v = workloads.make_custom(1, 2048, 8, 4, 2, 128, torch.bfloat16, seed=47)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    res = []
    for kw in (dict(kv_range=ra, kv_range2=rb), dict(kv_range=one)):
        if accumulate:
            o, l = tsp.fwd(qd, kd, vd, D=8, rank=r, kv_range=(1200, 1300))
            tsp.fwd(qd, kd, vd, D=8, rank=r, out=o, lse=l, accumulate=True, **kw)
        else:
            o, l = tsp.fwd(qd, kd, vd, D=8, rank=r, **kw)
        res.append((o, l))
    torch.cuda.synchronize()
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])
