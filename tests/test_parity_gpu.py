"""HIP path vs the fp64 oracle, through the C ABI, on an MI355X (gfx950).

Tolerances: max-abs 2e-2 (bf16 inputs) / 1e-4 (fp32 inputs) on out and on lse; for bf16
also a relative Frobenius error <= 1e-2 per (head, chunk), because late rows of long
sequences have |out| far below 2e-2. The device zigzag map must match bit-exactly.
"""

import math

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


def run(q, k, v, D, rank):
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out, lse = tsp.fwd(qd, kd, vd, D=D, rank=rank)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check(out, lse, ref_out, ref_lse, dtype, C=None, rows=None):
    tol = TOL[dtype]
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    err_o = np.abs(out - ref_out).max()
    err_l = np.abs(lse - ref_lse).max()
    assert err_o <= tol, f"max |out - ref| = {err_o:.3g} > {tol}"
    assert err_l <= tol, f"max |lse - ref| = {err_l:.3g} > {tol}"
    if dtype == torch.bfloat16:
        rows = np.arange(out.shape[1]) if rows is None else np.asarray(rows)
        chunk = rows >= C if C is not None else np.zeros(len(rows), bool)
        for h in range(out.shape[2]):
            for c in (False, True):
                sel = chunk == c
                if not sel.any():
                    continue
                d = out[:, sel, h] - ref_out[:, sel, h]
                rel = np.linalg.norm(d) / max(np.linalg.norm(ref_out[:, sel, h]), 1e-30)
                assert rel <= 1e-2, f"head {h} chunk {int(c)}: relative error {rel:.3g}"
    return err_o, err_l


# -- full-row parity on shards small enough for the oracle ------------------------------

SMALL = [  # (B, S_total, D, rank, Hq, Hkv, dh, dtype)
    (1, 512, 4, 1, 4, 1, 64, torch.float32),       # the tiny zigzag GQA shard itself
    (1, 512, 4, 0, 4, 1, 64, torch.float32),
    (1, 512, 4, 3, 4, 1, 64, torch.float32),
    (1, 2048, 8, 3, 4, 4, 128, torch.bfloat16),    # 7B-style MHA shard, scaled down
    (1, 2048, 8, 0, 4, 4, 128, torch.bfloat16),
    (1, 2048, 8, 7, 4, 4, 128, torch.bfloat16),
    (1, 4096, 4, 2, 12, 2, 256, torch.bfloat16),   # GQA 6:1, dh 256, scaled down
    (1, 4096, 1, 0, 4, 4, 128, torch.bfloat16),    # Ulysses head subset (D = 1)
    (1, 1024, 2, 1, 8, 2, 64, torch.bfloat16),     # dh 64
    (1, 1200, 3, 2, 6, 2, 128, torch.bfloat16),    # ragged: C = 200 (no tile divides it)
    (1, 1200, 3, 0, 6, 3, 256, torch.bfloat16),    # ragged, dh 256, grp 2
    (1, 600, 3, 1, 2, 1, 128, torch.float32),      # ragged fp32, dh 128
    (1, 288, 2, 1, 4, 2, 256, torch.float32),      # ragged fp32, dh 256, C = 72
    (2, 1024, 4, 1, 4, 2, 128, torch.bfloat16),    # batch of 2
    (1, 2, 1, 0, 1, 1, 128, torch.bfloat16),       # two tokens
    (1, 8, 4, 3, 2, 1, 64, torch.bfloat16),        # one token per chunk
    (1, 8, 4, 2, 2, 2, 64, torch.float32),
    (1, 96, 1, 0, 3, 1, 128, torch.bfloat16),      # grp 3 (no divisor of the wave count)
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}_S{}_D{}_r{}_H{}x{}_d{}_{}".format(*c[:7], str(c[7])[6:]))
def test_small_shard_matches_oracle(case):
    B, S, D, r, Hq, Hkv, dh, dt = case
    _note(f"small {case}")
    q, k, v = workloads.make_custom(B, S, D, Hq, Hkv, dh, dt, seed=7 * S + 13 * D + r + dh)
    out, lse = run(q, k, v, D, r)
    ref_out, ref_lse = oracle.causal_attention(q, k, v, D, r)
    check(out, lse, ref_out, ref_lse, dt, C=S // (2 * D))


# -- the workloads at their real sizes: sampled rows, all heads -------------------------

def sample_rows(w, n_random=512, seed=0, edge=64, tile_block=256):
    """Local rows compared at full size: the first and last `edge` rows of each chunk,
    rows on both sides of every 64-row boundary up to 256, `n_random` seeded random rows,
    and a complete block of `tile_block` rows in the middle of the first chunk together
    with its mirror image in the second chunk. The kernels process local rows in
    mirrored pairs of query tiles (tile p with tile n-1-p) of 64, 128 or 256 rows, all of
    which divide `tile_block`, so the block and its mirror hold every row of whole
    workgroups."""
    C, S = w.C, w.S_local
    rows = set()
    for base in (0, C):
        rows.update(range(base, base + min(edge, C)))
        rows.update(range(base + max(0, C - edge), base + C))
        for t in (63, 64, 127, 128, 255, 256):
            if t < C:
                rows.add(base + t)
    if S >= 2 * tile_block and S % tile_block == 0:
        a = (C // 2 // tile_block) * tile_block
        rows.update(range(a, a + tile_block))
        rows.update(range(S - a - tile_block, S - a))
    rng = np.random.default_rng(seed)
    rows.update(int(x) for x in rng.integers(0, S, n_random))
    return np.array(sorted(x for x in rows if 0 <= x < S))


def oracle_rows(q, k, v, D, r, rows, block=64):
    """The oracle on the given rows, one query head per worker thread (numpy's kernels
    run without the interpreter lock; the threaded BLAS is held to one thread each)."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    Hq = q.shape[2]
    n = max(1, min(16, os.cpu_count() or 1, Hq))
    with threadpool_limits(limits=1), ThreadPoolExecutor(n) as ex:
        parts = list(ex.map(lambda h: oracle.causal_attention(q, k, v, D, r, rows=rows, heads=[h], block=block),
                            range(Hq)))
    return np.concatenate([o for o, _ in parts], axis=2), np.concatenate([l for _, l in parts], axis=1)


def _rank_cases():
    out = []
    for w in workloads.WORKLOADS:
        for r in w.ranks:
            out.append((w, r))
    return out


@pytest.mark.parametrize("wr", _rank_cases(), ids=lambda wr: f"{wr[0].name}_r{wr[1]}")
def test_workload_sampled_rows_match_oracle(wr):
    w, r = wr
    q, k, v = workloads.make_inputs(w, r)
    # dh-256 tiles are 64 or 128 rows; 128 random rows at 256K keys keep the oracle near a minute
    rows = np.arange(w.S_local) if w.index == 0 else sample_rows(
        w, n_random=512 if w.S_total <= 131072 else 128, tile_block=256 if w.dh <= 128 else 128)
    _note(f"workload {w.name} rank {r}: {len(rows)} rows, all {w.Hq} heads")
    out, lse = run(q, k, v, w.D, r)
    ref_out, ref_lse = oracle_rows(q, k, v, w.D, r, rows)
    check(out[:, rows], lse[:, :, rows], ref_out, ref_lse, w.torch_dtype(), C=w.C, rows=rows)


@pytest.mark.parametrize("name", ["tiny_zigzag_gqa_f32", "tsp_7b_shard_s32k"])
def test_fwd_entry_point_direct(name):
    """tsp_attn_fwd called through the C ABI itself (no binding logic in between) on the
    tiny fp32 shard in full and the 7B shard on sampled rows, against the oracle; and bit
    for bit equal to the same attention taken as the key range [0, S_total)."""
    w = workloads.BY_NAME[name]
    r = w.ranks[0]
    _note(f"tsp_attn_fwd direct {name}")
    q, k, v = workloads.make_inputs(w, r)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((w.B, w.Hq, w.S_local), float("nan"), device=DEV)
    code = tsp.TSP_BF16 if w.dtype == "bf16" else tsp.TSP_F32
    stream = torch.cuda.current_stream()
    st = tsp.lib().tsp_attn_fwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                w.B, w.S_total, w.D, r, w.Hq, w.Hkv, w.dh, code, stream.cuda_stream)
    assert st == tsp.TSP_OK, tsp.lib().tsp_attn_last_error()
    out_r, lse_r = tsp.fwd(qd, kd, vd, D=w.D, rank=r, kv_range=(0, w.S_total))
    torch.cuda.synchronize()
    assert torch.equal(out, out_r) and torch.equal(lse, lse_r)
    rows = np.arange(w.S_local) if w.index == 0 else sample_rows(w, n_random=128, edge=16)
    ref_out, ref_lse = oracle_rows(q, k, v, w.D, r, rows)
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    check(o[:, rows], l[:, :, rows], ref_out, ref_lse, w.torch_dtype(), C=w.C, rows=rows)


@pytest.mark.parametrize("rank", range(8))
def test_every_rank_of_the_7b_shard(rank):
    """Each of the 8 ranks of the 7B-dense shard at full size (its own queries, the shared
    K/V): rows at both ends of both chunks and seeded random rows, all 32 heads."""
    w = workloads.BY_NAME["tsp_7b_shard_s32k"]
    _note(f"7B shard rank {rank}")
    q, k, v = workloads.make_inputs(w, rank)
    out, lse = run(q, k, v, w.D, rank)
    C = w.C
    rng = np.random.default_rng(100 + rank)
    rows = np.unique(np.concatenate([[0, 1, C - 2, C - 1, C, C + 1, 2 * C - 2, 2 * C - 1],
                                     rng.integers(0, 2 * C, 16)]))
    ref_out, ref_lse = oracle.causal_attention(q, k, v, w.D, rank, rows=rows, block=64)
    check(out[:, rows], lse[:, :, rows], ref_out, ref_lse, torch.bfloat16, C=C, rows=rows)


# -- the zigzag map ---------------------------------------------------------------------

@pytest.mark.parametrize("S,D,r", [(512, 4, 1), (32768, 8, 3), (262144, 8, 0), (262144, 8, 7), (131072, 1, 0),
                                   (1200, 3, 2), (2, 1, 0)])
def test_device_map_bit_exact(S, D, r):
    got = tsp.zigzag_positions_device(S, D, r, DEV).cpu().numpy().astype(np.int64)
    assert np.array_equal(got, oracle.zigzag_positions(S, D, r))


# -- closed forms and special inputs -----------------------------------------------------

@pytest.mark.parametrize("S,D,r,Hq,Hkv,dh", [(32768, 8, 3, 4, 4, 128), (8192, 4, 2, 12, 2, 256),
                                             (1200, 3, 1, 2, 1, 64)])
def test_zero_queries_count_visible_keys_exactly(S, D, r, Hq, Hkv, dh):
    """q = 0: every visible key weighs exactly 1, so exp(lse) is the visible-key count
    g(i) + 1, and out is the prefix mean of v."""
    _note(f"zero q {S} {D} {r}")
    q, k, v = workloads.make_custom(1, S, D, Hq, Hkv, dh, torch.bfloat16, seed=99)
    q.zero_()
    out, lse = run(q, k, v, D, r)
    pos = oracle.zigzag_positions(S, D, r)
    counts = np.rint(np.exp(lse[0])).astype(np.int64)
    assert np.array_equal(counts, np.broadcast_to(pos + 1, counts.shape))
    assert int(counts[0].sum()) == (S // (2 * D)) * (S + 1)
    vf = v.double().numpy()[0]
    for h in range(Hq):
        pm = np.cumsum(vf[:, h // (Hq // Hkv)], axis=0) / np.arange(1, S + 1)[:, None]
        assert np.abs(out[0, :, h] - pm[pos]).max() <= 2e-2


def test_values_one_give_one():
    q, k, v = workloads.make_custom(1, 4096, 4, 4, 2, 128, torch.bfloat16, seed=5)
    v.fill_(1.0)
    out, _ = run(q, k, v, 4, 1)
    assert np.all(out == 1.0)


def test_first_position_row():
    """Rank 0's first query sees only key 0: out = v_0, lse = q.k_0 / sqrt(dh)."""
    q, k, v = workloads.make_custom(1, 2048, 8, 2, 1, 128, torch.bfloat16, seed=6)
    out, lse = run(q, k, v, 8, 0)
    v0 = v[0, 0, 0].double().numpy()
    for h in range(2):
        assert np.array_equal(out[0, 0, h], v0)  # exactly: weight 1 times a bf16 value
        ref = float(q[0, 0, h].double() @ k[0, 0, 0].double()) / math.sqrt(128)
        assert abs(lse[0, h, 0] - ref) < 1e-3


def test_keys_past_the_shard_are_never_read():
    """NaN in every key/value row past the rank's last query position must not reach
    the output: causal tile skipping never loads them."""
    S, D, r = 32768, 8, 3
    q, k, v = workloads.make_custom(1, S, D, 4, 4, 128, torch.bfloat16, seed=8)
    last = int(oracle.zigzag_positions(S, D, r).max())
    k[:, last + 1:] = float("nan")
    v[:, last + 1:] = float("nan")
    out, lse = run(q, k, v, D, r)
    rows = np.array([0, 1, 2047, 2048, 4094, 4095])
    ref_out, ref_lse = oracle.causal_attention(q, k, v, D, r, rows=rows)
    check(out[:, rows], lse[:, :, rows], ref_out, ref_lse, torch.bfloat16)
    assert np.isfinite(out).all() and np.isfinite(lse).all()


def test_large_masked_scores_do_not_leak():
    """Keys inside partly visible tiles get large values (scores ~ +100); each query must
    still see only keys up to its own position."""
    S, D, r = 2048, 4, 1
    q, k, v = workloads.make_custom(1, S, D, 2, 1, 128, torch.bfloat16, seed=9)
    pos = oracle.zigzag_positions(S, D, r)
    hot = np.concatenate([np.arange(p0 + 1, p0 + 40) for p0 in pos[::37]])
    hot = hot[hot < S]
    k[0, hot] = 8.0
    out, lse = run(q, k, v, D, r)
    ref_out, ref_lse = oracle.causal_attention(q, k, v, D, r)
    check(out, lse, ref_out, ref_lse, torch.bfloat16, C=S // (2 * D))


def _rising_scores(rise_target, seed, dh, S=8192, D=2, r=0):
    """A shard whose scores rise along the key index: q_i[0] = 8 and k_j[0] = g * j / S with
    g chosen so that the last row's top score lies about `rise_target` log2 units above its
    top score over the first 32 keys; the other dims N(0, 1). Returns the inputs and that
    rise as it comes out of the rounded inputs (how far above a running max taken at the
    sweep's first step the weights go)."""
    q, k, v = workloads.make_custom(1, S, D, 2, 1, dh, torch.bfloat16, seed=seed)
    growth = rise_target * math.sqrt(dh) * math.log(2) / 8.0
    q[..., 0] = 8.0
    k[0, :, 0, 0] = (torch.arange(S, dtype=torch.float64) * growth / S).to(torch.bfloat16)
    pos = oracle.zigzag_positions(S, D, r)
    i = int(np.argmax(pos))
    s = k[0, : pos[i] + 1, 0].double().numpy() @ q[0, i].double().numpy().T / math.sqrt(dh)  # [keys, heads]
    rise = float((s.max(axis=0) - s[:32].max(axis=0)).max() / math.log(2))
    return q, k, v, rise


# The kernels that run one wave per SIMD (dh 256; dh 128 one-range launches) keep the running
# max of the sweep's first step in their unrolled steps: weights up to 2^rise must stay exact,
# and an overflow must send the tile through a second, checked sweep.
@pytest.mark.parametrize("dh", [128, 256])
def test_scores_far_above_the_first_step(dh):
    q, k, v, rise = _rising_scores(75.0, seed=41 + dh, dh=dh)
    assert 40.0 < rise < 100.0, rise
    out, lse = run(q, k, v, 2, 0)
    ref_out, ref_lse = oracle.causal_attention(q, k, v, 2, 0)
    check(out, lse, ref_out, ref_lse, torch.bfloat16, C=8192 // 4)


@pytest.mark.parametrize("dh", [128, 256])
def test_overflow_is_swept_again(dh):
    q, k, v, rise = _rising_scores(290.0, seed=43 + dh, dh=dh)
    assert rise > 160.0, rise
    out, lse = run(q, k, v, 2, 0)
    ref_out, ref_lse = oracle.causal_attention(q, k, v, 2, 0)
    check(out, lse, ref_out, ref_lse, torch.bfloat16, C=8192 // 4)


def test_overflow_in_a_two_range_launch():
    """The dh-256 two-range launch (the rank's two own chunks, one sweep over both) with
    scores rising past the fp32 range of the fixed-max weights in the second range: the
    result must equal the oracle's attention over the union of the two ranges."""
    S, D, r = 8192, 2, 0
    q, k, v, rise = _rising_scores(290.0, seed=47, dh=256, S=S, D=D, r=r)
    assert rise > 160.0, rise
    C = S // (2 * D)
    ra, rb = (r * C, (r + 1) * C), ((2 * D - 1 - r) * C, (2 * D - r) * C)
    o, l = tsp.fwd(q.to(DEV), k.to(DEV), v.to(DEV), D=D, rank=r, kv_range=ra, kv_range2=rb)
    torch.cuda.synchronize()
    out, lse = o.float().cpu().numpy().astype(np.float64), l.cpu().numpy().astype(np.float64)
    oa, la = oracle.causal_attention_range(q, k, v, D, r, *ra)
    ob, lb = oracle.causal_attention_range(q, k, v, D, r, *rb)
    ref_out, ref_lse = oracle.merge_partials(oa, la, ob, lb)
    check(out, lse, ref_out, ref_lse, torch.bfloat16, C=C)


# -- structural identities ---------------------------------------------------------------

def test_concatenation_of_all_ranks_equals_unsharded():
    """Each rank's rows, scattered by global position, rebuild the D = 1 result."""
    S, D, Hq, Hkv, dh = 4096, 8, 4, 2, 128
    g = torch.Generator().manual_seed(11)
    qf = torch.randn(1, S, Hq, dh, generator=g).to(torch.bfloat16)
    k = torch.randn(1, S, Hkv, dh, generator=g).to(torch.bfloat16)
    v = torch.randn(1, S, Hkv, dh, generator=g).to(torch.bfloat16)
    full_out, full_lse = run(qf, k, v, 1, 0)
    got_out = np.full_like(full_out, np.nan)
    got_lse = np.full_like(full_lse, np.nan)
    for r in range(D):
        pos = oracle.zigzag_positions(S, D, r)
        o, l = run(qf[:, pos].contiguous(), k, v, D, r)
        got_out[:, pos] = o
        got_lse[:, :, pos] = l
    assert np.abs(got_out - full_out).max() <= 2e-2
    assert np.abs(got_lse - full_lse).max() <= 2e-2
    ref_out, ref_lse = oracle.causal_attention(qf, k, v, 1, 0)
    check(got_out, got_lse, ref_out, ref_lse, torch.bfloat16)


def test_gqa_equals_repeated_heads():
    S, D, r, Hq, Hkv, dh = 4096, 4, 2, 12, 2, 256
    q, k, v = workloads.make_custom(1, S, D, Hq, Hkv, dh, torch.bfloat16, seed=12)
    out_g, lse_g = run(q, k, v, D, r)
    grp = Hq // Hkv
    out_m, lse_m = run(q, k.repeat_interleave(grp, dim=2).contiguous(), v.repeat_interleave(grp, dim=2).contiguous(),
                       D, r)
    assert np.abs(out_g - out_m).max() <= 2e-2
    assert np.abs(lse_g - lse_m).max() <= 2e-2


@pytest.mark.parametrize("dh", [128, 256])
def test_key_shift_invariance(dh):
    """Adding one vector c to every key leaves out unchanged and shifts lse by
    q_i . c / sqrt(dh). Keys and c lie on a 1/16 grid with |k + c| < 16, so k + c is exact
    in bf16 and the property holds for the stored values; both runs are also checked
    against the oracle."""
    S, D, r, Hq, Hkv = 2048, 4, 1, 4, 2
    q, k, v = workloads.make_custom(1, S, D, Hq, Hkv, dh, torch.bfloat16, seed=21 + dh)
    k = (k.float() * 16).round().clamp(-96, 96).div(16).to(torch.bfloat16)
    g = torch.Generator().manual_seed(5)
    c = (torch.randn(Hkv, dh, generator=g) * 16).round().clamp(-32, 32).div(16)
    k2 = (k.float() + c).to(torch.bfloat16)
    assert torch.equal(k2.float() - k.float(), c.expand_as(k2.float()))  # exact in bf16
    out1, lse1 = run(q, k, v, D, r)
    out2, lse2 = run(q, k2, v, D, r)
    grp = Hq // Hkv
    shift = np.einsum("bshd,hd->bhs", q.double().numpy(), c.double().numpy().repeat(grp, axis=0)) / math.sqrt(dh)
    assert np.abs(out2 - out1).max() <= 2e-2
    assert np.abs(lse2 - lse1 - shift).max() <= 2e-2
    for kk, out, lse in ((k, out1, lse1), (k2, out2, lse2)):
        ref_out, ref_lse = oracle.causal_attention(q, kk, v, D, r)
        check(out, lse, ref_out, ref_lse, torch.bfloat16, C=S // (2 * D))


def test_deterministic_bitwise():
    q, k, v = workloads.make_custom(1, 8192, 8, 8, 2, 128, torch.bfloat16, seed=13)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o1, l1 = tsp.fwd(qd, kd, vd, D=8, rank=5)
    o2, l2 = tsp.fwd(qd, kd, vd, D=8, rank=5)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dt,dh", [(torch.bfloat16, 128), (torch.bfloat16, 256), (torch.float32, 64)])
def test_outputs_stay_inside_their_buffers(dt, dh):
    """Canary words after out and lse are untouched."""
    B, S, D, r, Hq, Hkv = 1, 1200, 3, 1, 4, 2
    q, k, v = workloads.make_custom(B, S, D, Hq, Hkv, dh, dt, seed=14)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    n_out, n_lse, pad = q.numel(), B * Hq * (S // D), 4096
    out_buf = torch.full((n_out + pad,), 7.0, dtype=dt, device=DEV)
    lse_buf = torch.full((n_lse + pad,), -3.0, dtype=torch.float32, device=DEV)
    out = out_buf[:n_out].view(q.shape)
    lse = lse_buf[:n_lse].view(B, Hq, S // D)
    tsp.fwd(qd, kd, vd, D=D, rank=r, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(out_buf[n_out:] == 7.0)
    assert torch.all(lse_buf[n_lse:] == -3.0)
    assert torch.isfinite(out.float()).all()


def test_invalid_call_writes_nothing():
    q, k, v = workloads.make_custom(1, 512, 4, 4, 1, 64, torch.bfloat16, seed=15)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.full_like(qd, 3.0)
    lse = torch.full((1, 4, 128), 5.0, device=DEV)
    st = tsp.fwd_raw(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out.data_ptr(), lse.data_ptr(),
                     1, 512, 4, 4, 4, 1, 64, tsp.TSP_BF16, torch.cuda.current_stream().cuda_stream)
    assert st == tsp.TSP_EINVAL  # rank 4 of 4
    st = tsp.fwd_raw(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out.data_ptr(), lse.data_ptr(),
                     1, 512, 4, 1, 4, 1, 96, tsp.TSP_BF16, torch.cuda.current_stream().cuda_stream)
    assert st == tsp.TSP_EUNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(out == 3.0) and torch.all(lse == 5.0)
    with pytest.raises(tsp.TspAttnError):
        tsp.fwd(qd, kd, vd, D=4, rank=4)


def test_binding_rejects_host_and_mistyped_buffers():
    """Caller-supplied outputs on the host, or of the wrong type, are refused before any
    launch (their pointers would otherwise reach the kernels)."""
    q, k, v = workloads.make_custom(1, 512, 4, 4, 1, 64, torch.bfloat16, seed=3)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out, lse = tsp.fwd(qd, kd, vd, D=4, rank=1)
    with pytest.raises(tsp.TspAttnError):
        tsp.fwd(qd, kd, vd, D=4, rank=1, out=torch.empty_like(q), lse=lse)
    with pytest.raises(tsp.TspAttnError):
        tsp.fwd(qd, kd, vd, D=4, rank=1, out=out, lse=lse.cpu())
    with pytest.raises(tsp.TspAttnError):
        tsp.merge(out, lse, out, lse, out=out.cpu(), lse=lse)
    dout = torch.zeros_like(qd)
    with pytest.raises(tsp.TspAttnError):
        tsp.bwd(qd, kd, vd, out, lse, dout, D=4, rank=1, dk=torch.empty_like(k))
    with pytest.raises(tsp.TspAttnError):
        tsp.ulysses_pack_heads(qd, 2, out=torch.empty(2, 1, 128, 2, 64, dtype=torch.bfloat16))
    a = torch.zeros(64, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(tsp.TspAttnError):
        tsp.gemm_nt(a, a, out=torch.empty(64, 64, dtype=torch.float16, device=DEV))
    with pytest.raises(tsp.TspAttnError):
        tsp.gemm_nt(a, a, out=torch.empty(64, 64, dtype=torch.bfloat16, device=DEV), accumulate=True)
    with pytest.raises(tsp.TspAttnError):
        tsp.gemm_nt(a, a, out=torch.empty(64, 64, dtype=torch.float32))
    torch.cuda.synchronize()
