"""The ring-order forward (tsp_attn_fwd_ring) against the fp64 oracle, on an MI355X.

The rank's own chunks run in one launch and every peer's chunks, in the order a ring
all-gather delivers them, in a second launch that reads a chunk only once its arrival flag
holds the expected value. The result must be the full causal attention of the rank's
queries (same bar as tsp_attn_fwd: max-abs 2e-2 on out and lse, relative Frobenius error
<= 1e-2 per head and chunk). A wait that never sees its flag must give up after its spin
limit, report it in wait_status, and let the launch complete.
"""

import numpy as np
import pytest
import torch

import oracle
import sequence_causal_attention_amd as tsp
import workloads

from test_parity_gpu import DEV, check, sample_rows

pytestmark = pytest.mark.gpu


def _note(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _inputs(B, S, D, rank, Hq, Hkv, dh, seed):
    w = workloads.Workload(f"ring_{S}_{D}_{rank}", B, S, D, (rank,), Hq, Hkv, dh, "bf16", seed)
    q, k, v = workloads.make_inputs(w, rank)
    return w, q, k, v


RING = [  # (B, S_total, D, rank, Hq, Hkv, dh)
    (1, 4096, 4, 0, 4, 2, 128),   # rank 0: its low tiles see no peer chunk
    (1, 4096, 4, 1, 4, 2, 128),
    (1, 4096, 4, 3, 4, 2, 128),   # last rank: its low tiles see every peer's first chunk
    (1, 8192, 8, 5, 4, 4, 128),
    (1, 4096, 2, 1, 6, 1, 256),   # GQA 6:1, dh 256
    (1, 2048, 4, 2, 4, 2, 64),    # dh 64
    (2, 4096, 4, 2, 2, 2, 128),   # batch of 2
    (1, 2048, 1, 0, 2, 2, 128),   # D = 1: the own chunks only
]


@pytest.mark.parametrize("case", RING, ids=lambda c: "B{}_S{}_D{}_r{}_H{}x{}_d{}".format(*c))
def test_ring_matches_oracle(case):
    B, S, D, r, Hq, Hkv, dh = case
    _note(f"ring B{B} S{S} D{D} r{r} H{Hq}x{Hkv} d{dh}")
    w, q, k, v = _inputs(B, S, D, r, Hq, Hkv, dh, 40 + r)
    out, lse = tsp.fwd_ring(q.to(DEV), k.to(DEV), v.to(DEV), D=D, rank=r)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.causal_attention(q, k, v, D, r)
    check(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_out, ref_lse,
          torch.bfloat16, C=w.C)


def test_ring_with_arrival_flags_equals_without():
    """Flags already set: the same launches, bit for bit."""
    B, S, D, r, Hq, Hkv, dh = 1, 8192, 4, 2, 4, 2, 128
    _note("ring flags set")
    w, q, k, v = _inputs(B, S, D, r, Hq, Hkv, dh, 50)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out0, lse0 = tsp.fwd_ring(qd, kd, vd, D=D, rank=r)
    ready = torch.full((2 * D,), 7, dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out1, lse1 = tsp.fwd_ring(qd, kd, vd, D=D, rank=r, chunk_ready=ready, ready_value=7, spin_limit=1000,
                              wait_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(out0, out1) and torch.equal(lse0, lse1)


def test_ring_wait_gives_up_and_reports():
    """A chunk whose flag never arrives: every wait stops after its spin limit, bit 0 of
    wait_status is set, and the launch completes (the stream stays usable)."""
    B, S, D, r, Hq, Hkv, dh = 1, 4096, 4, 3, 2, 2, 128
    _note("ring flag never set")
    w, q, k, v = _inputs(B, S, D, r, Hq, Hkv, dh, 51)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    ready = torch.full((2 * D,), 1, dtype=torch.int32, device=DEV)
    ready[1] = 0  # chunk 1 (peer 1's first chunk) has not arrived
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    tsp.fwd_ring(qd, kd, vd, D=D, rank=r, chunk_ready=ready, ready_value=1, spin_limit=4, wait_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 1
    # the stream still works: a plain forward afterwards is correct
    out, lse = tsp.fwd(qd, kd, vd, D=D, rank=r)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.causal_attention(q, k, v, D, r)
    check(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_out, ref_lse,
          torch.bfloat16, C=w.C)


def test_ring_7b_shard_sampled_rows():
    """The 7B shard at full size (S_total 32768, D 8, rank 3, 32 heads, dh 128)."""
    w = workloads.BY_NAME["tsp_7b_shard_s32k"]
    r = 3
    _note("ring 7B shard rank 3")
    q, k, v = workloads.make_inputs(w, r)
    out, lse = tsp.fwd_ring(q.to(DEV), k.to(DEV), v.to(DEV), D=w.D, rank=r)
    torch.cuda.synchronize()
    rows = sample_rows(w, n_random=32)
    ref_out, ref_lse = oracle.causal_attention(q, k, v, w.D, r, rows=rows, block=64)
    check(out.float().cpu().numpy()[:, rows].astype(np.float64), lse.cpu().numpy()[:, :, rows].astype(np.float64),
          ref_out, ref_lse, torch.bfloat16, C=w.C, rows=rows)


def test_ring_refusals():
    qf = torch.zeros(1, 1024, 2, 128, device=DEV)
    kf = torch.zeros(1, 4096, 2, 128, device=DEV)
    with pytest.raises(tsp.TspAttnError) as e:  # fp32: no ring kernel
        tsp.fwd_ring(qf, kf, kf.clone(), D=4, rank=1)
    assert e.value.status == tsp.TSP_EUNSUPPORTED
    q = torch.zeros(1, 256, 2, 128, device=DEV, dtype=torch.bfloat16)
    k = torch.zeros(1, 1024, 2, 128, device=DEV, dtype=torch.bfloat16)
    with pytest.raises(tsp.TspAttnError) as e:  # C = 128: not a multiple of the 256-row query tile
        tsp.fwd_ring(q, k, k.clone(), D=4, rank=1)
    assert e.value.status == tsp.TSP_EUNSUPPORTED
    out = torch.empty_like(q)
    lse = torch.empty(1, 2, 256, device=DEV)
    ready = torch.ones(8, dtype=torch.int32, device=DEV)
    st = tsp.lib().tsp_attn_fwd_ring(q.data_ptr(), k.data_ptr(), k.data_ptr(), out.data_ptr(), lse.data_ptr(), 1,
                                     1024, 4, 1, 2, 2, 128, ready.data_ptr(), 1, 10, None, tsp.TSP_BF16, None)
    assert st == tsp.TSP_EINVAL  # flags without a status word


def test_ring_reads_chunks_only_after_they_arrive():
    """K/V chunks delivered by host-to-device copies on a second stream while the ring
    launch runs: the peers' chunks start as NaN on the device and each chunk's flag is
    copied in after its data, so a chunk read before its flag would put NaN into the
    result. The launch is enqueued first and the copies only afterwards (a host pause in
    between), so its waits see the flags arrive. The spin budget (2^22 polls of ~1 us, some
    seconds per wait) lies far above any copy time, so the outcome does not depend on how
    fast the box delivers the copies; a wait that did give up would be reported through
    the status word, never hang."""
    import time

    B, S, D, r, Hq, Hkv, dh = 1, 4096, 4, 3, 4, 2, 128
    _note("ring with chunks copied in during the launch")
    w, q, k, v = _inputs(B, S, D, r, Hq, Hkv, dh, 52)
    C = w.C
    k_host, v_host = k.pin_memory(), v.pin_memory()
    kd = torch.full(k.shape, float("nan"), dtype=k.dtype, device=DEV)
    vd = torch.full(v.shape, float("nan"), dtype=v.dtype, device=DEV)
    for c in (r, 2 * D - 1 - r):  # the rank's own chunks are local
        kd[:, c * C:(c + 1) * C].copy_(k[:, c * C:(c + 1) * C])
        vd[:, c * C:(c + 1) * C].copy_(v[:, c * C:(c + 1) * C])
    qd = q.to(DEV)
    ready = torch.zeros(2 * D, dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    one = torch.ones(1, dtype=torch.int32).pin_memory()
    compute, comm = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(comm):  # the first pinned copies of a process set up their path (~15 ms)
        torch.empty(1, dtype=torch.int32, device=DEV).copy_(one, non_blocking=True)
        torch.empty_like(kd[:, :C]).copy_(k_host[:, :C], non_blocking=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(compute):
        out, lse = tsp.fwd_ring(qd, kd, vd, D=D, rank=r, chunk_ready=ready, ready_value=1, spin_limit=1 << 22,
                                wait_status=status, stream=compute)
    time.sleep(0.005)
    with torch.cuda.stream(comm):
        for s in range(1, D):  # ring order: both chunks of peer (r - s) mod D per step
            p = (r - s) % D
            for c in (p, 2 * D - 1 - p):
                kd[:, c * C:(c + 1) * C].copy_(k_host[:, c * C:(c + 1) * C], non_blocking=True)
                vd[:, c * C:(c + 1) * C].copy_(v_host[:, c * C:(c + 1) * C], non_blocking=True)
                ready[c:c + 1].copy_(one, non_blocking=True)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "a wait gave up before its chunk arrived"
    ref_out, ref_lse = oracle.causal_attention(q, k, v, D, r)
    check(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_out, ref_lse,
          torch.bfloat16, C=w.C)


def test_ring_gqa_shard_sampled_rows():
    """The GQA dh-256 shard at full size (S_total 65536, D 4, rank 2, 24 query heads on 4
    KV heads): 64-row query tiles, 32-key stages."""
    w = workloads.BY_NAME["gqa_shard_s64k"]
    r = 2
    _note("ring GQA shard rank 2")
    q, k, v = workloads.make_inputs(w, r)
    ready = torch.ones(2 * w.D, dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, lse = tsp.fwd_ring(q.to(DEV), k.to(DEV), v.to(DEV), D=w.D, rank=r, chunk_ready=ready, ready_value=1,
                            spin_limit=1 << 10, wait_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    rows = sample_rows(w, n_random=24)
    ref_out, ref_lse = oracle.causal_attention(q, k, v, w.D, r, rows=rows, block=64)
    check(out.float().cpu().numpy()[:, rows].astype(np.float64), lse.cpu().numpy()[:, :, rows].astype(np.float64),
          ref_out, ref_lse, torch.bfloat16, C=w.C, rows=rows)
