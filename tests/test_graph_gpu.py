"""The C-ABI entry points under HIP graph capture, on an MI355X (gfx950).

The library allocates nothing and enqueues only kernels on the caller's stream, so a
sequence of calls with preallocated outputs can be captured once and replayed (a serving
loop, or the chunk pipeline of one layer without per-launch host work). Each test captures
through torch's graph API, replays several times with eager work and synchronisations in
between, and checks every replay bit for bit against the same calls run eagerly; one test
changes the inputs between replays.
"""

import pytest
import torch

import sequence_causal_attention_amd as tsp
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _note(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _pairs(S, D, r):
    """The ring-step key ranges: the rank's own chunks, then peer r-1, r-2, ... (mod D)."""
    C = S // (2 * D)
    return [((p * C, (p + 1) * C), ((2 * D - 1 - p) * C, (2 * D - p) * C)) for p in ((r - s) % D for s in range(D))]


def _pipeline(q, k, v, D, r, out, lse):
    for i, (ra, rb) in enumerate(_pairs(k.shape[1], D, r)):
        tsp.fwd(q, k, v, D=D, rank=r, kv_range=ra, kv_range2=rb, out=out, lse=lse, accumulate=i > 0)


def _capture(fn):
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # one eager run on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _eager_noise():
    """Unrelated eager work between replays: another attention call and a device copy."""
    a, b, c = workloads.make_custom(1, 512, 4, 4, 1, 64, torch.bfloat16, seed=5)
    tsp.fwd(a.to(DEV), b.to(DEV), c.to(DEV), D=4, rank=2)
    x = torch.ones(1 << 20, device=DEV)
    (x * 3).sum().item()


@pytest.mark.parametrize("case", [(2048, 8, 3, 4, 4, 128), (1200, 3, 2, 6, 2, 128), (1024, 2, 1, 8, 2, 64)],
                         ids=lambda c: "S{}_D{}_r{}_H{}x{}_d{}".format(*c))
def test_pair_pipeline_graph_replays(case):
    S, D, r, Hq, Hkv, dh = case
    _note(f"graph pair pipeline {case}")
    q, k, v = (t.to(DEV) for t in workloads.make_custom(1, S, D, Hq, Hkv, dh, torch.bfloat16, seed=61))
    ref_o, ref_l = torch.empty_like(q), torch.empty((1, Hq, q.shape[1]), device=DEV)
    _pipeline(q, k, v, D, r, ref_o, ref_l)
    torch.cuda.synchronize()
    out, lse = torch.full_like(q, 9.0), torch.full_like(ref_l, 9.0)
    g = _capture(lambda: _pipeline(q, k, v, D, r, out, lse))
    for i in range(3):
        out.fill_(7.0)
        lse.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {i}"
        _eager_noise()


def test_graph_replay_sees_new_inputs():
    """Inputs copied into the captured buffers between replays are the ones attended to."""
    _note("graph new inputs")
    S, D, r = 2048, 8, 5
    q, k, v = (t.to(DEV) for t in workloads.make_custom(1, S, D, 4, 2, 128, torch.bfloat16, seed=62))
    out, lse = torch.empty_like(q), torch.empty((1, 4, q.shape[1]), device=DEV)
    g = _capture(lambda: tsp.fwd(q, k, v, D=D, rank=r, out=out, lse=lse))
    for seed in (63, 64, 65):
        q2, k2, v2 = (t.to(DEV) for t in workloads.make_custom(1, S, D, 4, 2, 128, torch.bfloat16, seed=seed))
        ref_o, ref_l = tsp.fwd(q2, k2, v2, D=D, rank=r)
        q.copy_(q2)
        k.copy_(k2)
        v.copy_(v2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"seed {seed}"
        _eager_noise()


@pytest.mark.parametrize("dh", [64, 128, 256])
def test_fwd_bwd_graph_replays(dh):
    _note(f"graph fwd+bwd dh{dh}")
    S, D, r, Hq, Hkv = 1024, 4, 1, 4, 2
    q, k, v = (t.to(DEV) for t in workloads.make_custom(1, S, D, Hq, Hkv, dh, torch.bfloat16, seed=66))
    do = workloads.make_grad(q.shape, 67, torch.bfloat16).to(DEV)
    out, lse = torch.empty_like(q), torch.empty((1, Hq, q.shape[1]), device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty_like(lse)

    def step():
        tsp.fwd(q, k, v, D=D, rank=r, out=out, lse=lse)
        tsp.bwd(q, k, v, out, lse, do, D=D, rank=r, dq=dq, dk=dk, dv=dv, delta=delta)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, lse, dq, dk, dv, delta)]
    g = _capture(step)
    for i in range(3):
        for t in (out, lse, dq, dk, dv, delta):
            t.fill_(5.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "lse", "dq", "dk", "dv", "delta"), (out, lse, dq, dk, dv, delta), ref):
            assert torch.equal(a, b), f"replay {i}: {name}"
        _eager_noise()


def test_ring_graph_replays():
    """tsp_attn_fwd_ring (two launches, arrival flags set) captured once and replayed."""
    _note("graph ring")
    S, D, r, Hq, Hkv, dh = 4096, 4, 2, 4, 2, 128
    q, k, v = (t.to(DEV) for t in workloads.make_custom(1, S, D, Hq, Hkv, dh, torch.bfloat16, seed=68))
    ready = torch.ones(2 * D, dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    ref_o, ref_l = tsp.fwd_ring(q, k, v, D=D, rank=r, chunk_ready=ready, ready_value=1, spin_limit=1 << 10,
                                wait_status=status)
    torch.cuda.synchronize()
    out, lse = torch.empty_like(q), torch.empty_like(ref_l)
    g = _capture(lambda: tsp.fwd_ring(q, k, v, D=D, rank=r, out=out, lse=lse, chunk_ready=ready, ready_value=1,
                                      spin_limit=1 << 10, wait_status=status))
    for i in range(3):
        out.fill_(7.0)
        lse.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {i}"
        _eager_noise()
