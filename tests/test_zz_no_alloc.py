"""tsp_attn_bwd_noalloc (the backward for callers that cannot allocate) against
tsp_attn_bwd, through the C ABI, on an MI355X.

Both entry points run the same kernels on the same inputs; the only difference is where
delta lives (the caller's buffer, or the library's static device array), so the results
must agree bit for bit, which is stronger than the backward's tolerance against the
oracle. Calls follow one another with shrinking inputs, so a workspace left over from an
earlier, larger call cannot stand in for the current one; the last call is fp32.
"""

import numpy as np
import pytest
import torch

import oracle
import sequence_causal_attention_amd as tsp
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CALLS = [  # (B, S_total, D, rank, Hq, Hkv, dh, dtype), largest first
    (1, 8192, 4, 1, 8, 2, 128, torch.bfloat16),
    (1, 4096, 4, 2, 12, 2, 256, torch.bfloat16),
    (1, 1200, 3, 2, 6, 2, 64, torch.bfloat16),
    (1, 512, 4, 1, 4, 1, 64, torch.float32),
]


def _note(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _inputs(case, seed):
    B, S, D, r, Hq, Hkv, dh, dt = case
    q, k, v = workloads.make_custom(B, S, D, Hq, Hkv, dh, dt, seed=seed)
    dout = workloads.make_grad(q.shape, seed + 1, dt)
    return tuple(t.to(DEV) for t in (q, k, v, dout))


def _noalloc(qd, kd, vd, out, lse, dod, case, dq, dk, dv):
    B, S, D, r, Hq, Hkv, dh, dt = case
    code = tsp.TSP_BF16 if dt == torch.bfloat16 else tsp.TSP_F32
    return tsp.lib().tsp_attn_bwd_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out.data_ptr(),
                                          lse.data_ptr(), dod.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                          B, S, D, r, Hq, Hkv, dh, code, torch.cuda.current_stream().cuda_stream)


def test_noalloc_matches_allocating_backward():
    for i, case in enumerate(CALLS):
        B, S, D, r, Hq, Hkv, dh, dt = case
        _note(f"bwd_noalloc call {i}: {case}")
        qd, kd, vd, dod = _inputs(case, 300 + i)
        out, lse = tsp.fwd(qd, kd, vd, D=D, rank=r)
        ref = tsp.bwd(qd, kd, vd, out, lse, dod, D=D, rank=r)
        dq = torch.full_like(qd, float("nan"))
        dk = torch.full_like(kd, float("nan"))
        dv = torch.full_like(vd, float("nan"))
        st = _noalloc(qd, kd, vd, out, lse, dod, case, dq, dk, dv)
        assert st == tsp.TSP_OK, tsp.lib().tsp_attn_last_error()
        torch.cuda.synchronize()
        for name, got, want in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
            assert torch.equal(got, want), f"call {i} {case}: {name} differs from tsp_attn_bwd"
        if i == len(CALLS) - 1:  # the smallest call also against the oracle's gradients
            rq, rk, rv = oracle.causal_attention_backward(qd.cpu(), kd.cpu(), vd.cpu(), dod.cpu(), D, r)
            for name, got, want in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
                g = got.double().cpu().numpy()
                scale = max(np.abs(want).max(), 1.0)
                assert np.abs(g - want).max() <= 1e-4 * scale, name


def test_noalloc_rejects_more_rows_than_its_workspace():
    """B * Hq * 2C above the static array: TSP_EINVAL, nothing launched, outputs untouched.
    The buffers are the real sizes of that call, so even a launch would stay in bounds."""
    case = (1, 262144, 1, 0, 17, 1, 64, torch.bfloat16)  # 17 * 262144 rows > 4 Mi
    B, S, D, r, Hq, Hkv, dh, dt = case
    assert B * Hq * (S // D) > tsp.MAX_NOALLOC_ROWS
    _note(f"bwd_noalloc oversize {case}")
    qd = torch.zeros((B, S // D, Hq, dh), dtype=dt, device=DEV)
    kd = torch.zeros((B, S, Hkv, dh), dtype=dt, device=DEV)
    vd = torch.zeros_like(kd)
    out = torch.zeros_like(qd)
    lse = torch.zeros((B, Hq, S // D), dtype=torch.float32, device=DEV)
    dq, dk, dv = torch.full_like(qd, 3.0), torch.full_like(kd, 3.0), torch.full_like(vd, 3.0)
    st = _noalloc(qd, kd, vd, out, lse, qd, case, dq, dk, dv)
    assert st == tsp.TSP_EINVAL
    assert "workspace" in tsp.lib().tsp_attn_last_error().decode()
    torch.cuda.synchronize()
    assert bool((dq == 3.0).all()) and bool((dk == 3.0).all()) and bool((dv == 3.0).all())
