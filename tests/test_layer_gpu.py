"""The bf16 GEMM (tsp_gemm_bf16_nt) and one rank's TSP attention layer
(tsp_attn_layer_fwd) vs the oracle, through the C ABI, on an MI355X.

GEMM tolerances: bf16 output, relative Frobenius error <= 2^-8 and max-abs error
<= 2^-7 * max|ref| (one bf16 rounding of an fp32 sum); fp32 output, 1e-5 and 1e-4.
Layer tolerances: relative Frobenius error <= 2e-2 and max-abs <= 2^-4 * max|ref| on y
(q, k, v and the attention output are each rounded to bf16 on the way, and the
attention itself keeps its own bf16 bounds); the rank's rows of the gathered K/V within
2^-7 * max|ref| of the oracle's projections, every other row untouched bit for bit.
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


def _rel(got, ref):
    return np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)


GEMM_CASES = [  # (M, N, K, padded leading dims)
    (128, 128, 64, False),
    (300, 200, 128, False),   # ragged tiles in M and N
    (1, 4, 64, False),
    (4096, 512, 4096, False),  # a shard's Q projection of the 7B shard
    (4096, 4096, 256, False),  # enough 256 x 256 tiles for the big-tile kernel
    (4000, 4100, 128, False),  # ... with ragged tails
    (257, 132, 192, True),    # strided operands and output
]


@pytest.mark.parametrize("case", GEMM_CASES, ids=lambda c: "M{}_N{}_K{}_{}".format(*c[:3], "strided" if c[3] else "dense"))
def test_gemm_vs_reference(case):
    M, N, K, padded = case
    _note(f"gemm {case}")
    g = torch.Generator().manual_seed(M * 7 + N)
    pad = 24 if padded else 0
    a_full = torch.randn(M, K + pad, generator=g).to(torch.bfloat16)
    b_full = torch.randn(N, K + 2 * pad, generator=g).to(torch.bfloat16)
    a, b = a_full[:, :K], b_full[:, :K]
    ref = a.double().numpy() @ b.double().numpy().T
    ad, bd = a_full.to(DEV)[:, :K], b_full.to(DEV)[:, :K]
    out_full = torch.zeros(M, N + pad, dtype=torch.bfloat16, device=DEV)
    out = tsp.gemm_nt(ad, bd, out=out_full[:, :N])
    f32 = tsp.gemm_nt(ad, bd, out=torch.empty(M, N, device=DEV))
    acc = torch.full((M, N), 1.5, device=DEV)
    tsp.gemm_nt(ad, bd, out=acc, accumulate=True)
    torch.cuda.synchronize()
    got = _np(out)
    assert _rel(got, ref) <= 2.0 ** -8 and np.abs(got - ref).max() <= 2.0 ** -7 * np.abs(ref).max()
    if padded:
        assert (out_full[:, N:] == 0).all()
    got32 = _np(f32)
    assert _rel(got32, ref) <= 1e-5 and np.abs(got32 - ref).max() <= 1e-4 * np.abs(ref).max()
    gotacc = _np(acc) - 1.5
    assert np.abs(gotacc - ref).max() <= 1e-4 * np.abs(ref).max()


def _layer_inputs(B, S, D, Hq, Hkv, dh, dm, seed):
    g = torch.Generator().manual_seed(seed)
    S_local = S // D
    x = (torch.randn(B, S_local, dm, generator=g) / dm ** 0.5).to(torch.bfloat16)
    w_qkv = torch.randn((Hq + 2 * Hkv) * dh, dm, generator=g).to(torch.bfloat16)
    w_o = (torch.randn(dm, Hq * dh, generator=g) / (Hq * dh) ** 0.5).to(torch.bfloat16)
    k = torch.randn(B, S, Hkv, dh, generator=g).to(torch.bfloat16)
    v = torch.randn(B, S, Hkv, dh, generator=g).to(torch.bfloat16)
    return x, w_qkv, w_o, k, v


LAYER_CASES = [  # (B, S_total, D, rank, Hq, Hkv, dh, d_model, shards per group)
    (1, 512, 4, 1, 8, 4, 64, 256, 1),
    (1, 512, 4, 1, 8, 4, 64, 256, 2),
    (1, 512, 4, 1, 8, 4, 64, 256, 4),
    (1, 1024, 2, 0, 4, 2, 128, 512, 1),
    (1, 1024, 2, 0, 4, 2, 128, 512, 0),
    (2, 256, 2, 1, 4, 4, 64, 128, 1),
    (1, 1200, 3, 2, 6, 3, 128, 384, 1),   # ragged: C = 200
    (1, 1200, 3, 2, 6, 3, 128, 384, 3),
    (1, 2048, 8, 3, 8, 8, 128, 256, 1),   # D = 8, one query head per shard
    (1, 2048, 8, 3, 8, 8, 128, 256, 0),
    (1, 1024, 1, 0, 4, 2, 128, 256, 0),   # D = 1: one shard, the Ulysses layout
    (1, 512, 2, 1, 4, 2, 256, 256, 1),    # dh 256
    (1, 512, 2, 1, 4, 2, 256, 256, 2),
]


@pytest.mark.parametrize("case", LAYER_CASES, ids=lambda c: "B{}_S{}_D{}_r{}_H{}x{}_d{}_m{}_G{}".format(*c))
def test_layer_vs_oracle(case):
    B, S, D, r, Hq, Hkv, dh, dm, G = case
    _note(f"layer {case}")
    x, w_qkv, w_o, k, v = _layer_inputs(B, S, D, Hq, Hkv, dh, dm, seed=S + D + r)
    pos = oracle.zigzag_positions(S, D, r)
    k_in = k.clone()
    k_in[:, torch.as_tensor(pos)] = 77.0  # the rank's rows must be overwritten
    kd, vd = k_in.to(DEV), v.to(DEV)
    y = tsp.attn_layer_fwd(x.to(DEV), w_qkv.to(DEV), w_o.to(DEV), kd, vd, D=D, rank=r, Hq=Hq, Hkv=Hkv, dh=dh,
                           shards_per_group=G)
    torch.cuda.synchronize()
    ref_y, ref_k, ref_v = oracle.tsp_layer.attention_layer(x, w_qkv, w_o, k_in, v, D, r, Hq, Hkv, dh)
    got = _np(y)
    assert np.isfinite(got).all()
    assert _rel(got, ref_y) <= 2e-2, _rel(got, ref_y)
    assert np.abs(got - ref_y).max() <= 2.0 ** -4 * np.abs(ref_y).max()
    gk, gv = _np(kd), _np(vd)
    assert np.abs(gk[:, pos] - ref_k[:, pos]).max() <= 2.0 ** -7 * np.abs(ref_k[:, pos]).max()
    assert np.abs(gv[:, pos] - ref_v[:, pos]).max() <= 2.0 ** -7 * np.abs(ref_v[:, pos]).max()
    other = np.setdiff1d(np.arange(S), pos)
    assert torch.equal(kd.cpu()[:, torch.as_tensor(other)], k_in[:, torch.as_tensor(other)])
    assert torch.equal(vd.cpu()[:, torch.as_tensor(other)], v[:, torch.as_tensor(other)])


@pytest.mark.parametrize("G", [0, 1])
def test_layer_full_size_sampled_rows(G):
    """The 7B-dense shard's attention layer (d_model 4096, 32 heads of 128, 32K tokens,
    rank 3 of 8): every output column of sampled rows against the oracle's pieces."""
    B, S, D, r, Hq, Hkv, dh, dm = 1, 32768, 8, 3, 32, 32, 128, 4096
    _note(f"layer full size G={G}")
    x, w_qkv, w_o, k, v = _layer_inputs(B, S, D, Hq, Hkv, dh, dm, seed=5)
    kd, vd = k.to(DEV), v.to(DEV)
    y = tsp.attn_layer_fwd(x.to(DEV), w_qkv.to(DEV), w_o.to(DEV), kd, vd, D=D, rank=r, Hq=Hq, Hkv=Hkv, dh=dh,
                           shards_per_group=G)
    torch.cuda.synchronize()
    C = S // (2 * D)
    rows = np.concatenate([np.arange(0, 16), np.arange(C - 8, C + 8), np.arange(2 * C - 16, 2 * C)])
    xf = x.double().numpy()
    W = w_qkv.double().numpy()
    pos = oracle.zigzag_positions(S, D, r)
    K = k.double().numpy()
    V = v.double().numpy()
    K[:, pos] = (xf @ W[Hq * dh:(Hq + Hkv) * dh].T).reshape(B, 2 * C, Hkv, dh)
    V[:, pos] = (xf @ W[(Hq + Hkv) * dh:].T).reshape(B, 2 * C, Hkv, dh)
    q = (xf @ W[:Hq * dh].T).reshape(B, 2 * C, Hq, dh)
    o, _ = oracle.causal_attention(q, K, V, D, r, rows=rows)
    ref = o.reshape(B, len(rows), Hq * dh) @ w_o.double().numpy().T
    got = _np(y[:, torch.as_tensor(rows)])
    assert _rel(got, ref) <= 2e-2 and np.abs(got - ref).max() <= 2.0 ** -4 * np.abs(ref).max()


def test_layer_workspace_counted_in_bytes_and_on_device():
    """A workspace of any element type is sized in bytes; one on the host is refused."""
    B, S, D, r, Hq, Hkv, dh, dm = 1, 512, 2, 1, 4, 2, 64, 128
    x, w_qkv, w_o, k, v = _layer_inputs(B, S, D, Hq, Hkv, dh, dm, seed=3)
    nbytes = tsp.attn_layer_workspace_bytes(B, S, D, Hq, Hkv, dh, dm, 1)
    args = (x.to(DEV), w_qkv.to(DEV), w_o.to(DEV))
    kd1, vd1, kd2, vd2 = k.to(DEV), v.to(DEV), k.to(DEV), v.to(DEV)
    y1 = tsp.attn_layer_fwd(*args, kd1, vd1, D=D, rank=r, Hq=Hq, Hkv=Hkv, dh=dh, shards_per_group=1)
    ws = torch.empty((nbytes + 3) // 4, dtype=torch.float32, device=DEV)
    y2 = tsp.attn_layer_fwd(*args, kd2, vd2, D=D, rank=r, Hq=Hq, Hkv=Hkv, dh=dh, shards_per_group=1, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    with pytest.raises(tsp.TspAttnError):
        tsp.attn_layer_fwd(*args, kd1, vd1, D=D, rank=r, Hq=Hq, Hkv=Hkv, dh=dh, shards_per_group=1,
                           workspace=torch.empty(nbytes, dtype=torch.uint8))
