"""Ulysses layout changes (tsp_ulysses_*) vs the oracle, through the C ABI, on an MI355X:
bit-exact copies, at small ragged shapes and at the full 8-rank shape, plus a simulated
P-rank Ulysses attention on one GPU against the unsharded oracle attention."""

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


def _bits(shape, dtype, seed):
    """Arbitrary bit patterns (NaN and inf payloads included): a permute must copy bits."""
    g = torch.Generator().manual_seed(seed)
    if dtype == torch.bfloat16:
        return torch.randint(-32768, 32767, shape, generator=g, dtype=torch.int16).view(torch.bfloat16)
    return torch.randint(-2 ** 31, 2 ** 31 - 1, shape, generator=g, dtype=torch.int32).view(torch.float32)


def _same_bits(a: torch.Tensor, b: np.ndarray):
    a = a.cpu()
    iv = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    return np.array_equal(a.view(iv).numpy(), torch.from_numpy(np.ascontiguousarray(b)).view(iv).numpy())


CASES = [  # (B, S_local, H, dh, P, dtype)
    (1, 16, 8, 128, 4, torch.bfloat16),
    (2, 7, 6, 64, 3, torch.bfloat16),     # ragged sizes
    (1, 5, 4, 256, 2, torch.float32),
    (1, 3, 24, 256, 4, torch.bfloat16),   # the lesson's 24 heads over degree 4
    (1, 1, 1, 128, 1, torch.bfloat16),
    (2, 33, 12, 128, 6, torch.float32),
    (3, 100, 8, 64, 8, torch.bfloat16),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_S{}_H{}_d{}_P{}_{}".format(*c[:5], str(c[5])[6:]))
def test_permutes_bit_exact(case):
    B, S_local, H, dh, P, dtype = case
    _note(f"ulysses {case}")
    iv = torch.int16 if dtype == torch.bfloat16 else torch.int32
    x = _bits((B, S_local, H, dh), dtype, 1)
    send = tsp.ulysses_pack_heads(x.to(DEV), P)
    assert _same_bits(send, oracle.ulysses.pack_heads(x.view(iv).numpy(), P))
    assert _same_bits(tsp.ulysses_unpack_heads(send), x.view(iv).numpy())
    Hl = H // P
    recv = _bits((P, B, S_local, Hl, dh), dtype, 2)
    full = tsp.ulysses_gather_sequence(recv.to(DEV))
    assert _same_bits(full, oracle.ulysses.gather_sequence(recv.view(iv).numpy()))
    back = tsp.ulysses_scatter_sequence(full, P)
    assert _same_bits(back, recv.view(iv).numpy())
    torch.cuda.synchronize()


def test_permutes_full_shape():
    """The 8-rank Ulysses shape of the 128K head-subset workload: every rank holds 16384
    tokens of all 32 heads before the exchange, 4 heads of all 131072 tokens after."""
    w = workloads.BY_NAME["ulysses_head_subset_s128k"]
    P = 8
    S_local, H = w.S_total // P, w.Hq * P
    _note(f"ulysses full shape S_local={S_local} H={H}")
    x = _bits((1, S_local, H, w.dh), torch.bfloat16, 3)
    send = tsp.ulysses_pack_heads(x.to(DEV), P)
    assert _same_bits(send, oracle.ulysses.pack_heads(x.view(torch.int16).numpy(), P))
    full = tsp.ulysses_gather_sequence(send)  # as if every block came from another rank
    assert _same_bits(full, oracle.ulysses.gather_sequence(send.cpu().view(torch.int16).numpy()))


@pytest.mark.parametrize("P,Hkv", [(4, 4), (2, 2), (4, 8)])
def test_simulated_ulysses_attention(P, Hkv):
    """P ranks on one GPU: pack -> (exchange) -> gather -> one-rank causal attention over
    the rank's heads -> scatter -> (exchange) -> unpack equals the unsharded attention over
    all heads for every rank's tokens. The exchange is a plain copy standing in for the
    all-to-all."""
    B, S, Hq, dh = 1, 1024, 8, 128
    _note(f"ulysses attention P={P} Hkv={Hkv}")
    q = workloads.make_grad((B, S, Hq, dh), 41, torch.bfloat16)
    k = workloads.make_grad((B, S, Hkv, dh), 42, torch.bfloat16)
    v = workloads.make_grad((B, S, Hkv, dh), 43, torch.bfloat16)
    S_local = S // P

    def exchange(sends):
        return [torch.stack([sends[p][r] for p in range(P)], dim=0).contiguous() for r in range(P)]

    def to_heads(t):
        shards = [t[:, p * S_local:(p + 1) * S_local].contiguous().to(DEV) for p in range(P)]
        recvs = exchange([tsp.ulysses_pack_heads(x, P) for x in shards])
        return [tsp.ulysses_gather_sequence(rv) for rv in recvs]

    qs, ks, vs = to_heads(q), to_heads(k), to_heads(v)
    outs = [tsp.fwd(qs[r], ks[r], vs[r], D=1, rank=0)[0] for r in range(P)]
    back = exchange([tsp.ulysses_scatter_sequence(o, P) for o in outs])
    got = torch.cat([tsp.ulysses_unpack_heads(b) for b in back], dim=1).float().cpu().numpy()
    torch.cuda.synchronize()
    ref, _ = oracle.causal_attention(q, k, v, 1, 0)
    err = np.abs(got - ref).max()
    assert err <= 2e-2, err
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel <= 1e-2, rel


def test_permute_canaries():
    _note("ulysses canaries")
    x = _bits((2, 9, 8, 128), torch.bfloat16, 5).to(DEV)
    big = torch.full((x.numel() + 512,), 1.0, dtype=x.dtype, device=DEV)
    out = big[:x.numel()].view(4, 2, 9, 2, 128)
    tsp.ulysses_pack_heads(x, 4, out=out)
    torch.cuda.synchronize()
    assert (big[x.numel():] == 1).all()
