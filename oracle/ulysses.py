"""Plain CPU oracle of the Ulysses layout changes around the one-rank (D = 1) attention.

TEST INFRASTRUCTURE ONLY: used by tests/, never by the product path; shares no code with
the HIP library.

What is computed:

* "Tensor, pipeline e sequence parallelism", section 01 (Conceito), sequence-parallel
  paragraph: DeepSpeed-Ulysses transposes between sequence partitions and head
  partitions with an all-to-all, so that every rank computes full attention for a
  subset of the heads, and transposes back afterwards.
* "AutoSP ...", section 2.A item 2 (buffer resizing): attention buffers hold the whole
  sequence for a subset of heads, MLP buffers a part of the sequence for the whole model
  width; item 3 (communication insertion): all-to-all at the boundaries of attention.

Readings taken where the pages are silent:

* P ranks; before attention rank p holds the contiguous sequence chunk p of S_local
  tokens, [B, S_local, H, dh], all heads;
* heads are split contiguously: rank r computes heads [r*H/P, (r+1)*H/P) (H divisible by
  P; for GQA the KV heads are split the same way, so Hkv must be divisible by P too);
* the all-to-all sends rank p's block for rank r (its tokens, r's heads) to rank r, and
  rank r stores the blocks in source order, i.e. in sequence order.

Every function is a plain index rearrangement written with explicit slices; the pins
in tests/pins.py check them against element-by-element loops and the head-subset
definition.
"""

from __future__ import annotations

import numpy as np


def _arr(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").numpy()
    return np.asarray(x)


def heads_of_rank(H: int, P: int, r: int) -> range:
    """Contiguous head split: the heads rank r attends to."""
    if H % P != 0:
        raise ValueError("H must be divisible by P")
    Hl = H // P
    return range(r * Hl, (r + 1) * Hl)


def pack_heads(x, P: int) -> np.ndarray:
    """Before the all-to-all: x [B, S_local, H, dh] -> send [P, B, S_local, H/P, dh], where
    send[r] is this rank's tokens for the heads of rank r (the block sent to rank r)."""
    x = _arr(x)
    B, S_local, H, dh = x.shape
    hs = [heads_of_rank(H, P, r) for r in range(P)]
    return np.stack([x[:, :, hs[r].start:hs[r].stop, :] for r in range(P)], axis=0)


def unpack_heads(send, P: int) -> np.ndarray:
    """Inverse of pack_heads: [P, B, S_local, H/P, dh] -> [B, S_local, H, dh]."""
    send = _arr(send)
    _, B, S_local, Hl, dh = send.shape
    x = np.empty((B, S_local, Hl * P, dh), dtype=send.dtype)
    for r in range(P):
        hs = heads_of_rank(Hl * P, P, r)
        x[:, :, hs.start:hs.stop, :] = send[r]
    return x


def gather_sequence(recv) -> np.ndarray:
    """After the all-to-all: recv [P, B, S_local, Hl, dh] (block p from rank p, i.e. sequence
    chunk p) -> [B, P*S_local, Hl, dh], the whole sequence for this rank's heads."""
    recv = _arr(recv)
    P, B, S_local, Hl, dh = recv.shape
    full = np.empty((B, P * S_local, Hl, dh), dtype=recv.dtype)
    for p in range(P):
        full[:, p * S_local:(p + 1) * S_local] = recv[p]
    return full


def scatter_sequence(full, P: int) -> np.ndarray:
    """Inverse of gather_sequence: [B, P*S_local, Hl, dh] -> [P, B, S_local, Hl, dh], block p
    being the chunk sent back to rank p."""
    full = _arr(full)
    B, S, Hl, dh = full.shape
    if S % P != 0:
        raise ValueError("sequence length must be divisible by P")
    S_local = S // P
    return np.stack([full[:, p * S_local:(p + 1) * S_local] for p in range(P)], axis=0)


def all_to_all(sends):
    """The exchange itself (the collective, simulated): sends[p][r] goes to rank r, which
    stores it as block p. Returns the list of per-rank receive buffers."""
    P = len(sends)
    return [np.stack([_arr(sends[p])[r] for p in range(P)], axis=0) for r in range(P)]
