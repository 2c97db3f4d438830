"""Python binding of the MI355X per-rank zigzag / GQA causal attention library.

Argument marshalling only: every step of the computation runs in the HIP kernels of
``libtsp_attn.so`` (built from ``csrc/`` by ``python -m sequence_causal_attention_amd.build``).
PyTorch provides device memory and the stream. There is no fallback: if the library is
missing or a call fails, an exception is raised.

The operation ("Folding Tensor and Sequence Parallelism for Memory-Efficient Transformer
Training & Inference", section 2, attention layers; "AutoSP ...", section 2.A item 4;
"Tensor, pipeline e sequence parallelism", section 01, GQA and sequence-parallel
paragraphs): rank ``rank`` of ``D`` holds chunks ``rank`` and ``2D-1-rank`` of the
sequence (2D chunks of C = S_total/(2D) tokens) as its local queries and attends
causally, by global position, to the full-sequence keys/values.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# TSP_ATTN_LIB names another build of the same library (the host-sanitized one of the
# build script's --host-sanitize check); by default the in-tree libtsp_attn.so
LIB_PATH = os.environ.get("TSP_ATTN_LIB") or os.path.join(_HERE, "libtsp_attn.so")

TSP_OK = 0
TSP_EINVAL = -1
TSP_EUNSUPPORTED = -2
TSP_ELAUNCH = -3
TSP_EINTERNAL = -4
TSP_BF16 = 0
TSP_F32 = 1
MAX_NOALLOC_ROWS = 4 * 1024 * 1024  # TSP_BWD_NOALLOC_MAX_ROWS: B * Hq * 2C of tsp_attn_bwd_noalloc

# Every entry point the header declares, with its ctypes signature.
_I64 = ctypes.c_int64
_VP = ctypes.c_void_p
SIGNATURES = {
    "tsp_attn_fwd": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                                    ctypes.c_int, _VP]),
    "tsp_attn_fwd_range": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                                          _I64, _I64, ctypes.c_int, ctypes.c_int, _VP]),
    "tsp_attn_fwd_range2": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                                           _I64, _I64, _I64, _I64, ctypes.c_int, ctypes.c_int, _VP]),
    "tsp_attn_fwd_ring": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                                         _VP, ctypes.c_int32, ctypes.c_int32, _VP, ctypes.c_int, _VP]),
    "tsp_attn_merge": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _I64, ctypes.c_int, _VP]),
    "tsp_attn_bwd": (ctypes.c_int, [_VP] * 10 + [_I64] * 7 + [ctypes.c_int, _VP]),
    "tsp_attn_bwd_noalloc": (ctypes.c_int, [_VP] * 9 + [_I64] * 7 + [ctypes.c_int, _VP]),
    "tsp_gemm_bf16_nt": (ctypes.c_int, [_VP, _VP, _VP] + [_I64] * 6 + [ctypes.c_int, _VP]),
    "tsp_attn_layer_workspace_bytes": (ctypes.c_int, [_I64] * 8 + [ctypes.POINTER(_I64)]),
    "tsp_attn_layer_fwd": (ctypes.c_int, [_VP] * 7 + [_I64] * 10 + [_VP]),
    "tsp_ulysses_pack_heads": (ctypes.c_int, [_VP, _VP] + [_I64] * 5 + [ctypes.c_int, _VP]),
    "tsp_ulysses_unpack_heads": (ctypes.c_int, [_VP, _VP] + [_I64] * 5 + [ctypes.c_int, _VP]),
    "tsp_ulysses_gather_sequence": (ctypes.c_int, [_VP, _VP] + [_I64] * 5 + [ctypes.c_int, _VP]),
    "tsp_ulysses_scatter_sequence": (ctypes.c_int, [_VP, _VP] + [_I64] * 5 + [ctypes.c_int, _VP]),
    "tsp_attn_zigzag_positions": (ctypes.c_int, [_I64, _I64, _I64, ctypes.POINTER(_I64)]),
    "tsp_attn_zigzag_positions_device": (ctypes.c_int, [_VP, _I64, _I64, _I64, _VP]),
    "tsp_attn_unmasked_pairs": (_I64, [_I64, _I64, _I64]),
    "tsp_attn_schedule": (ctypes.c_int, [_I64, _I64, _I64, _I64, _I64, _I64, _I64, ctypes.c_int,
                                         ctypes.POINTER(_I64), ctypes.POINTER(_I64), ctypes.POINTER(_I64)]),
    "tsp_attn_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "tsp_attn_last_error": (ctypes.c_char_p, []),
}

_lib_handle = None


class TspAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"tsp_attn status {status}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m sequence_causal_attention_amd.build`"
            )
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib_handle = h
    return _lib_handle


def _check(status: int):
    if status != TSP_OK:
        msg = lib().tsp_attn_last_error().decode() or lib().tsp_attn_strerror(status).decode()
        raise TspAttnError(status, msg)


def _on_device(device, **tensors):
    """Every tensor must live on `device` (a host or other-device pointer would reach the
    kernels as a wild address)."""
    for name, t in tensors.items():
        if not t.is_cuda or t.device != device:
            raise TspAttnError(TSP_EINVAL, f"{name} must be on {device}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return TSP_BF16
    if t.dtype == torch.float32:
        return TSP_F32
    raise TspAttnError(TSP_EUNSUPPORTED, f"unsupported element type {t.dtype}")


def fwd(q_local: torch.Tensor, k_full: torch.Tensor, v_full: torch.Tensor, *, D: int, rank: int,
        out: torch.Tensor | None = None, lse: torch.Tensor | None = None, stream=None, kv_range=None,
        kv_range2=None, accumulate: bool = False):
    """Causal attention of this rank's zigzag queries against the full K/V.

    q_local [B, 2C, Hq, dh], k_full / v_full [B, S_total, Hkv, dh]: contiguous, same
    device and dtype (bf16 or fp32). Returns (out [B, 2C, Hq, dh] same dtype,
    lse [B, Hq, 2C] fp32). ``out`` / ``lse`` may be passed in preallocated.
    Without a key range this is ``tsp_attn_fwd``.
    ``kv_range=(begin, end)`` restricts the keys (tsp_attn_fwd_range): rows without a
    visible key in the range get out = 0, lse = -inf. With ``accumulate=True`` the
    partial over the range is merged into the ``out`` / ``lse`` passed in (a result over
    disjoint keys) instead of overwriting them. ``kv_range2=(begin2, end2)``, after
    ``kv_range``, adds a second key range to the same call (tsp_attn_fwd_range2).
    The call is asynchronous on ``stream`` (default: the current stream).
    """
    for name, t in (("q_local", q_local), ("k_full", k_full), ("v_full", v_full)):
        if not t.is_cuda:
            raise TspAttnError(TSP_EINVAL, f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise TspAttnError(TSP_EINVAL, f"{name} must be contiguous")
        if t.dim() != 4:
            raise TspAttnError(TSP_EINVAL, f"{name} must be 4-D [B, S, H, dh]")
    if not (q_local.dtype == k_full.dtype == v_full.dtype):
        raise TspAttnError(TSP_EINVAL, "q_local, k_full and v_full must share one dtype")
    if not (q_local.device == k_full.device == v_full.device):
        raise TspAttnError(TSP_EINVAL, "inputs must be on one device")
    B, S_local, Hq, dh = q_local.shape
    Bk, S_total, Hkv, dhk = k_full.shape
    if tuple(v_full.shape) != tuple(k_full.shape) or Bk != B or dhk != dh:
        raise TspAttnError(TSP_EINVAL, "k_full / v_full must be [B, S_total, Hkv, dh] matching q_local")
    if D < 1 or S_total % (2 * D) != 0 or S_local != S_total // D:
        raise TspAttnError(TSP_EINVAL, f"q_local must hold S_total / D = {S_total // max(D, 1)} rows")
    code = _dtype_code(q_local)
    if accumulate and (out is None or lse is None):
        raise TspAttnError(TSP_EINVAL, "accumulate needs the running out and lse")
    if out is None:
        out = torch.empty_like(q_local)
    if lse is None:
        lse = torch.empty((B, Hq, S_local), dtype=torch.float32, device=q_local.device)
    if out.shape != q_local.shape or out.dtype != q_local.dtype or not out.is_contiguous():
        raise TspAttnError(TSP_EINVAL, "out must match q_local")
    if tuple(lse.shape) != (B, Hq, S_local) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise TspAttnError(TSP_EINVAL, "lse must be float32 [B, Hq, S_local]")
    _on_device(q_local.device, out=out, lse=lse)
    if stream is None:
        stream = torch.cuda.current_stream(q_local.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    lo, hi = (0, S_total) if kv_range is None else (int(kv_range[0]), int(kv_range[1]))
    with torch.cuda.device(q_local.device):
        if kv_range is None and kv_range2 is None and not accumulate:  # the whole key sequence
            st = lib().tsp_attn_fwd(q_local.data_ptr(), k_full.data_ptr(), v_full.data_ptr(), out.data_ptr(),
                                    lse.data_ptr(), B, S_total, D, rank, Hq, Hkv, dh, code, handle)
        elif kv_range2 is None:
            st = lib().tsp_attn_fwd_range(q_local.data_ptr(), k_full.data_ptr(), v_full.data_ptr(), out.data_ptr(),
                                          lse.data_ptr(), B, S_total, D, rank, Hq, Hkv, dh, lo, hi,
                                          int(bool(accumulate)), code, handle)
        else:
            lo2, hi2 = int(kv_range2[0]), int(kv_range2[1])
            st = lib().tsp_attn_fwd_range2(q_local.data_ptr(), k_full.data_ptr(), v_full.data_ptr(), out.data_ptr(),
                                           lse.data_ptr(), B, S_total, D, rank, Hq, Hkv, dh, lo, hi, lo2, hi2,
                                           int(bool(accumulate)), code, handle)
    _check(st)
    return out, lse


def fwd_ring(q_local: torch.Tensor, k_full: torch.Tensor, v_full: torch.Tensor, *, D: int, rank: int,
             out: torch.Tensor | None = None, lse: torch.Tensor | None = None, chunk_ready: torch.Tensor | None = None,
             ready_value: int = 1, spin_limit: int = 1 << 20, wait_status: torch.Tensor | None = None, stream=None):
    """The same attention as fwd(), swept chunk by chunk in ring arrival order
    (tsp_attn_fwd_ring): the rank's own two chunks in one launch, then every peer's chunks
    in a second, which reads chunk c only once chunk_ready[c] == ready_value.

    chunk_ready: int32 [2D] on the inputs' device, or None (all chunks present). With
    flags, wait_status (int32 [1], same device) receives bit 0 if a wait gave up after
    spin_limit polls. bf16 only. Returns (out, lse)."""
    for name, t in (("q_local", q_local), ("k_full", k_full), ("v_full", v_full)):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise TspAttnError(TSP_EINVAL, f"{name} must be a contiguous 4-D GPU tensor")
    if not (q_local.dtype == k_full.dtype == v_full.dtype) or not (q_local.device == k_full.device == v_full.device):
        raise TspAttnError(TSP_EINVAL, "q_local, k_full and v_full must share one dtype and device")
    B, S_local, Hq, dh = q_local.shape
    Bk, S_total, Hkv, dhk = k_full.shape
    if tuple(v_full.shape) != tuple(k_full.shape) or Bk != B or dhk != dh:
        raise TspAttnError(TSP_EINVAL, "k_full / v_full must be [B, S_total, Hkv, dh] matching q_local")
    if D < 1 or S_total % (2 * D) != 0 or S_local != S_total // D:
        raise TspAttnError(TSP_EINVAL, f"q_local must hold S_total / D = {S_total // max(D, 1)} rows")
    code = _dtype_code(q_local)
    out = torch.empty_like(q_local) if out is None else out
    if lse is None:
        lse = torch.empty((B, Hq, S_local), dtype=torch.float32, device=q_local.device)
    if out.shape != q_local.shape or out.dtype != q_local.dtype or not out.is_contiguous():
        raise TspAttnError(TSP_EINVAL, "out must match q_local")
    if tuple(lse.shape) != (B, Hq, S_local) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise TspAttnError(TSP_EINVAL, "lse must be float32 [B, Hq, S_local]")
    _on_device(q_local.device, out=out, lse=lse)
    ready_ptr = status_ptr = None
    if chunk_ready is not None:
        if (chunk_ready.dtype != torch.int32 or chunk_ready.numel() != 2 * D or not chunk_ready.is_contiguous()
                or wait_status is None or wait_status.dtype != torch.int32 or wait_status.numel() < 1):
            raise TspAttnError(TSP_EINVAL, "chunk_ready must be int32 [2D] and wait_status int32 [1]")
        _on_device(q_local.device, chunk_ready=chunk_ready, wait_status=wait_status)
        ready_ptr, status_ptr = chunk_ready.data_ptr(), wait_status.data_ptr()
    if stream is None:
        stream = torch.cuda.current_stream(q_local.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q_local.device):
        st = lib().tsp_attn_fwd_ring(q_local.data_ptr(), k_full.data_ptr(), v_full.data_ptr(), out.data_ptr(),
                                     lse.data_ptr(), B, S_total, D, rank, Hq, Hkv, dh, ready_ptr, int(ready_value),
                                     int(spin_limit), status_ptr, code, handle)
    _check(st)
    return out, lse


def merge(out_a: torch.Tensor, lse_a: torch.Tensor, out_b: torch.Tensor, lse_b: torch.Tensor, *,
          out: torch.Tensor | None = None, lse: torch.Tensor | None = None, stream=None):
    """Log-sum-exp merge of two partials (tsp_attn_merge). out/lse default to new
    tensors; pass out=out_a, lse=lse_a to accumulate in place."""
    for t in (out_a, lse_a, out_b, lse_b):
        if not t.is_cuda or not t.is_contiguous():
            raise TspAttnError(TSP_EINVAL, "merge operands must be contiguous GPU tensors")
    if out_a.shape != out_b.shape or out_a.dtype != out_b.dtype or out_a.dim() != 4:
        raise TspAttnError(TSP_EINVAL, "out_a / out_b must match, [B, S_local, Hq, dh]")
    B, S_local, Hq, dh = out_a.shape
    if (tuple(lse_a.shape) != (B, Hq, S_local) or lse_b.shape != lse_a.shape or lse_a.dtype != torch.float32
            or lse_b.dtype != torch.float32):
        raise TspAttnError(TSP_EINVAL, "lse_a / lse_b must be float32 [B, Hq, S_local]")
    code = _dtype_code(out_a)
    out = torch.empty_like(out_a) if out is None else out
    lse = torch.empty_like(lse_a) if lse is None else lse
    if (out.shape != out_a.shape or out.dtype != out_a.dtype or lse.shape != lse_a.shape
            or lse.dtype != torch.float32 or not out.is_contiguous() or not lse.is_contiguous()):
        raise TspAttnError(TSP_EINVAL, "out / lse must match the operands")
    _on_device(out_a.device, lse_a=lse_a, out_b=out_b, lse_b=lse_b, out=out, lse=lse)
    if stream is None:
        stream = torch.cuda.current_stream(out_a.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(out_a.device):
        st = lib().tsp_attn_merge(out_a.data_ptr(), lse_a.data_ptr(), out_b.data_ptr(), lse_b.data_ptr(),
                                  out.data_ptr(), lse.data_ptr(), B, S_local, Hq, dh, code, handle)
    _check(st)
    return out, lse


def _bwd_check(q_local, k_full, v_full, out, lse, dout, outputs):
    """Validates the backward's tensors; `outputs` are (name, tensor, like) triples.
    Returns (B, S_local, Hq, dh, S_total, Hkv, dtype code)."""
    ins = (("q_local", q_local), ("k_full", k_full), ("v_full", v_full), ("out", out), ("dout", dout))
    for name, t in ins + (("lse", lse),):
        if not t.is_cuda or not t.is_contiguous():
            raise TspAttnError(TSP_EINVAL, f"{name} must be a contiguous GPU tensor")
    if not (q_local.dtype == k_full.dtype == v_full.dtype == out.dtype == dout.dtype):
        raise TspAttnError(TSP_EINVAL, "q_local, k_full, v_full, out and dout must share one dtype")
    if q_local.dim() != 4 or k_full.dim() != 4:
        raise TspAttnError(TSP_EINVAL, "tensors must be 4-D [B, S, H, dh]")
    B, S_local, Hq, dh = q_local.shape
    _, S_total, Hkv, _ = k_full.shape
    if v_full.shape != k_full.shape or out.shape != q_local.shape or dout.shape != q_local.shape:
        raise TspAttnError(TSP_EINVAL, "shape mismatch between the forward's tensors")
    if tuple(lse.shape) != (B, Hq, S_local) or lse.dtype != torch.float32:
        raise TspAttnError(TSP_EINVAL, "lse must be float32 [B, Hq, S_local]")
    code = _dtype_code(q_local)
    for name, t, ref in outputs:
        if t.shape != ref.shape or t.dtype != ref.dtype or not t.is_contiguous() or not t.is_cuda:
            raise TspAttnError(TSP_EINVAL, f"{name} must match {tuple(ref.shape)} {ref.dtype}")
    _on_device(q_local.device, k_full=k_full, v_full=v_full, out=out, lse=lse, dout=dout,
               **{name: t for name, t, _ in outputs})
    return B, S_local, Hq, dh, S_total, Hkv, code


def _handle(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def bwd(q_local: torch.Tensor, k_full: torch.Tensor, v_full: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
        dout: torch.Tensor, *, D: int, rank: int, dq=None, dk=None, dv=None, delta=None, stream=None):
    """Backward of ``fwd`` (tsp_attn_bwd): returns (dq [B, 2C, Hq, dh], dk, dv
    [B, S_total, Hkv, dh] -- this rank's partial K/V gradients -- and delta [B, Hq, 2C]).
    Outputs may be passed in preallocated. bf16 or fp32."""
    dq = torch.empty_like(q_local) if dq is None else dq
    dk = torch.empty_like(k_full) if dk is None else dk
    dv = torch.empty_like(v_full) if dv is None else dv
    delta = torch.empty_like(lse) if delta is None else delta
    B, S_local, Hq, dh, S_total, Hkv, code = _bwd_check(
        q_local, k_full, v_full, out, lse, dout,
        (("dq", dq, q_local), ("dk", dk, k_full), ("dv", dv, v_full), ("delta", delta, lse)))
    handle = _handle(stream, q_local.device)
    with torch.cuda.device(q_local.device):
        st = lib().tsp_attn_bwd(q_local.data_ptr(), k_full.data_ptr(), v_full.data_ptr(), out.data_ptr(),
                                lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                delta.data_ptr(), B, S_total, D, rank, Hq, Hkv, dh, code, handle)
    _check(st)
    return dq, dk, dv, delta


def bwd_noalloc(q_local: torch.Tensor, k_full: torch.Tensor, v_full: torch.Tensor, out: torch.Tensor,
                lse: torch.Tensor, dout: torch.Tensor, *, D: int, rank: int, dq: torch.Tensor, dk: torch.Tensor,
                dv: torch.Tensor, stream=None):
    """The backward through tsp_attn_bwd_noalloc: the caller passes every output (dq, dk,
    dv) and the library allocates nothing (its delta lives in a static device array of
    MAX_NOALLOC_ROWS floats per GPU, shared by every call on that GPU). Returns (dq, dk, dv)."""
    B, S_local, Hq, dh, S_total, Hkv, code = _bwd_check(
        q_local, k_full, v_full, out, lse, dout, (("dq", dq, q_local), ("dk", dk, k_full), ("dv", dv, v_full)))
    handle = _handle(stream, q_local.device)
    with torch.cuda.device(q_local.device):
        st = lib().tsp_attn_bwd_noalloc(q_local.data_ptr(), k_full.data_ptr(), v_full.data_ptr(), out.data_ptr(),
                                        lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                        B, S_total, D, rank, Hq, Hkv, dh, code, handle)
    _check(st)
    return dq, dk, dv


def _ulysses_call(fn, src: torch.Tensor, out_shape, B, S_local, H, dh, P, out=None, stream=None):
    if not src.is_cuda or not src.is_contiguous():
        raise TspAttnError(TSP_EINVAL, "input must be a contiguous GPU tensor")
    code = _dtype_code(src)
    out = torch.empty(out_shape, dtype=src.dtype, device=src.device) if out is None else out
    if tuple(out.shape) != tuple(out_shape) or out.dtype != src.dtype or not out.is_contiguous():
        raise TspAttnError(TSP_EINVAL, f"output must be contiguous {tuple(out_shape)} {src.dtype}")
    _on_device(src.device, out=out)
    if stream is None:
        stream = torch.cuda.current_stream(src.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(src.device):
        _check(fn(src.data_ptr(), out.data_ptr(), B, S_local, H, dh, P, code, handle))
    return out


def ulysses_pack_heads(x: torch.Tensor, P: int, out=None, stream=None) -> torch.Tensor:
    """x [B, S_local, H, dh] -> send [P, B, S_local, H/P, dh] (block r goes to rank r)."""
    B, S_local, H, dh = x.shape
    return _ulysses_call(lib().tsp_ulysses_pack_heads, x, (P, B, S_local, H // max(P, 1), dh), B, S_local, H, dh,
                         P, out, stream)


def ulysses_unpack_heads(send: torch.Tensor, out=None, stream=None) -> torch.Tensor:
    """send [P, B, S_local, H/P, dh] -> x [B, S_local, H, dh]."""
    P, B, S_local, Hl, dh = send.shape
    return _ulysses_call(lib().tsp_ulysses_unpack_heads, send, (B, S_local, Hl * P, dh), B, S_local, Hl * P, dh, P,
                         out, stream)


def ulysses_gather_sequence(recv: torch.Tensor, out=None, stream=None) -> torch.Tensor:
    """recv [P, B, S_local, Hl, dh] (block p = sequence chunk p) -> [B, P*S_local, Hl, dh]."""
    P, B, S_local, Hl, dh = recv.shape
    return _ulysses_call(lib().tsp_ulysses_gather_sequence, recv, (B, P * S_local, Hl, dh), B, S_local, Hl, dh, P,
                         out, stream)


def ulysses_scatter_sequence(full: torch.Tensor, P: int, out=None, stream=None) -> torch.Tensor:
    """full [B, S, Hl, dh] -> send [P, B, S/P, Hl, dh] (block p goes back to rank p)."""
    B, S, Hl, dh = full.shape
    if P < 1 or S % P != 0:
        raise TspAttnError(TSP_EINVAL, "sequence length must be divisible by P")
    return _ulysses_call(lib().tsp_ulysses_scatter_sequence, full, (P, B, S // P, Hl, dh), B, S // P, Hl, dh, P,
                         out, stream)


def gemm_nt(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor | None = None, accumulate=False, stream=None):
    """C = A B^T (tsp_gemm_bf16_nt) for bf16 a [M, K], b [N, K]. ``out`` bf16 (stored) or
    fp32 (stored, or added to when ``accumulate``)."""
    for t in (a, b):
        if not t.is_cuda or t.dtype != torch.bfloat16 or t.dim() != 2 or t.stride(1) != 1:
            raise TspAttnError(TSP_EINVAL, "a and b must be 2-D bf16 GPU tensors with unit column stride")
    M, K = a.shape
    N = b.shape[0]
    out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device) if out is None else out
    if out.dim() != 2 or out.shape != (M, N) or out.stride(1) != 1:
        raise TspAttnError(TSP_EINVAL, "out must be [M, N] with unit column stride")
    if out.dtype not in (torch.bfloat16, torch.float32) or (accumulate and out.dtype != torch.float32):
        raise TspAttnError(TSP_EINVAL, "out must be bf16, or float32 (which accumulate needs)")
    if b.shape[1] != K:
        raise TspAttnError(TSP_EINVAL, "a and b must share K")
    _on_device(a.device, b=b, out=out)
    mode = 0 if out.dtype == torch.bfloat16 else (2 if accumulate else 1)
    if stream is None:
        stream = torch.cuda.current_stream(a.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(a.device):
        _check(lib().tsp_gemm_bf16_nt(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, a.stride(0), b.stride(0),
                                      out.stride(0), mode, handle))
    return out


def attn_layer_workspace_bytes(B, S_total, D, Hq, Hkv, dh, d_model, shards_per_group=0) -> int:
    n = _I64(0)
    _check(lib().tsp_attn_layer_workspace_bytes(B, S_total, D, Hq, Hkv, dh, d_model, shards_per_group,
                                                ctypes.byref(n)))
    return n.value


def attn_layer_fwd(x_local: torch.Tensor, w_qkv: torch.Tensor, w_o: torch.Tensor, k_gathered: torch.Tensor,
                   v_gathered: torch.Tensor, *, D: int, rank: int, Hq: int, Hkv: int, dh: int, shards_per_group=0,
                   y=None, workspace=None, stream=None):
    """One rank's TSP attention layer forward (tsp_attn_layer_fwd). k_gathered / v_gathered
    are updated in place at the rank's positions. ``shards_per_group``: weight shards per
    projection / attention launch (a divisor of D; 0 = automatic). Returns y_local
    [B, 2C, d_model]."""
    ts = (x_local, w_qkv, w_o, k_gathered, v_gathered)
    for t in ts:
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise TspAttnError(TSP_EINVAL, "layer tensors must be contiguous bf16 GPU tensors")
    B, S_local, d_model = x_local.shape
    S_total = k_gathered.shape[1]
    if tuple(w_qkv.shape) != ((Hq + 2 * Hkv) * dh, d_model) or tuple(w_o.shape) != (d_model, Hq * dh):
        raise TspAttnError(TSP_EINVAL, "weight shapes do not match Hq, Hkv, dh, d_model")
    if tuple(k_gathered.shape) != (B, S_total, Hkv, dh) or v_gathered.shape != k_gathered.shape:
        raise TspAttnError(TSP_EINVAL, "gathered K/V must be [B, S_total, Hkv, dh]")
    y = torch.empty_like(x_local) if y is None else y
    if (not y.is_cuda or y.dtype != torch.bfloat16 or not y.is_contiguous()
            or tuple(y.shape) != tuple(x_local.shape)):
        raise TspAttnError(TSP_EINVAL, "y must be a contiguous bf16 GPU tensor shaped like x_local")
    if workspace is None:
        nbytes = attn_layer_workspace_bytes(B, S_total, D, Hq, Hkv, dh, d_model, shards_per_group)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=x_local.device)
    if not workspace.is_contiguous():
        raise TspAttnError(TSP_EINVAL, "workspace must be contiguous")
    _on_device(x_local.device, w_qkv=w_qkv, w_o=w_o, k_gathered=k_gathered, v_gathered=v_gathered, y=y,
               workspace=workspace)
    if stream is None:
        stream = torch.cuda.current_stream(x_local.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(x_local.device):
        _check(lib().tsp_attn_layer_fwd(x_local.data_ptr(), w_qkv.data_ptr(), w_o.data_ptr(), k_gathered.data_ptr(),
                                        v_gathered.data_ptr(), y.data_ptr(), workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(),
                                        B, S_total, D, rank, Hq, Hkv, dh, d_model, shards_per_group, handle))
    return y


def fwd_raw(q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, B, S_total, D, rank, Hq, Hkv, dh, dtype, stream) -> int:
    """Direct call of the C entry point with raw pointers; returns the status code."""
    return lib().tsp_attn_fwd(q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, B, S_total, D, rank, Hq, Hkv, dh, dtype,
                              stream)


def zigzag_positions(S_total: int, D: int, rank: int) -> torch.Tensor:
    """Host-side zigzag map of the library: global position of each local row (int64)."""
    if D < 1 or S_total % (2 * D) != 0:
        _check(lib().tsp_attn_zigzag_positions(S_total, D, rank, None))
    n = S_total // D
    out = torch.empty(n, dtype=torch.int64)
    _check(lib().tsp_attn_zigzag_positions(S_total, D, rank,
                                           ctypes.cast(out.data_ptr(), ctypes.POINTER(_I64))))
    return out


def zigzag_positions_device(S_total: int, D: int, rank: int, device="cuda") -> torch.Tensor:
    """The zigzag map as evaluated by the kernels' device code (int32, on ``device``)."""
    n = S_total // D if D >= 1 else 0
    out = torch.empty(max(n, 1), dtype=torch.int32, device=device)
    with torch.cuda.device(out.device):
        st = lib().tsp_attn_zigzag_positions_device(out.data_ptr(), S_total, D, rank,
                                                    torch.cuda.current_stream(out.device).cuda_stream)
    _check(st)
    return out[:n]


def unmasked_pairs(S_total: int, D: int, rank: int) -> int:
    r = lib().tsp_attn_unmasked_pairs(S_total, D, rank)
    if r < 0:
        _check(int(r))
    return int(r)


def schedule(B, S_total, D, rank, Hq, Hkv, dh, dtype=TSP_BF16):
    """(n_workgroups, kv tiles per workgroup [int64 tensor], kv tile length) of a launch."""
    n = _I64(0)
    _check(lib().tsp_attn_schedule(B, S_total, D, rank, Hq, Hkv, dh, dtype, ctypes.byref(n), None, None))
    tiles = torch.empty(n.value, dtype=torch.int64)
    bk = _I64(0)
    _check(lib().tsp_attn_schedule(B, S_total, D, rank, Hq, Hkv, dh, dtype, ctypes.byref(n),
                                   ctypes.cast(tiles.data_ptr(), ctypes.POINTER(_I64)), ctypes.byref(bk)))
    return n.value, tiles, bk.value
