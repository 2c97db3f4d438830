"""The C-ABI library on the CPU: it loads, exports every declared symbol, its host-side
zigzag map and pair count agree bit-exactly with the oracle, its schedule is balanced,
and invalid arguments are rejected before anything is launched (no GPU needed: every
call here returns during host-side validation or is a pure host computation)."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
import sequence_causal_attention_amd as tsp
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tsp_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tsp_(?:attn|ulysses|gemm)_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(tsp.LIB_PATH):
        pytest.fail(f"{tsp.LIB_PATH} not built: run `python -m sequence_causal_attention_amd.build`")
    return tsp.lib()


def test_header_declares_the_binding_surface():
    assert declared_functions() == sorted(tsp.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", tsp.LIB_PATH], capture_output=True, text=True, check=True)
    exported = {ln.split()[-1] for ln in out.stdout.splitlines() if ln.strip()}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_library_links_no_torch():
    # the DT_NEEDED names (ldd would also print resolved paths, which may sit under
    # torch's own library folder when LD_LIBRARY_PATH points there)
    out = subprocess.run(["readelf", "-d", tsp.LIB_PATH], capture_output=True, text=True)
    assert out.returncode == 0, out.stderr
    deps = [ln.split("[")[1].split("]")[0] for ln in out.stdout.splitlines() if "(NEEDED)" in ln]
    assert "libamdhip64.so.7" in deps or any(d.startswith("libamdhip64") for d in deps), deps
    assert not [d for d in deps if "torch" in d or "c10" in d], deps


MAP_CASES = [(2, 1, 0), (8, 4, 3), (512, 4, 1), (1200, 3, 2), (32768, 8, 3), (262144, 8, 0), (262144, 8, 7),
             (131072, 1, 0), (65536, 4, 2)]


@pytest.mark.parametrize("S,D,r", MAP_CASES)
def test_host_map_matches_oracle_bit_exact(lib, S, D, r):
    got = tsp.zigzag_positions(S, D, r).numpy()
    assert got.dtype == np.int64
    assert np.array_equal(got, oracle.zigzag_positions(S, D, r))


@pytest.mark.parametrize("S,D,r", MAP_CASES)
def test_unmasked_pairs_matches_oracle(lib, S, D, r):
    assert tsp.unmasked_pairs(S, D, r) == oracle.unmasked_pairs(S, D, r)


@pytest.mark.parametrize("w", workloads.WORKLOADS[1:], ids=lambda w: w.name)
def test_schedule_is_balanced_across_workgroups_and_ranks(lib, w):
    """Mirrored query-tile pairs: every workgroup sweeps the same number of KV tiles, and
    every rank launches the same number of workgroups with the same total."""
    per_rank = []
    for r in range(w.D):
        n, tiles, bk = tsp.schedule(w.B, w.S_total, w.D, r, w.Hq, w.Hkv, w.dh)
        assert n == tiles.numel() > 0
        assert int(tiles.max()) - int(tiles.min()) <= 1, (r, tiles.min(), tiles.max())
        per_rank.append((n, int(tiles.sum()), int(tiles.max())))
    assert len(set(per_rank)) == 1, per_rank


def _fake(addr=0x100000):
    return ctypes.c_void_p(addr)


VALID = dict(B=1, S_total=512, D=4, rank=1, Hq=4, Hkv=1, dh=64, dtype=tsp.TSP_F32)


def _call(lib, ptrs=None, **kw):
    a = dict(VALID)
    a.update(kw)
    q, k, v, o, l = ptrs if ptrs is not None else (_fake(), _fake(), _fake(), _fake(), _fake())
    return lib.tsp_attn_fwd(q, k, v, o, l, a["B"], a["S_total"], a["D"], a["rank"], a["Hq"], a["Hkv"], a["dh"],
                            a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(D=0), tsp.TSP_EINVAL),
    (dict(rank=4), tsp.TSP_EINVAL),
    (dict(rank=-1), tsp.TSP_EINVAL),
    (dict(S_total=500), tsp.TSP_EINVAL),
    (dict(S_total=0), tsp.TSP_EINVAL),
    (dict(B=0), tsp.TSP_EINVAL),
    (dict(Hq=6, Hkv=4), tsp.TSP_EINVAL),
    (dict(Hkv=0), tsp.TSP_EINVAL),
    (dict(dh=96), tsp.TSP_EUNSUPPORTED),
    (dict(dh=32), tsp.TSP_EUNSUPPORTED),
    (dict(dtype=7), tsp.TSP_EUNSUPPORTED),
    # past the size limits: positions must stay int32, per-lane byte offsets 32-bit
    (dict(S_total=1 << 31), tsp.TSP_EINVAL),
    (dict(S_total=(1 << 30) + 8), tsp.TSP_EINVAL),
    (dict(Hq=1 << 17, Hkv=1 << 17, dh=64), tsp.TSP_EINVAL),
    (dict(B=1 << 17), tsp.TSP_EINVAL),
])
def test_invalid_arguments_rejected(lib, kw, code):
    assert _call(lib, **kw) == code
    assert lib.tsp_attn_last_error().decode() != ""


def test_null_and_misaligned_pointers_rejected(lib):
    for i in range(5):
        ptrs = [_fake(), _fake(), _fake(), _fake(), _fake()]
        ptrs[i] = None
        assert _call(lib, ptrs=ptrs) == tsp.TSP_EINVAL
        ptrs[i] = _fake(0x100008)
        assert _call(lib, ptrs=ptrs) == tsp.TSP_EINVAL


@pytest.mark.parametrize("lo,hi", [(10, 9), (-1, 5), (0, 513), (600, 700), (-5, -1)])
def test_range_outside_sequence_rejected(lib, lo, hi):
    a = VALID
    f = _fake()
    st = lib.tsp_attn_fwd_range(f, f, f, f, f, a["B"], a["S_total"], a["D"], a["rank"], a["Hq"], a["Hkv"], a["dh"],
                                lo, hi, 0, a["dtype"], None)
    assert st == tsp.TSP_EINVAL
    assert "range" in lib.tsp_attn_last_error().decode()


@pytest.mark.parametrize("r1,r2", [
    ((0, 128), (64, 256)),    # overlapping
    ((256, 384), (0, 128)),   # second before the first
    ((0, 128), (256, 600)),   # second past S_total
    ((0, 128), (300, 200)),   # second reversed
])
def test_second_range_must_follow_the_first(lib, r1, r2):
    f = _fake()
    a = VALID
    assert lib.tsp_attn_fwd_range2(f, f, f, f, f, a["B"], a["S_total"], a["D"], a["rank"], a["Hq"], a["Hkv"],
                                   a["dh"], *r1, *r2, 0, a["dtype"], None) == tsp.TSP_EINVAL
    assert "second key range" in lib.tsp_attn_last_error().decode()


def _ring(lib, ptrs=None, ready=None, status=None, spin=16, **kw):
    a = dict(VALID, dtype=tsp.TSP_BF16, S_total=4096, D=4, Hq=4, Hkv=2, dh=128)
    a.update(kw)
    q, k, v, o, l = ptrs if ptrs is not None else (_fake(),) * 5
    return lib.tsp_attn_fwd_ring(q, k, v, o, l, a["B"], a["S_total"], a["D"], a["rank"], a["Hq"], a["Hkv"], a["dh"],
                                 ready, 1, spin, status, a["dtype"], None)


def test_ring_validation(lib):
    """Rejected before anything is enqueued (no GPU needed)."""
    assert _ring(lib, dtype=tsp.TSP_F32) == tsp.TSP_EUNSUPPORTED          # bf16 only
    assert "bf16" in lib.tsp_attn_last_error().decode()
    assert _ring(lib, S_total=512) == tsp.TSP_EUNSUPPORTED                # C = 64: below the 128-row query tile (GQA 2:1)
    assert "multiple" in lib.tsp_attn_last_error().decode()
    assert _ring(lib, ready=_fake()) == tsp.TSP_EINVAL                    # flags without a status word
    assert _ring(lib, ready=_fake(), status=_fake(), spin=0) == tsp.TSP_EINVAL  # no poll allowed
    assert _ring(lib, rank=4) == tsp.TSP_EINVAL
    assert _ring(lib, dh=96) == tsp.TSP_EUNSUPPORTED
    for i in range(5):
        ptrs = [_fake()] * 5
        ptrs[i] = None
        assert _ring(lib, ptrs=ptrs) == tsp.TSP_EINVAL
        ptrs[i] = _fake(0x100008)
        assert _ring(lib, ptrs=ptrs) == tsp.TSP_EINVAL


def test_range_shares_fwd_validation(lib):
    f = _fake()
    assert lib.tsp_attn_fwd_range(f, f, f, f, None, 1, 512, 4, 1, 4, 1, 64, 0, 512, 0, tsp.TSP_F32, None) == \
        tsp.TSP_EINVAL
    assert lib.tsp_attn_fwd_range(f, f, f, f, f, 1, 512, 4, 1, 4, 1, 96, 0, 512, 0, tsp.TSP_F32, None) == \
        tsp.TSP_EUNSUPPORTED
    assert lib.tsp_attn_fwd_range(f, f, f, f, f, 1, 512, 4, 1, 4, 1, 64, 0, 512, 2, tsp.TSP_F32, None) == \
        tsp.TSP_EINVAL


MERGE_VALID = dict(B=1, S_local=128, Hq=4, dh=128, dtype=tsp.TSP_BF16)


def _merge_call(lib, ptrs=None, **kw):
    a = dict(MERGE_VALID)
    a.update(kw)
    p = ptrs if ptrs is not None else [_fake()] * 6
    return lib.tsp_attn_merge(*p, a["B"], a["S_local"], a["Hq"], a["dh"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), tsp.TSP_EINVAL),
    (dict(S_local=0), tsp.TSP_EINVAL),
    (dict(Hq=0), tsp.TSP_EINVAL),
    (dict(dh=96), tsp.TSP_EUNSUPPORTED),
    (dict(dtype=5), tsp.TSP_EUNSUPPORTED),
])
def test_merge_invalid_arguments_rejected(lib, kw, code):
    assert _merge_call(lib, **kw) == code
    assert lib.tsp_attn_last_error().decode() != ""


def test_merge_null_and_misaligned_pointers_rejected(lib):
    for i in range(6):
        ptrs = [_fake()] * 6
        ptrs[i] = None
        assert _merge_call(lib, ptrs=ptrs) == tsp.TSP_EINVAL
        ptrs[i] = _fake(0x100004)
        assert _merge_call(lib, ptrs=ptrs) == tsp.TSP_EINVAL


BWD_VALID = dict(B=1, S_total=512, D=4, rank=1, Hq=4, Hkv=1, dh=64, dtype=tsp.TSP_BF16)


def _bwd_call(lib, ptrs=None, **kw):
    a = dict(BWD_VALID)
    a.update(kw)
    p = ptrs if ptrs is not None else [_fake()] * 10
    return lib.tsp_attn_bwd(*p, a["B"], a["S_total"], a["D"], a["rank"], a["Hq"], a["Hkv"], a["dh"], a["dtype"],
                            None)


@pytest.mark.parametrize("kw,code", [
    (dict(D=0), tsp.TSP_EINVAL),
    (dict(rank=4), tsp.TSP_EINVAL),
    (dict(S_total=500), tsp.TSP_EINVAL),
    (dict(B=0), tsp.TSP_EINVAL),
    (dict(Hq=6, Hkv=4), tsp.TSP_EINVAL),
    (dict(Hq=65536, Hkv=1, dh=128), tsp.TSP_EINVAL),   # Hq * dh above 2^22
    (dict(dh=96), tsp.TSP_EUNSUPPORTED),
    (dict(dtype=9), tsp.TSP_EUNSUPPORTED),
])
def test_bwd_invalid_arguments_rejected(lib, kw, code):
    assert _bwd_call(lib, **kw) == code
    assert lib.tsp_attn_last_error().decode() != ""


def test_bwd_null_and_misaligned_pointers_rejected(lib):
    for i in range(10):
        ptrs = [_fake()] * 10
        ptrs[i] = None
        assert _bwd_call(lib, ptrs=ptrs) == tsp.TSP_EINVAL
        ptrs[i] = _fake(0x100008)
        assert _bwd_call(lib, ptrs=ptrs) == tsp.TSP_EINVAL


ULYSSES = ["tsp_ulysses_pack_heads", "tsp_ulysses_unpack_heads", "tsp_ulysses_gather_sequence",
           "tsp_ulysses_scatter_sequence"]


@pytest.mark.parametrize("fn", ULYSSES)
@pytest.mark.parametrize("args,code", [
    ((0, 16, 8, 128, 4, tsp.TSP_BF16), tsp.TSP_EINVAL),      # B = 0
    ((1, 0, 8, 128, 4, tsp.TSP_BF16), tsp.TSP_EINVAL),       # S_local = 0
    ((1, 16, 8, 128, 0, tsp.TSP_BF16), tsp.TSP_EINVAL),      # P = 0
    ((1, 16, 8, 4, 4, tsp.TSP_BF16), tsp.TSP_EUNSUPPORTED),  # 8-byte rows
    ((1, 16, 8, 128, 4, 7), tsp.TSP_EUNSUPPORTED),           # dtype
])
def test_ulysses_invalid_arguments_rejected(lib, fn, args, code):
    f = _fake()
    assert getattr(lib, fn)(f, f, *args, None) == code
    assert getattr(lib, fn)(None, f, 1, 16, 8, 128, 4, tsp.TSP_BF16, None) == tsp.TSP_EINVAL
    assert getattr(lib, fn)(f, _fake(0x100008), 1, 16, 8, 128, 4, tsp.TSP_BF16, None) == tsp.TSP_EINVAL


def test_ulysses_heads_must_divide(lib):
    f = _fake()
    assert lib.tsp_ulysses_pack_heads(f, f, 1, 16, 6, 128, 4, tsp.TSP_BF16, None) == tsp.TSP_EINVAL
    assert lib.tsp_ulysses_unpack_heads(f, f, 1, 16, 6, 128, 4, tsp.TSP_BF16, None) == tsp.TSP_EINVAL


@pytest.mark.parametrize("args", [
    (64, 64, 100, 128, 128, 64, 0),   # K not a multiple of 64
    (64, 62, 128, 128, 128, 64, 0),   # N not a multiple of 4
    (64, 64, 128, 64, 128, 64, 0),    # lda < K
    (0, 64, 128, 128, 128, 64, 0),    # M = 0
    (64, 64, 128, 128, 128, 64, 3),   # mode
])
def test_gemm_invalid_arguments_rejected(lib, args):
    f = _fake()
    assert lib.tsp_gemm_bf16_nt(f, f, f, *args, None) == tsp.TSP_EINVAL
    assert lib.tsp_attn_last_error().decode() != ""


def test_attn_layer_validation(lib):
    n = ctypes.c_int64(0)
    rows, hs = 1 * 2048 // 4, 8 // 4
    for G in (1, 2, 4, 0):
        assert lib.tsp_attn_layer_workspace_bytes(1, 2048, 4, 8, 4, 128, 512, G, ctypes.byref(n)) == tsp.TSP_OK
        g = 4 if G == 0 else G  # automatic: sized for any group
        assert n.value >= rows * g * hs * 128 * 2 * 2 + rows * g * hs * 4 + rows * 512 * 4
    assert lib.tsp_attn_layer_workspace_bytes(1, 2048, 4, 6, 2, 128, 512, 1, ctypes.byref(n)) == tsp.TSP_EINVAL
    assert lib.tsp_attn_layer_workspace_bytes(1, 2048, 4, 8, 4, 128, 500, 1, ctypes.byref(n)) == tsp.TSP_EINVAL
    assert lib.tsp_attn_layer_workspace_bytes(1, 2048, 4, 8, 4, 128, 512, 3, ctypes.byref(n)) == tsp.TSP_EINVAL
    assert lib.tsp_attn_layer_workspace_bytes(1, 2048, 4, 8, 4, 128, 512, -1, ctypes.byref(n)) == tsp.TSP_EINVAL
    f = _fake()
    assert lib.tsp_attn_layer_fwd(f, f, f, f, f, f, f, 16, 1, 2048, 4, 1, 8, 4, 128, 512, 1, None) == tsp.TSP_EINVAL
    assert "workspace" in lib.tsp_attn_last_error().decode()
    assert lib.tsp_attn_layer_fwd(f, f, f, f, f, f, f, 1 << 30, 1, 2048, 4, 1, 8, 4, 128, 512, 3, None) == tsp.TSP_EINVAL
    assert "shards_per_group" in lib.tsp_attn_last_error().decode()


def test_map_helpers_reject_bad_sizes(lib):
    assert lib.tsp_attn_unmasked_pairs(500, 4, 0) == tsp.TSP_EINVAL
    assert lib.tsp_attn_zigzag_positions(512, 4, 9, None) == tsp.TSP_EINVAL
    assert lib.tsp_attn_zigzag_positions(512, 4, 0, None) == tsp.TSP_EINVAL  # null output
    assert lib.tsp_attn_zigzag_positions_device(None, 512, 0, 0, None) == tsp.TSP_EINVAL
    with pytest.raises(tsp.TspAttnError):
        tsp.zigzag_positions(500, 4, 0)


def test_strerror(lib):
    for code in (0, -1, -2, -3, -4):
        assert lib.tsp_attn_strerror(code)
    assert lib.tsp_attn_strerror(-99) == b"unknown status"
