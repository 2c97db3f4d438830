"""Benchmark: causal attention forward of one sequence-parallel rank on one MI355X.

One step = one call of the whole hot path (zigzag map, K/V tile staging, QK^T, causal
masking and tile skipping, online softmax, PV, epilogue: one kernel launch) over the
7B-dense TSP shard: B=1, S_total=32768, D=8, rank 3 (chunks 3 and 12, 4096 local
queries), Hq=Hkv=32, dh=128, bf16, synthetic N(0,1) inputs already resident in HBM.

Prints ONE JSON line. `value` is causal TFLOP/s = 4*B*Hq*dh*C*(S_total+1) / time per
step (visible (q,k) pairs only; softmax not counted). The roofline entry compares the
kernel's algorithmic FLOP rate, timed with HIP events on its own stream, with the
MI355X dense bf16 MFMA peak. The cpu_baseline entry times the fp64 CPU oracle on a
bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CUs x 4096 dense bf16 FLOP/clk/CU x 2.4 GHz (AMD's 2.5 PFLOP/s)
PEAK_F32_MFMA_TFLOPS = 157.3
METRIC = "causal attention TFLOP/s per rank shard + % of bf16 MFMA peak (1 GPU)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


# the sources of the forward kernel and of its launch configuration; its compile flags are
# taken from the build script's entry for that unit
FORWARD_SOURCES = ("csrc/attn_common.h", "csrc/attn_fwd_bf16.h", "csrc/zigzag.h", "csrc/host_common.h",
                   "csrc/tsp_attn_fwd_bf16.hip", "csrc/tsp_attn.hip")
FORWARD_UNIT = "tsp_attn_fwd_bf16.hip"
# the same for the backward kernels of dh <= 128 (the bench workload's backward)
BACKWARD_SOURCES = ("csrc/attn_common.h", "csrc/attn_fwd_bf16.h", "csrc/attn_bwd_bf16.h", "csrc/bwd_config.h",
                    "csrc/zigzag.h", "csrc/host_common.h", "csrc/tsp_attn_bwd.hip")
BACKWARD_UNIT = "tsp_attn_bwd.hip"


def kernel_source_digest(backward: bool = False) -> str:
    """A short hash of the kernel sources and the compile flags of their unit, which ties
    a profile summary to the code it was taken on (the forward's, or the backward's)."""
    from sequence_causal_attention_amd import build as b

    pkg = os.path.join(ROOT, "sequence_causal_attention_amd")
    h = hashlib.sha256()
    for name in BACKWARD_SOURCES if backward else FORWARD_SOURCES:
        with open(os.path.join(pkg, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    unit = BACKWARD_UNIT if backward else FORWARD_UNIT
    flags = [fl for src, fl in b.UNITS if os.path.basename(src) == unit]
    h.update(repr((b.COMMON, flags)).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload_name: str, flops_per_launch: float):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they were taken
    on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload_name)
    if not entry or entry.get("source_digest") != kernel_source_digest():
        return None
    return entry.get("hbm_bytes_per_launch")


def cpu_baseline(w, rank, q, k, v, budget_s: float):
    """The fp64 oracle on a bounded sample: leading rows of each chunk, a few heads."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: fall back to the affinity mask
        threads = len(os.sched_getaffinity(0))
    pos = oracle.zigzag_positions(w.S_total, w.D, rank)
    heads, n_rows = [0, 1], 128
    rows = np.concatenate([np.arange(0, n_rows), np.arange(w.C, w.C + n_rows)])
    pairs = int(np.sum(pos[rows] + 1))
    t0 = time.perf_counter()
    done = 0
    while True:
        oracle.causal_attention(q, k, v, w.D, rank, rows=rows, heads=heads, block=128)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = (time.perf_counter() - t0) / done
    flops = 4.0 * w.B * len(heads) * w.dh * pairs
    host = ""
    try:
        with open("/proc/cpuinfo") as f:
            host = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {
        "value": round(flops / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(min(threads, len(os.sched_getaffinity(0)))),
        "host": host,
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle, rank {rank} rows [0,{n_rows}) and [{w.C},{w.C + n_rows}) "
                   f"(both chunks), query heads {heads}, all visible keys; {done} pass(es), "
                   f"{dt:.2f} s each; same algorithmic FLOP count convention"),
    }


def step_stats(torch, stream, step, n=20):
    """Per-step times (HIP events on the launch stream) of n further steps, after the
    timed region: median and min in microseconds."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    us = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
    return {"median": round(us[n // 2], 1), "min": round(us[0], 1), "n": n}


def settle_clocks(torch, stream, step, settle_ms: float):
    """Untimed launches after the warm-up steps until the GPU has run the step for at least
    `settle_ms` of its own time since the first of them. From an idle GPU the clocks ramp
    over the first few tens of milliseconds of load (the 7B-shard forward falls from ~1.2 ms
    to ~0.94 ms per launch over its first ~40 launches), so a few warm-up steps alone would
    time the ramp instead of the kernel. Returns what was run, for the JSON line."""
    if settle_ms <= 0:
        return {"launches": 0, "ms": 0.0}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    step()
    e1.record(stream)
    torch.cuda.synchronize()
    one = max(e0.elapsed_time(e1), 1e-3)
    n = max(0, int(settle_ms / one))
    e0.record(stream)
    for _ in range(n):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    return {"launches": n + 1, "ms": round(one + e0.elapsed_time(e1), 1),
            "why": "untimed, after the warm-up steps: the GPU clocks ramp over the first tens of ms of load"}


def balance_bench(args, torch, tsp, workloads):
    """Forward time of several ranks of one workload, each timed like the main benchmark:
    the zigzag split should give every rank the same time."""
    w = workloads.BY_NAME[args.workload]
    ranks = list(range(w.D)) if args.balance == "all" else [int(x) for x in args.balance.split(",")]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(dev)
    flops = 4.0 * w.B * w.Hq * w.dh * w.C * (w.S_total + 1)
    per = {}
    for r in ranks:
        q, k, v = workloads.make_inputs(w, r)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        out = torch.empty_like(qd)
        lse = torch.empty((w.B, w.Hq, w.S_local), dtype=torch.float32, device=dev)

        def step():
            tsp.fwd(qd, kd, vd, D=w.D, rank=r, out=out, lse=lse, stream=stream)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(args.steps):
            step()
        ev1.record(stream)
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / args.steps
        per[str(r)] = {"ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1),
                       "launch_us": step_stats(torch, stream, step, n=min(20, max(5, args.steps)))}
        del qd, kd, vd, out, lse
        torch.cuda.empty_cache()
    times = [e["ms"] for e in per.values()]
    line = {
        "metric": "per-rank forward time, max / min over the ranks timed (1 GPU)",
        "value": round(max(times) / min(times), 4), "unit": "ratio", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "S_total": w.S_total, "D": w.D, "Hq": w.Hq, "Hkv": w.Hkv,
                   "dh": w.dh, "flops_per_rank": flops, "ranks": per},
    }
    print(json.dumps(line), flush=True)


def layer_bench(args, torch, tsp, workloads):
    """One rank's TSP attention layer forward on the workload's shard (weights synthetic)."""
    w = workloads.BY_NAME[args.workload]
    rank = w.ranks[0] if args.rank is None else args.rank
    dm = args.layer
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = (workloads.make_grad((w.B, w.S_local, dm), 11, torch.float32) / dm ** 0.5).to(torch.bfloat16).to(dev)
    w_qkv = workloads.make_grad(((w.Hq + 2 * w.Hkv) * w.dh, dm), 12, torch.bfloat16).to(dev)
    w_o = (workloads.make_grad((dm, w.Hq * w.dh), 13, torch.float32) / (w.Hq * w.dh) ** 0.5).to(torch.bfloat16).to(dev)
    _, k, v = workloads.make_inputs(w, rank)
    kd, vd = k.to(dev), v.to(dev)
    y = torch.empty_like(x)
    G = args.layer_group
    ws = torch.empty(tsp.attn_layer_workspace_bytes(w.B, w.S_total, w.D, w.Hq, w.Hkv, w.dh, dm, G), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.Stream(dev)
    torch.cuda.synchronize()

    def step():
        tsp.attn_layer_fwd(x, w_qkv, w_o, kd, vd, D=w.D, rank=rank, Hq=w.Hq, Hkv=w.Hkv, dh=w.dh, shards_per_group=G,
                           y=y, workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    kernel_ms = ev0.elapsed_time(ev1) / args.steps
    rows = w.B * w.S_local
    proj = 2.0 * rows * dm * (w.Hq + 2 * w.Hkv) * w.dh + 2.0 * rows * w.Hq * w.dh * dm
    attn = 4.0 * w.B * w.Hq * w.dh * w.C * (w.S_total + 1)
    flops = proj + attn
    line = {
        "metric": "TSP attention layer TFLOP/s per rank (1 GPU)", "value": round(flops / ms / 1e9, 3),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "rank": rank, "d_model": dm, "Hq": w.Hq, "Hkv": w.Hkv, "dh": w.dh,
                   "D": w.D, "shards_per_group": G or "auto", "projection_flops": proj, "attention_flops": attn,
                   "form": f"{w.D} weight shards x (Q, K, V projections, attention, output projection)"},
        "roofline": {"bound": "mfma", "achieved": round(flops / kernel_ms / 1e9, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(flops / kernel_ms / 1e9 / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "kernel_ms": round(kernel_ms, 4)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def ulysses_bench(args, torch, tsp, workloads):
    """The local permutes of Ulysses sequence parallelism for one of P ranks (HBM-bound)."""
    name = args.workload if args.workload != "tsp_7b_shard_s32k" else "ulysses_head_subset_s128k"
    w = workloads.BY_NAME[name]
    P = args.ulysses
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    S_local = w.S_total // P
    shapes = {"q": (w.B, S_local, w.Hq * P, w.dh), "k": (w.B, S_local, w.Hkv * P, w.dh),
              "v": (w.B, S_local, w.Hkv * P, w.dh)}
    xs = {n: workloads.make_grad(s, 7 + i, torch.bfloat16).to(dev) for i, (n, s) in enumerate(shapes.items())}
    sends = {n: torch.empty((P, w.B, S_local, s[2] // P, w.dh), dtype=torch.bfloat16, device=dev)
             for n, s in shapes.items()}
    fulls = {n: torch.empty((w.B, w.S_total, s[2] // P, w.dh), dtype=torch.bfloat16, device=dev)
             for n, s in shapes.items()}
    o_send = torch.empty_like(sends["q"])
    o_back = torch.empty_like(xs["q"])
    stream = torch.cuda.Stream(dev)
    torch.cuda.synchronize()

    def step():
        for n in ("q", "k", "v"):
            tsp.ulysses_pack_heads(xs[n], P, out=sends[n], stream=stream)
            tsp.ulysses_gather_sequence(sends[n], out=fulls[n], stream=stream)  # (exchange elided)
        tsp.ulysses_scatter_sequence(fulls["q"], P, out=o_send, stream=stream)  # attention output stand-in
        tsp.ulysses_unpack_heads(o_send, out=o_back, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = ev0.elapsed_time(ev1) / args.steps
    moved = 2 * sum(2 * t.numel() * 2 for t in xs.values()) + 2 * 2 * o_back.numel() * 2  # read + write
    ms = wall * 1e3 / args.steps
    line = {
        "metric": "Ulysses layout-change bandwidth per rank (1 GPU)", "value": round(moved / (ms * 1e-3) / 1e9, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "P": P, "S_local": S_local, "heads_before": shapes["q"][2],
                   "heads_after": w.Hq, "dh": w.dh, "bytes_per_step": moved,
                   "form": "pack + gather of q, k, v; scatter + unpack of the output (8 launches)"},
        "roofline": {"bound": "hbm", "achieved": round(moved / (kernel_ms * 1e-3) / 1e9, 1), "peak": 8000.0,
                     "unit": "GB/s", "frac": round(moved / (kernel_ms * 1e-3) / 1e9 / 8000.0, 4), "traffic": None,
                     "kernel_ms": round(kernel_ms, 4)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="tsp_7b_shard_s32k")
    ap.add_argument("--rank", type=int, default=None)
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle timing")
    ap.add_argument("--settle-ms", type=float, default=250.0,
                    help="after the warm-up steps, untimed launches until this much GPU time has passed "
                         "(the clock ramp from idle); 0 disables")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--chunk-pipeline", nargs="?", const="fused", choices=["fused", "merge", "pairs", "ring"],
                    default=None,
                    help="time the chunk-pipelined form instead: one key-range launch per gathered "
                         "chunk (2D of them, in ring arrival order), folded into the running result "
                         "in the kernel's epilogue (fused, the default) or by a separate merge launch; "
                         "pairs: one two-range launch per ring step (D of them, a peer's two chunks "
                         "each), folded in the epilogue")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward instead (tsp_attn_bwd: delta, dQ and dK/dV kernels) on the "
                         "forward's out / lse; FLOPs counted as 5 products of 2*dh per visible pair")
    ap.add_argument("--ulysses", type=int, default=0, metavar="P",
                    help="time the Ulysses layout changes of one of P ranks instead: head pack and "
                         "sequence gather of q, k, v before the attention, sequence scatter and head "
                         "unpack of its output after (the workload is the attention shape after the "
                         "exchange); reports GB/s moved")
    ap.add_argument("--layer", type=int, default=0, metavar="D_MODEL",
                    help="time one rank's TSP attention layer instead (projections with every weight "
                         "shard, zigzag attention, output projection) at this model width; FLOPs of the "
                         "projections plus the causal attention")
    ap.add_argument("--layer-group", type=int, default=0, metavar="G",
                    help="with --layer: weight shards per projection / attention launch (0 = automatic)")
    ap.add_argument("--balance", default=None, metavar="RANKS",
                    help="time the forward of several ranks of the workload instead (comma list, or "
                         "'all'); reports each rank's time and the max / min ratio")
    ap.add_argument("--inputs", default="normal", choices=["normal", "zero-q", "zeros"],
                    help="diagnostic: run the same launches on zero queries (zero-q) or on all-zero "
                         "inputs (zeros) to show how the speed depends on the operand values; the "
                         "line is then not the metric's workload (its data field says so)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run plain device copies of MIB MiB (the known-size "
                         "kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the per-rank attention runs on a single MI355X and "
              "there is no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import sequence_causal_attention_amd as tsp
    import workloads

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.randn(n, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n * 4, "copies": max(1, args.steps)}), flush=True)
        return

    if args.balance:
        return balance_bench(args, torch, tsp, workloads)
    if args.ulysses:
        return ulysses_bench(args, torch, tsp, workloads)
    if args.layer:
        return layer_bench(args, torch, tsp, workloads)

    w = workloads.BY_NAME[args.workload]
    rank = w.ranks[0] if args.rank is None else args.rank
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    q, k, v = workloads.make_inputs(w, rank)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    if args.inputs != "normal":  # diagnostic only: same launches, other operand values
        qd.zero_()
        if args.inputs == "zeros":
            kd.zero_()
            vd.zero_()
    out = torch.empty_like(qd)
    lse = torch.empty((w.B, w.Hq, w.S_local), dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream(dev)  # default priority
    torch.cuda.synchronize()

    # ring arrival order of the gathered chunks: the rank's own pair first, then the pair
    # (p, 2D-1-p) of peer p = rank-1, rank-2, ... (mod D)
    pairs = [((p * w.C, (p + 1) * w.C), ((2 * w.D - 1 - p) * w.C, (2 * w.D - p) * w.C))
             for p in ((rank - s) % w.D for s in range(w.D))]
    bounds = [rng for pair in pairs for rng in pair]
    part_o, part_l = torch.empty_like(out), torch.empty_like(lse)
    # ring form: every chunk's arrival flag already set (the gathered K/V is resident), so the
    # kernel's waits pass at the first poll
    ring_ready = torch.ones(2 * w.D, dtype=torch.int32, device=dev)
    ring_status = torch.zeros(1, dtype=torch.int32, device=dev)

    if args.backward:
        tsp.fwd(qd, kd, vd, D=w.D, rank=rank, out=out, lse=lse, stream=stream)
        dout = workloads.make_grad(qd.shape, 99, qd.dtype).to(dev)
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        delta = torch.empty_like(lse)
        torch.cuda.synchronize()

    def step():
        if args.backward:
            tsp.bwd(qd, kd, vd, out, lse, dout, D=w.D, rank=rank, dq=dq, dk=dk, dv=dv, delta=delta, stream=stream)
            return
        if not args.chunk_pipeline:
            tsp.fwd(qd, kd, vd, D=w.D, rank=rank, out=out, lse=lse, stream=stream)
            return
        if args.chunk_pipeline == "ring":
            tsp.fwd_ring(qd, kd, vd, D=w.D, rank=rank, out=out, lse=lse, chunk_ready=ring_ready, ready_value=1,
                         spin_limit=1 << 20, wait_status=ring_status, stream=stream)
            return
        if args.chunk_pipeline == "pairs":
            tsp.fwd(qd, kd, vd, D=w.D, rank=rank, out=out, lse=lse, stream=stream, kv_range=pairs[0][0],
                    kv_range2=pairs[0][1])
            for ra, rb in pairs[1:]:
                tsp.fwd(qd, kd, vd, D=w.D, rank=rank, out=out, lse=lse, stream=stream, kv_range=ra,
                        kv_range2=rb, accumulate=True)
            return
        tsp.fwd(qd, kd, vd, D=w.D, rank=rank, out=out, lse=lse, stream=stream, kv_range=bounds[0])
        for rng in bounds[1:]:
            if args.chunk_pipeline == "fused":
                tsp.fwd(qd, kd, vd, D=w.D, rank=rank, out=out, lse=lse, stream=stream, kv_range=rng,
                        accumulate=True)
            else:
                tsp.fwd(qd, kd, vd, D=w.D, rank=rank, out=part_o, lse=part_l, stream=stream, kv_range=rng)
                tsp.merge(out, lse, part_o, part_l, out=out, lse=lse, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    settle = settle_clocks(torch, stream, step, args.settle_ms)

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = ev0.elapsed_time(ev1) / args.steps
    launch = step_stats(torch, stream, step)
    if args.chunk_pipeline == "ring" and int(ring_status.item()) != 0:
        raise RuntimeError("a ring wait gave up although every chunk was flagged present")

    # causal FLOPs: 2 products (forward) or 5 (backward) of 2*dh per visible pair per query head
    flops = (10.0 if args.backward else 4.0) * w.B * w.Hq * w.dh * w.C * (w.S_total + 1)
    ms_per_step = wall * 1e3 / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_MFMA_TFLOPS

    cpu = None
    if not args.no_cpu_baseline and not args.chunk_pipeline and not args.backward and args.inputs == "normal":
        cpu = cpu_baseline(w, rank, q, k, v, args.cpu_budget)

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "pct_of_peak": round(100.0 * value / peak, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic" if args.inputs == "normal" else
                f"diagnostic: {args.inputs} inputs instead of N(0,1), not the metric's workload",
        "config": {
            "workload": w.name, "B": w.B, "S_total": w.S_total, "D": w.D, "rank": rank, "Hq": w.Hq,
            "Hkv": w.Hkv, "dh": w.dh, "local_queries": w.S_local, "flops_per_step": flops,
            "parallelism": "one sequence-parallel rank's shard on 1 GPU",
            "form": ("backward: delta, dQ and dK/dV launches" if args.backward else
                     "single launch" if not args.chunk_pipeline else
                     f"chunk pipeline: {len(bounds)} key-range launches, merged in the epilogue"
                     if args.chunk_pipeline == "fused" else
                     f"chunk pipeline: {len(pairs)} two-range launches (a peer's two chunks each), merged "
                     "in the epilogue" if args.chunk_pipeline == "pairs" else
                     "chunk pipeline, ring order: the own chunks in one launch, every peer's chunks in a second "
                     "(arrival flags polled per chunk), merged in its epilogue" if args.chunk_pipeline == "ring" else
                     f"chunk pipeline: {len(bounds)} key-range launches + {len(bounds) - 1} merge launches"),
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": None if (args.chunk_pipeline or args.backward) else measured_traffic(w.name, flops),
            "kernel_ms": round(kernel_ms, 4),
        },
        "step_us": launch,
        "settle": settle,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
