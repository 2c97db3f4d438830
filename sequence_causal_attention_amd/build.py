"""Build the HIP library in-tree: ``python -m sequence_causal_attention_amd.build``.

Compiles the translation units under csrc/ for gfx950 and links them into
``libtsp_attn.so`` next to this file. Packed fp32 VALU instructions are disabled for all
device code.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtsp_attn.so")
# (source, flags of that translation unit only)
UNITS = [
    # forward kernels: MFMA results in arch VGPRs, the score tiles feed the VALU softmax;
    # no NaN reaches the row maxima (only finite scores and -inf masks), so the maxima
    # need no NaN-quieting instructions; the scheduler groups LDS reads into clauses
    # (+0.7% on the 7B shard in A/B runs)
    (os.path.join(CSRC, "tsp_attn.hip"), ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-fno-honor-nans",
                                          "-mllvm", "-amdgpu-sched-strategy=max-memory-clause"]),
    # backward kernels, dh 64 / 128: MFMA results in arch VGPRs; LLVM's max-ilp scheduling
    # strategy (+1.9-2.5% on the 7B shard backward in A/B runs) with its own register
    # pressure trackers (+1.1-1.8% more); same results bit for bit
    (os.path.join(CSRC, "tsp_attn_bwd.hip"), ["-mllvm", "-amdgpu-mfma-vgpr-form=1",
                                              "-mllvm", "-amdgpu-sched-strategy=max-ilp",
                                              "-mllvm", "-amdgpu-use-amdgpu-trackers"]),
    # backward kernels, dh 256: the dK/dV accumulators fill the arch VGPRs, so MFMA
    # results stay in the accumulation registers; max-ilp scheduling (+9.5% on the GQA
    # dh-256 shard backward in an A/B run, same results bit for bit)
    (os.path.join(CSRC, "tsp_attn_bwd256.hip"), ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]),
    # projection GEMM and the attention layer: MFMA accumulators in the accumulation registers
    (os.path.join(CSRC, "tsp_layer.hip"), []),
]
SOURCES = [u[0] for u in UNITS]
HEADERS = [os.path.join(ROOT, "include", "tsp_attn.h")] + [
    os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith(".h")
]
COMMON = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def commands(out: str, objdir: str, extra=()) -> list:
    """The compile command of every unit, then the link command."""
    cmds, objs = [], []
    for src, flags in UNITS:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmds.append([hipcc(), *COMMON, *flags, "-I", os.path.join(ROOT, "include"), "-I", CSRC, *extra,
                     "-c", "-o", obj, src])
    cmds.append([hipcc(), "--offload-arch=gfx950", "-fPIC", "-shared", "-o", out, *objs])
    return cmds


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)


def build(verbose: bool = True, extra=()) -> str:
    tmp = LIB + ".tmp"
    with tempfile.TemporaryDirectory(prefix="tsp_attn_build_") as objdir:
        for cmd in commands(tmp, objdir, extra):
            _run(cmd, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=tuple(sys.argv[1:]))
