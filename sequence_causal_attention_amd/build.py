"""Build the HIP library in-tree: ``python -m sequence_causal_attention_amd.build``.

Compiles csrc/tsp_attn.hip for gfx950 into ``libtsp_attn.so`` next to this file.
Packed fp32 VALU instructions are disabled for all device code.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtsp_attn.so")
SOURCES = [os.path.join(CSRC, "tsp_attn.hip")]
HEADERS = [os.path.join(ROOT, "include", "tsp_attn.h")] + [
    os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith(".h")
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def command(out: str = LIB, extra=()) -> list:
    return [
        hipcc(),
        "--offload-arch=gfx950",
        "-O3",
        "-std=c++20",
        "-fPIC",
        "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA results in arch VGPRs: the score tiles feed VALU softmax directly
        "-mllvm", "-amdgpu-mfma-vgpr-form=1",
        "-I", os.path.join(ROOT, "include"),
        "-I", CSRC,
        *extra,
        "-o", out,
        *SOURCES,
    ]


def build(verbose: bool = True, extra=()) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=tuple(sys.argv[1:]))
