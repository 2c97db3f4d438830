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
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtsp_attn.so")
# (source, flags of that translation unit only)
UNITS = [
    # bf16 forward kernels: MFMA results in arch VGPRs, the score tiles feed the VALU
    # softmax; no NaN reaches the row maxima (only finite scores and -inf masks), so the
    # maxima need no NaN-quieting instructions; the scheduler groups LDS reads into
    # clauses (+0.7% on the 7B shard in A/B runs)
    (os.path.join(CSRC, "tsp_attn_fwd_bf16.hip"), ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-fno-honor-nans",
                                                   "-mllvm", "-amdgpu-sched-strategy=max-memory-clause"]),
    # the C ABI of the forward, the fp32 forward, the merge, the Ulysses layout changes and
    # the map helpers: default code generation (IEEE NaN semantics)
    (os.path.join(CSRC, "tsp_attn.hip"), []),
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


# Host-code sanitizers (AddressSanitizer and UndefinedBehaviorSanitizer) for a CPU-only
# check of the library's host side: argument checks, range clipping and folding, the tile
# plan, workspace sizing. Each flag applies to the host pass only; device code is built as
# usual. The result is a separate library that a process loads with the sanitizer runtime
# preloaded (see run_host_sanitized below); it is never the library the package loads.
HOSTSAN_LIB = os.path.join(ROOT, "_build", "libtsp_attn_hostsan.so")
HOSTSAN_FLAGS = "-Xarch_host -fsanitize=address,undefined -Xarch_host -fno-sanitize-recover=undefined".split()
HOSTSAN_FLAGS += "-Xarch_host -fno-omit-frame-pointer -Xarch_host -g".split()
HOSTSAN_LINK = "-Xarch_host -fsanitize=address,undefined -Xarch_host -shared-libasan".split()


def commands(out: str, objdir: str, extra=(), link_extra=()) -> list:
    """The compile command of every unit, then the link command."""
    cmds, objs = [], []
    for src, flags in UNITS:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmds.append([hipcc(), *COMMON, *flags, "-I", os.path.join(ROOT, "include"), "-I", CSRC, *extra,
                     "-c", "-o", obj, src])
    cmds.append([hipcc(), "--offload-arch=gfx950", "-fPIC", "-shared", *link_extra, "-o", out, *objs])
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


def build(verbose: bool = True, extra=(), host_sanitize: bool = False) -> str:
    """Compiles the units side by side (one hipcc process each), then links."""
    lib = HOSTSAN_LIB if host_sanitize else LIB
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    tmp = lib + ".tmp"
    with tempfile.TemporaryDirectory(prefix="tsp_attn_build_") as objdir:
        cmds = commands(tmp, objdir, tuple(extra) + (tuple(HOSTSAN_FLAGS) if host_sanitize else ()),
                        HOSTSAN_LINK if host_sanitize else ())
        with ThreadPoolExecutor(max_workers=min(len(cmds) - 1, os.cpu_count() or 1)) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds[:-1]))
        _run(cmds[-1], verbose)
    os.replace(tmp, lib)
    return lib


def sanitizer_runtime() -> str:
    """The clang AddressSanitizer runtime (shared) that ships with the ROCm compiler."""
    llvm = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "llvm")
    if not os.path.isdir(llvm):
        llvm = "/opt/rocm/llvm"
    base = os.path.join(llvm, "lib", "clang")
    for ver in sorted(os.listdir(base), reverse=True):
        cand = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(cand):
            return cand
    raise RuntimeError("no libclang_rt.asan-x86_64.so under " + base)


def run_host_sanitized(pytest_args) -> int:
    """Runs pytest (CPU tests) against the host-sanitized library in a child process with
    the sanitizer runtime preloaded. Returns its exit status."""
    env = dict(os.environ)
    env["LD_PRELOAD"] = sanitizer_runtime()
    env["TSP_ATTN_LIB"] = HOSTSAN_LIB
    # the interpreter's own allocations are not this library's: no leak report at exit
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return subprocess.run([sys.executable, "-m", "pytest", *pytest_args], env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    args = sys.argv[1:]
    if args[:1] == ["--host-sanitize"]:
        # build the host-sanitized library, then run the given pytest arguments against it
        build(verbose=False, extra=(), host_sanitize=True)
        sys.exit(run_host_sanitized(args[1:] or ["-q", "-m", "not gpu", "tests/test_abi.py"]))
    build(verbose=True, extra=tuple(args))
