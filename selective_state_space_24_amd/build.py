"""Builds the in-tree HIP library ``lib/libssm_scan.so`` for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libssm_scan.so")

# Kernel instantiations are split by io dtype and A mode so that the units compile in parallel.
SOURCES = ["scan_fwd_bf16_diag.hip", "scan_fwd_bf16_head.hip", "scan_fwd_f32_diag.hip",
           "scan_fwd_f32_head.hip", "scan_state.hip", "scan_decode.hip",
           "scan_bwd.hip", "scan_bwd_wide_bf16.hip", "scan_bwd_wide_f32.hip", "scan_ssd.hip",
           "scan_noalloc.hip", "scan_complex.hip", "scan_api.cpp"]

# Packed fp32 instructions are switched off for all device code.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wall", "-Wno-unused-command-line-argument"]


# Per-source additions. The chunked kernel scales its MFMA accumulators elementwise every chunk;
# kept in accumulation registers (AGPRs) each such operation needs a copy out and back, so its
# accumulators are placed in ordinary VGPRs (they fit: one wavefront per SIMD).
EXTRA_FLAGS = {"scan_ssd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _filtered(out: str) -> str:
    # the host pass does not know the packed-fp32 feature and says so; drop that line only
    return "\n".join(ln for ln in out.splitlines()
                     if "not a recognized feature for this target" not in ln)


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = False, jobs: int = 0, only=None) -> str:
    """Compiles every source to an object in parallel, then links the shared library.

    ``only``: names of the sources to recompile; the objects of the others are reused (they
    must exist from an earlier full build)."""
    os.makedirs(LIBDIR, exist_ok=True)
    objdir = os.path.join(LIBDIR, "obj")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    jobs = jobs or max(1, min(len(SOURCES), os.cpu_count() or 1))
    pending = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        objs.append(obj)
        if only is not None and src not in only:
            if not os.path.exists(obj):
                raise RuntimeError(f"{obj} is missing: run a full build first")
            continue
        cmd = ([hipcc()] + HIPCC_FLAGS + EXTRA_FLAGS.get(src, []) + inc
               + ["-c", os.path.join(CSRC, src), "-o", obj])
        if verbose:
            print(" ".join(cmd), flush=True)
        pending.append((src, cmd))
    failed = []
    running = []
    while pending or running:
        while pending and len(running) < jobs:
            src, cmd = pending.pop(0)
            running.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                  stderr=subprocess.STDOUT, text=True)))
        src, proc = running.pop(0)
        out, _ = proc.communicate()
        msg = _filtered(out)
        if msg:
            print(msg, file=sys.stderr)
        if proc.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed on {', '.join(failed)}")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msg = _filtered(res.stdout + res.stderr)
    if msg:
        print(msg, file=sys.stderr)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc link failed with status {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, only=sys.argv[1:] or None))
