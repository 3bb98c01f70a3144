"""Builds libspecverify.so (all HIP sources + the C ABI) for gfx950 with hipcc.

Kept beside the package it builds; ``__graft_entry__.build()`` calls it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libspecverify.so")
SOURCES = ["capi.cpp", "attn.hip", "sample.hip", "kvcache.hip", "check.hip", "probe.hip"]
ARCH = "gfx950"

# -packed-fp32-ops off: hipcc emits no packed fp32 add/mul/fma (v_pk_*_f32).
# amdgpu-mfma-vgpr-form: matrix-core accumulators live in ordinary VGPRs, so
# the attention loop's rare rescale branch does not force a copy of every
# accumulator between the AGPR and VGPR files on each iteration.
COMPILE_FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
                 "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                 "-mllvm", "-amdgpu-mfma-vgpr-form=1",
                 "-Wall", "-Wno-unused-result"]


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compiles each source to an object in parallel, links the shared library,
    and returns its path.  Always rebuilds."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") or src.endswith(".cpp") else []
        cmd = ["hipcc", *COMPILE_FLAGS, "-c", *lang, os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _drain(procs, verbose)
    _drain(procs, verbose)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["hipcc", "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def _drain(procs, verbose):
    while procs:
        src, pr = procs.pop(0)
        out, _ = pr.communicate()
        text = out.decode(errors="replace")
        # the host pass of hipcc warns that it does not know the device-only feature
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
        if pr.returncode != 0:
            sys.stderr.write("\n".join(lines) + "\n")
            raise RuntimeError("hipcc failed on " + src)
        if verbose and lines:
            print("\n".join(lines), flush=True)


if __name__ == "__main__":
    print(build(verbose=True))
