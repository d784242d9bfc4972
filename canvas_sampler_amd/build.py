"""Builds the HIP library libdgcanvas.so for gfx950 with hipcc, in-tree, and
beside it libdgprobe.so, the plain streaming read that the measurements set
next to the statistics pass.

Every source is compiled on each call (the caller decides when to build).
Packed-FP32 instructions are disabled for all device code.
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdgcanvas.so")
SOURCES = ["dg_canvas.hip", "canvas_stats.hip", "accept_renoise.hip", "lmhead_gemm.hip",
           "self_cond.hip"]
PROBE_LIB = os.path.join(PKG, "libdgprobe.so")
PROBE_SOURCES = ["stream_read_probe.hip"]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: cannot build the canvas sampler library")


def flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build(verbose=False):
    """Compiles every source to an object in _build/ (in parallel), links the
    two shared libraries next to this file and returns the sampler's path."""
    obj_dir = os.path.join(ROOT, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    procs, objs = [], {}
    for src in SOURCES + PROBE_SOURCES:
        obj = os.path.join(obj_dir, src.replace(".hip", ".o"))
        cmd = [hipcc()] + flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs[src] = obj
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        if p.returncode != 0:
            failed.append(src + ":\n" + text)
        elif verbose and text.strip():
            print(text, flush=True)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(failed))
    for lib, srcs in ((LIB, SOURCES), (PROBE_LIB, PROBE_SOURCES)):
        tmp = lib + ".tmp"
        cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC"]
        subprocess.run(cmd + [objs[s] for s in srcs] + ["-o", tmp], check=True)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
