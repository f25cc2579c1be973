"""Build the gfx950 libraries in-tree with hipcc.

* contextual_activation_sparsity_amd/libdejavu_hip.so : the sparse layer step (C ABI in
  include/dejavu_hip.h)
* synth/libdv_synth.so : the device filler of the seeded synthetic inputs, and the plain
                         streaming-read kernel the bench reports as its read reference

Every HIP source is compiled for gfx950 only, with packed-fp32 instructions disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdejavu_hip.so")
SYNTH_SRC = os.path.join(ROOT, "synth", "fill.hip")
SYNTH_STREAM_SRC = os.path.join(ROOT, "synth", "stream.hip")
SYNTH_LIB = os.path.join(ROOT, "synth", "libdv_synth.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
SOURCES = ["dv_api.hip", "k_rowdot.hip", "k_rowaxpy.hip", "k_attn.hip", "k_topk.hip", "k_batched.hip", "k_blocked.hip",
           "k_train.hip", "k_check.hip", "dv_noalloc.hip"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def build(verbose: bool = False, jobs: int = 8) -> None:
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    cmds = []
    for s in SOURCES:
        o = os.path.join(BUILD, s.replace(".hip", ".o"))
        objs.append(o)
        cmds.append([HIPCC, *FLAGS, *inc, "-c", os.path.join(CSRC, s), "-o", o])
    synth_obj = os.path.join(BUILD, "synth_fill.o")
    cmds.append([HIPCC, *FLAGS, "-c", SYNTH_SRC, "-o", synth_obj])
    stream_obj = os.path.join(BUILD, "synth_stream.o")
    cmds.append([HIPCC, *FLAGS, "-c", SYNTH_STREAM_SRC, "-o", stream_obj])
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    tmp = SYNTH_LIB + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, synth_obj, stream_obj])
    os.replace(tmp, SYNTH_LIB)
    if verbose:
        print("built", LIB, SYNTH_LIB)


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
