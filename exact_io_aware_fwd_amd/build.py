"""Build the HIP library (gfx950 only) in-tree: exact_io_aware_fwd_amd/libexact_attn.so.

    python -m exact_io_aware_fwd_amd.build [--debug]

Every source is compiled with hipcc for gfx950; objects go to _build/ and are
linked into one shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libexact_attn.so")
# a standalone streaming-read probe (the practical HBM read rate beside the
# published peak); not part of the library
PROBE_SRC = os.path.join(CSRC, "hbm_read_probe.hip")
PROBE = os.path.join(BUILD, "hbm_read_probe")
SOURCES = ["api.hip", "prefill_bf16.hip", "prefill_f32.hip", "decode.hip", "backward.hip", "backward_f32.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-fp32 VALU forms are kept out of generated code (they are disabled at
# the target-feature level rather than relied on).
COMMON = ["--offload-arch=" + ARCH, "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include")]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def build(debug: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    opt = ["-O0", "-g"] if debug else ["-O3"]
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([HIPCC, *COMMON, *opt, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(4, len(cmds))) as ex:
        for r, cmd in zip(ex.map(_run, cmds), cmds):
            if verbose:
                print(" ".join(cmd))
                sys.stdout.write(r.stderr)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    _run([HIPCC, *COMMON, "-O3", PROBE_SRC, "-o", PROBE + ".tmp"])
    os.replace(PROBE + ".tmp", PROBE)
    return LIB


if __name__ == "__main__":
    print(build(debug="--debug" in sys.argv, verbose="-v" in sys.argv))
