"""Build the gfx950 shared library ``libdcn_mi355x.so`` in-tree with hipcc.

``python -m modulated_deformable_convolution_dcn_amd.build`` or ``build()``.
Every HIP translation unit is compiled with packed-fp32 instructions turned
off (``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host pass
warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdcn_mi355x.so")

SOURCES = ["dcn_kernels.hip", "dcn_wsk.hip", "dcn_quad.hip", "dcn_bf16.hip", "dcn_bf16win.hip",
           "dcn_backward.hip",
           "dcn_msda.hip", "dcn_dsample.hip", "dcn_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I", INCLUDE, "-I", CSRC]
DEVICE = ["-x", "hip", "--offload-arch=" + ARCH,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-rdc"]


def _obj(src: str, build_dir: str) -> str:
    return os.path.join(build_dir, os.path.splitext(src)[0] + ".o")


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    build_dir = os.path.join(PKG, "_build")
    os.makedirs(build_dir, exist_ok=True)
    procs = []
    for src in SOURCES:
        cmd = [HIPCC] + COMMON + DEVICE + ["-c", os.path.join(CSRC, src), "-o", _obj(src, build_dir)]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # drop the known harmless host-pass warning about the device-only feature
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l]
        if p.returncode != 0 or (verbose and lines):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    tmp = LIB + ".tmp%d" % os.getpid()
    link = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + \
        [_obj(s, build_dir) for s in SOURCES]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
