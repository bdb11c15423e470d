"""Build libmc.so (the C-ABI library) and libmcpeak.so (the benchmark's ceiling kernels)
in-tree with hipcc for gfx950.

    python -m chunked_linear_attention_segment_amd.build

Every source is compiled on each call (the build check compiles even where a library is
already present); objects go to _build/ and the libraries next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmc.so")
PEAK_OUT = os.path.join(HERE, "libmcpeak.so")
BUILD_DIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["abi.cpp", "scan.hip", "readout.hip", "decode.hip", "read_mfma.hip", "scan_mfma.hip",
           "gate.hip", "backward.hip", "backward_mfma.hip", "ssc_gather.hip", "dgamma_mfma.hip"]
PEAK_SOURCES = ["peak.hip"]
# Per-file flags.  The gated read and the dgamma pass are written in the exact issue order
# they need (each MFMA followed by the VALU work it hides, LDS reads two k-steps ahead); the
# machine schedulers would regroup it, so they are off for those files.
FILE_FLAGS = {name: ["-mllvm", "-enable-misched=false", "-mllvm", "-enable-post-misched=false"]
              for name in ("read_mfma.hip", "dgamma_mfma.hip")}

# Packed-fp32 VALU ops are kept out of the device code (the host pass warns that it does
# not know the feature; that warning is harmless).
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH, "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + FILE_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC] + [f for f in FLAGS if not f.startswith("--offload-arch")] + \
              ["-x", "c++", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def _link(objs, out):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PEAK_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], OUT)
    _link([objs[s] for s in PEAK_SOURCES], PEAK_OUT)
    if verbose:
        print("built", OUT, PEAK_OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
