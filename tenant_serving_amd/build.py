"""In-tree build of the native libraries (hipcc for gfx950, gcc for host C).

    python -m tenant_serving_amd.build        # builds everything into lib/

Libraries:
  lib/libbitdelta.so      the C-ABI library (include/bitdelta.h): HIP kernels + host API
  lib/libbdsynth_dev.so   device side of the synthetic input generator
  lib/libbdsynth_host.so  host side of the synthetic input generator (gcc, no HIP)
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_DIR = os.path.join(HERE, "lib")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Every HIP compile: gfx950 only, packed-fp32 VALU ops disabled, no fast-math.
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I" + INCLUDE, "-I" + CSRC]

BITDELTA_SOURCES = ["bd_api.hip", "bd_compress.hip", "bd_apply.hip", "bd_decode.hip", "bd_delta.hip", "bd_gemm.hip",
                    "bd_reconstruct.hip"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    return r


def build_synth_host(verbose=False):
    out = os.path.join(LIB_DIR, "libbdsynth_host.so")
    _run(["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-I" + CSRC, os.path.join(CSRC, "synth_host.c"), "-o", out], verbose)
    return out


def build_synth_dev(verbose=False):
    out = os.path.join(LIB_DIR, "libbdsynth_dev.so")
    _run([HIPCC] + HIP_FLAGS + ["-ffp-contract=off", "-shared",
                                os.path.join(CSRC, "synth_dev.hip"), "-o", out], verbose)
    return out


def build_bitdelta(verbose=False):
    out = os.path.join(LIB_DIR, "libbitdelta.so")
    objs = []

    def comp(src):
        obj = os.path.join(LIB_DIR, "obj", src.replace(".hip", ".o"))
        _run([HIPCC] + HIP_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj], verbose)
        return obj

    os.makedirs(os.path.join(LIB_DIR, "obj"), exist_ok=True)
    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(comp, BITDELTA_SOURCES))
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", out], verbose)
    return out


def build_all(verbose=False):
    os.makedirs(LIB_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=3) as ex:
        futs = [ex.submit(build_synth_host, verbose), ex.submit(build_synth_dev, verbose)]
        if all(os.path.exists(os.path.join(CSRC, s)) for s in BITDELTA_SOURCES):
            futs.append(ex.submit(build_bitdelta, verbose))
        return [f.result() for f in futs]


if __name__ == "__main__":
    for p in build_all(verbose="-v" in sys.argv):
        print("built", p)
