"""Build libtcb.so (the HIP library behind include/tcb.h) in-tree for gfx950.

    python -m trie_constrained_beam_amd.build

hipcc cross-compiles without a GPU. Every HIP source is compiled with packed FP32
instructions disabled. Sources are compiled to objects in parallel (some with flags of
their own) and linked into one shared library.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtcb.so")
SOURCES = ["kernels.hip", "tile_f32.hip", "tile_bf16.hip", "tile_f32_sampled.hip", "tile_bf16_sampled.hip",
           "tile_head.hip", "lmhead.hip", "score.hip", "tcb_api.cpp", "score_api.cpp", "trie_builder.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


# The scoring kernels use no NaN (inputs are finite; -inf marks SIDs past the end), so
# max and min need no quieting of signalling NaNs there.
EXTRA_FLAGS = {"score.hip": ["-fno-honor-nans"]}


def hipcc_flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-result", "-I", os.path.join(ROOT, "include")]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd[-3:]))
    if verbose and (r.stdout or r.stderr):
        sys.stderr.write(r.stdout + r.stderr)


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="tcb_build_") as tmpdir:
        jobs = []
        for src in SOURCES:
            obj = os.path.join(tmpdir, src + ".o")
            jobs.append((obj, [HIPCC] + hipcc_flags() + EXTRA_FLAGS.get(src, []) +
                         ["-c", os.path.join(CSRC, src), "-o", obj]))
        with cf.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
            list(ex.map(lambda j: _run(j[1], verbose), jobs))
        tmp = LIB + ".tmp"
        _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + [o for o, _ in jobs] + ["-o", tmp], verbose)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
