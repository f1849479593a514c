"""Build the gfx950 scorer library (libmxscore.so) in-tree with hipcc.

Runs on any machine with ROCm (hipcc cross-compiles for gfx950 without a GPU).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmxscore.so")
SOURCES = [os.path.join(CSRC, "mxs_api.cpp"), os.path.join(CSRC, "mxs_decode.hip"), os.path.join(CSRC, "mxs_prefill.hip"),
           os.path.join(CSRC, "mxs_logits.hip"), os.path.join(CSRC, "mxs_select.hip"),
           os.path.join(CSRC, "mxs_write.hip"), os.path.join(CSRC, "mxs_attn.hip")]
HEADERS = [os.path.join(ROOT, "include", "mxscore.h"), os.path.join(CSRC, "mxs_internal.h"),
           os.path.join(CSRC, "mxs_device.h")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 ops (v_pk_*_f32) are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


# The prefill and logits kernels compare and fold finite scores (masked tokens are -inf,
# never NaN), so their translation unit is compiled without NaN semantics,
# which removes NaN-quieting copies around the max folds of loop-carried
# MFMA results. Decode runs measurably faster with default semantics.
# The block-score kernel's loops start on 64-byte boundaries: where its tile
# loop happened to start moved the chunked prefill by 2% between builds that
# differed only in code outside the loop (start at byte 40 of a 64-byte line
# against byte 4); aligned, its speed no longer depends on such changes.
EXTRA_FLAGS = {"mxs_prefill.hip": ["-fno-honor-nans", "-falign-loops=64"], "mxs_logits.hip": ["-fno-honor-nans"]}


def build(force: bool = True, verbose: bool = False) -> str:
    if not force and os.path.exists(LIB):
        newest = max(os.path.getmtime(p) for p in SOURCES + HEADERS)
        if os.path.getmtime(LIB) >= newest:
            return LIB
    tmp = LIB + ".tmp"
    objs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, os.path.basename(src) + ".o")
        extra = EXTRA_FLAGS.get(os.path.basename(src), [])
        cmd = [HIPCC, *FLAGS, *extra, "-c", "-o", obj, src]
        cmd.remove("-shared")
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc failed to compile {os.path.basename(src)}")
        objs.append(obj)
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to link libmxscore.so")
    os.replace(tmp, LIB)
    for obj in objs:
        os.remove(obj)
    return LIB


if __name__ == "__main__":
    print(build(force=True, verbose=True))
