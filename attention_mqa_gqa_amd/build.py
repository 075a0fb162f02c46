"""Build libmqa_attn.so (and the probe library libmqa_peaks.so) in-tree
with hipcc for gfx950.

``python attention_mqa_gqa_amd/build.py`` (or ``build_library()``) compiles
every ``csrc/*.hip`` file to an object and links them into
``attention_mqa_gqa_amd/libmqa_attn.so``, and ``peaks/peaks.hip`` into
``attention_mqa_gqa_amd/libmqa_peaks.so``.  It always recompiles.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_NAME = "libmqa_attn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
PEAKS_SRC = os.path.join(PKG_DIR, "peaks", "peaks.hip")
PEAKS_LIB_PATH = os.path.join(PKG_DIR, "libmqa_peaks.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Kernels whose large O^T accumulators are pinned to AGPRs by inline asm
# take the VGPR form for every compiler-generated MFMA, which keeps their
# score accumulators in VGPRs (where the softmax reads them) instead of
# shuffling one O^T tile between the two register files every key tile.
PER_FILE_FLAGS = {
    "prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "mla_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, extra):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, *PER_FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines()
                     if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    return obj, errs


def _link(objs, path):
    tmp = path + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, path)


def build_library(verbose=False, extra_flags=()):
    """Compile all HIP sources and link the shared libraries. Returns the
    attention library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = _sources() + [PEAKS_SRC]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda s: _compile(s, list(extra_flags)), srcs))
    objs = [r[0] for r in results]
    if verbose:
        for _, errs in results:
            if errs.strip():
                print(errs, file=sys.stderr)
    _link(objs[:-1], LIB_PATH)
    _link(objs[-1:], PEAKS_LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
