"""Build ``libpred.so`` (the predictor's C-ABI library) for gfx950 with hipcc, in-tree."""

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpred.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    # packed fp32 VALU ops are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
SOURCES = ["pred_api.hip", "proj.hip", "score_decode.hip", "score_prefill.hip", "score_rows.hip", "rank.hip",
           "prng.cpp"]
# the projection generator must be plain IEEE float64 arithmetic, one operation at a time
EXTRA = {
    "prng.cpp": ["-ffp-contract=off", "-fno-fast-math"],
    # MFMA results straight into VGPRs: the max epilogue then reads them without
    # accumulator-register copies
    "score_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"],
    # The MFMA scorers take maxima of MFMA results.  Without NaN semantics fmaxf
    # is a plain v_max3_f32; with them every operand the compiler cannot prove
    # quiet first goes through a canonicalising v_max_f32 (one more instruction
    # per element), and the NaN-propagating maximum (v_maximum3_f32) measured
    # slower than both.  These files write NaN only as integer bit patterns, and
    # a NaN product (a slot holding non-finite keys) gives an unspecified score.
    "score_rows.hip": ["-fno-honor-nans"],
}


def _compile(src):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
