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
    # MFMA results straight into VGPRs (both MFMA scorers): the max epilogue then
    # reads them without accumulator-register copies
    "score_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"],
    # The MFMA scorers take maxima of MFMA results.  Without NaN semantics fmaxf
    # is a plain v_max3_f32; with them every operand the compiler cannot prove
    # quiet first goes through a canonicalising v_max_f32 (one more instruction
    # per element), and the NaN-propagating maximum (v_maximum3_f32) measured
    # slower than both.  These files write NaN only as integer bit patterns, and
    # a NaN product (a slot holding non-finite keys) gives an unspecified score.
    "score_rows.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"],
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


# Host-side sanitizer build: the same library with AddressSanitizer and
# UndefinedBehaviorSanitizer on its host code (argument checks, sizing, the
# projection generator, launch set-up), for the CPU tests of the C ABI.  The
# device code is the normal build's.  An object is rebuilt only when a source
# or header is newer than it.
SANITIZE_DIR = os.path.join(BUILD, "sanitize")
SANITIZED_LIB = os.path.join(SANITIZE_DIR, "libpred_san.so")
_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
        "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _newest_input(src):
    paths = [os.path.join(CSRC, src), os.path.join(INCLUDE, "pred.h"), os.path.join(CSRC, "common.h"),
             os.path.join(CSRC, "kernels.h"), os.path.abspath(__file__)]
    return max(os.path.getmtime(q) for q in paths)


def _compile_host_sanitized(src):
    obj = os.path.join(SANITIZE_DIR, src + ".o")
    if os.path.exists(obj) and os.path.getmtime(obj) > _newest_input(src):
        return obj
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), *_SAN, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build_host_sanitized(verbose=False):
    """libpred with ASan + UBSan on its host code: load it with the sanitizer
    runtime preloaded (the library links it as a shared runtime)."""
    os.makedirs(SANITIZE_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile_host_sanitized, SOURCES))
    if not (os.path.exists(SANITIZED_LIB) and os.path.getmtime(SANITIZED_LIB) > max(map(os.path.getmtime, objs))):
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-fsanitize=address,undefined",
               "-shared-libsan", "-o", SANITIZED_LIB, *objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {SANITIZED_LIB}")
    return SANITIZED_LIB


def sanitizer_runtime():
    """Path of the ASan runtime the sanitized library links against (to preload)."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
        return path
    import glob
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv:
        build_host_sanitized(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
