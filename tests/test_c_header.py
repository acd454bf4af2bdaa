"""include/pred.h is a plain C header: a C11 program (and a C++17 one) that includes it builds
with every warning an error, links against the library, and its host-only calls behave as the
header states when called from C (no device needed)."""

import os
import shutil
import subprocess

import pytest

import rank_kv_block_amd as rk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_PROGRAM = r"""
#include "pred.h"
#include <stdio.h>
#include <string.h>

#define CHECK(cond) do { if (!(cond)) { printf("failed: %s (line %d)\n", #cond, __LINE__); return 1; } } while (0)

int main(void) {
    pred_dims d = {32, 32, 8, 128, 32, 16, 8192};
    /* A_g = L * N * Hk * B * r * 2 bytes */
    CHECK(pred_a_g_bytes(&d) == (int64_t)32 * 8192 * 8 * 16 * 32 * 2);
    CHECK(pred_check_fit(&d, (uint64_t)1 << 40) == PRED_OK);
    CHECK(pred_check_fit(&d, (uint64_t)1 << 20) == PRED_ERR_OOM);
    CHECK(strlen(pred_last_error()) > 0);
    pred_dims bad = d;
    bad.num_kv_heads = 5;                       /* 32 is not a multiple of 5 */
    CHECK(pred_a_g_bytes(&bad) < 0);
    /* rows of up to 2048 keys sort inside one workgroup: no workspace */
    CHECK(pred_rank_workspace_bytes(2048, 7) == 0);
    CHECK(pred_rank_workspace_bytes(8192, 32) >= (size_t)8 * 8192 * 32);
    CHECK(pred_set_score_path(7) == PRED_ERR_OUT_OF_RANGE);
    CHECK(pred_get_score_path() == PRED_SCORE_PATH_AUTO);
    /* a NULL handle is refused before any device work */
    pred_bf16 q[8] = {0};
    CHECK(pred_project_q(NULL, q, 1, q, NULL) == PRED_ERR_NULL_ARG);
    CHECK(pred_score_kernel_name(NULL, 1) == NULL);
    printf("ok\n");
    return 0;
}
"""


def _build(tmp_path, compiler, std, src_name):
    src = tmp_path / src_name
    src.write_text(C_PROGRAM)
    exe = tmp_path / (src_name + ".out")
    libdir = os.path.dirname(os.path.abspath(rk._lib.LIB_PATH))
    libname = os.path.basename(rk._lib.LIB_PATH)
    if libname != "libpred.so":
        pytest.skip("the binding loads a library under another name")
    cmd = [compiler, f"-std={std}", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           str(src), "-o", str(exe), "-L", libdir, "-lpred", f"-Wl,-rpath,{libdir}"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


@pytest.mark.parametrize("compiler,std,src_name", [("gcc", "c11", "abi.c"), ("g++", "c++17", "abi.cpp")])
def test_header_compiles_links_and_runs(tmp_path, compiler, std, src_name):
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not found")
    rk.lib()   # the library is built
    exe = _build(tmp_path, compiler, std, src_name)
    env = dict(os.environ)
    env.pop("PRED_SCORE_PATH", None)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
