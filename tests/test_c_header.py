"""include/cpa.h and include/cpa_diag.h are plain C: a C99 program that includes both compiles
with warnings as errors, links against libcpa.so and libcpa_diag.so by the declared names, and
gets the host-side argument checks' codes back (no GPU needed: every call here is rejected, or
answered, before any HIP call).  The same source also compiles as C++17."""
import os
import shutil
import subprocess

import pytest

from sparse_attention_long_reduce_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
PKG = os.path.dirname(_lib.LIB_PATH)
HIP_INCLUDE = "/opt/rocm/include"

PROGRAM = r"""
#include "cpa.h"
#include "cpa_diag.h"
#include <stdio.h>
#include <string.h>

int main(void) {
  int32_t zero = 0;
  int bad = 0;
  /* B < 0 */
  if (cpa_build_block_tables(NULL, -1, 1, 1, 1, 1, &zero, &zero, NULL, 1, NULL, 0) != CPA_ERR_SHAPE) bad |= 1;
  /* table capacity below the KV-block count */
  if (cpa_build_block_tables(NULL, 1, 1, 1, 1, 8, &zero, &zero, NULL, 4, NULL, 0) != CPA_ERR_CAPACITY) bad |= 2;
  /* head dim 96 */
  if (cpa_chunked_prefill(NULL, CPA_BF16, NULL, NULL, 96 * 64, 96 * 64, 96, 1, NULL, 1, NULL, 1, NULL, NULL, NULL,
                          1, 1, 1, 96, 64, 0.0f, NULL, NULL, 0) != CPA_ERR_UNSUPPORTED) bad |= 4;
  /* Hq not a multiple of Hkv */
  if (cpa_chunked_prefill(NULL, CPA_BF16, NULL, NULL, 128 * 64, 128 * 64, 128, 1, NULL, 1, NULL, 1, NULL, NULL,
                          NULL, 1, 3, 2, 128, 64, 0.0f, NULL, NULL, 0) != CPA_ERR_SHAPE) bad |= 8;
  if (strcmp(cpa_status_string(CPA_OK), "ok") != 0) bad |= 16;
  /* 8 ranges of 256 pages over a 2048-block table, 2048 rows, 32 heads, d = 128 */
  if (cpa_split_workspace_bytes(2048, 32, 128, 2048, 256) != (size_t)8 * 2048 * 32 * 129 * 4) bad |= 32;
  if (cpa_split_workspace_bytes(2048, 32, 128, 2048, 4096) != 0) bad |= 64;
  /* threads not a multiple of 64 */
  if (cpa_diag_mfma_loop(1, 100, 1, NULL, NULL, 0) == CPA_OK) bad |= 128;
  printf("version %d block %d bad %d\n", cpa_version(), CPA_BLOCK, bad);
  return bad;
}
"""


def _toolchain(name):
    path = shutil.which(name)
    if path is None:
        pytest.skip(f"{name} is not installed")
    if not os.path.exists(os.path.join(HIP_INCLUDE, "hip", "hip_runtime_api.h")):
        pytest.skip("the HIP headers are not installed")
    return path


@pytest.fixture(scope="module")
def built():
    for p in (_lib.LIB_PATH, _lib.DIAG_LIB_PATH):
        if not os.path.exists(p):
            pytest.fail(f"{p} is not built (run __graft_entry__.build())")


@pytest.mark.parametrize("lang", ["c", "c++"])
def test_headers_compile_link_and_check_arguments(built, tmp_path, lang):
    compiler = _toolchain("gcc" if lang == "c" else "g++")
    src = tmp_path / ("abi.c" if lang == "c" else "abi.cpp")
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    std = "-std=c99" if lang == "c" else "-std=c++17"
    cmd = [compiler, std, "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I" + INCLUDE,
           "-I" + HIP_INCLUDE, str(src), "-L" + PKG, "-lcpa", "-lcpa_diag", "-Wl,-rpath," + PKG, "-o", str(exe)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    run = subprocess.run([str(exe)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    assert run.returncode == 0, run.stdout
    assert "block 64 bad 0" in run.stdout, run.stdout
