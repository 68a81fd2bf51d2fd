"""The boundary from plain C: a C99 program compiled against include/infini.h
with -Wall -Werror and linked against libinfini.so.

The program makes only calls that fail validation or query sizes, so it runs
without a GPU (validation happens on the host before any HIP call).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(ROOT, "compressive_linear_memory_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "infini.h"

#define CHECK(cond) do { if (!(cond)) { printf("FAILED: %s (line %d)\n", #cond, __LINE__); return 1; } } while (0)

int main(void) {
  infini_problem_t p = {1, 4, 2, 64, 64, 16, INFINI_BF16, INFINI_FEATURE_ELU1};
  char fake[64];
  void* a = fake;
  const float* fa = (const float*)fake;
  float* fo = (float*)fake;

  CHECK(infini_version() == INFINI_VERSION);
  CHECK(strcmp(infini_status_string(INFINI_OK), "ok") == 0);
  CHECK(infini_fwd_workspace_bytes(&p) > 0);
  CHECK(infini_bwd_workspace_bytes(&p) > 0);
  CHECK(infini_fwd_workspace_bytes(NULL) == 0);

  /* a NULL problem, a bad head split and an unsupported head_dim are refused
     before anything is launched */
  CHECK(infini_attn_fwd(NULL, a, a, a, fa, NULL, NULL, a, fo, fo, NULL, a, 0, NULL) == INFINI_ERR_NULL);
  infini_problem_t bad = p;
  bad.kv_heads = 3;
  CHECK(infini_attn_fwd(&bad, a, a, a, fa, NULL, NULL, a, fo, fo, NULL, a, 0, NULL) == INFINI_ERR_SHAPE);
  bad = p;
  bad.head_dim = 48;
  CHECK(infini_attn_fwd(&bad, a, a, a, fa, NULL, NULL, a, fo, fo, NULL, a, 0, NULL) == INFINI_ERR_UNSUPPORTED);
  /* a workspace smaller than the query returns (long segments: memory phase
     then attention phase) */
  infini_problem_t lp = {1, 4, 2, 256, 64, 128, INFINI_BF16, INFINI_FEATURE_ELU1};
  CHECK(infini_attn_fwd(&lp, a, a, a, fa, NULL, NULL, a, fo, fo, NULL, a,
                        infini_fwd_workspace_bytes(&lp) - 1, NULL) == INFINI_ERR_WORKSPACE);
  /* the fused short-segment forward needs none: with no workspace the call
     gets as far as the aliasing check (every pointer here is the same) */
  CHECK(strcmp(infini_fwd_path(&p), "mfma_bf16_short") == 0);
  CHECK(infini_attn_fwd(&p, a, a, a, fa, NULL, NULL, a, fo, fo, NULL, NULL, 0, NULL) == INFINI_ERR_ALIAS);
  CHECK(infini_attn_bwd(&p, a, a, a, fa, NULL, NULL, NULL, NULL, NULL, NULL, a, a, a, fo, NULL, NULL,
                        a, 1u << 30, NULL) == INFINI_ERR_NULL);
  CHECK(infini_decode_workspace_bytes(&p) == 0); /* 64 new tokens do not fit a 16-token segment */
  printf("ok\n");
  return 0;
}
"""


def test_header_compiles_as_c99_and_links():
    gcc = shutil.which("gcc")
    lib = os.path.join(LIBDIR, "libinfini.so")
    if gcc is None or not os.path.exists(lib):
        pytest.skip("gcc or libinfini.so missing")
    work = os.path.join(ROOT, "_build", "c_abi_test")
    os.makedirs(work, exist_ok=True)
    src = os.path.join(work, "abi.c")
    exe = os.path.join(work, "abi")
    with open(src, "w") as f:
        f.write(PROGRAM)
    cc = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", INCLUDE, src,
                         "-L", LIBDIR, "-linfini", "-Wl,-rpath," + LIBDIR, "-o", exe],
                        capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
