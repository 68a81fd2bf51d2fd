"""The boundary's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

api.cpp (validation, workspace layout, aliasing checks) is compiled with the
sanitizers on its host code only (-Xarch_host before each -fsanitize=; the
device code is untouched) and linked with the ordinary kernel objects into a
separate library.  A C program linked with the sanitizer runtime then drives
every entry point through calls that fail validation or only query sizes -
null pointers, bad shapes, extreme sizes, overlapping buffers, misaligned
pointers, half-given state, pointer arrays with holes - so no HIP call is
made and no GPU is needed.  Any out-of-bounds read, use of uninitialised
memory through a bad pointer, or signed overflow in that code fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(ROOT, "compressive_linear_memory_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]

DRIVER = r"""
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include "infini.h"

static int fails = 0;
#define EXPECT(cond) do { if (!(cond)) { printf("FAILED: %s (line %d)\n", #cond, __LINE__); ++fails; } } while (0)

/* distinct fake device addresses, never dereferenced (validation fails first) */
#define FAKE(i) ((void*)(uintptr_t)(0x10000000u * (uintptr_t)((i) + 1)))

int main(void) {
  infini_problem_t p = {1, 4, 2, 64, 64, 16, INFINI_BF16};
  const float* F = (const float*)FAKE(12);
  float* Fo = (float*)FAKE(13);

  /* size queries over valid, invalid and extreme shapes */
  const int32_t dims[] = {-1, 0, 1, 3, 16, 64, 100, 2048, 65536, 2147483647};
  for (int a = 0; a < 10; ++a)
    for (int b = 0; b < 10; ++b) {
      infini_problem_t q = {dims[a], 4, 2, dims[b], 128, 64, INFINI_BF16};
      (void)infini_fwd_workspace_bytes(&q);
      (void)infini_bwd_workspace_bytes(&q);
      (void)infini_fwd_saved_bytes(&q);
      (void)infini_decode_workspace_bytes(&q);
      (void)infini_fwd_path(&q);
      for (int np = -1; np <= 3; ++np)
        for (int gr = -1; gr <= 9; gr += 5) (void)infini_fwd_stream_workspace_bytes(&q, np, gr);
      q.seg_len = dims[b] > 0 ? dims[b] : 1;
      q.seq_len = dims[a];
      (void)infini_fwd_workspace_bytes(&q);
      (void)infini_bwd_workspace_bytes(&q);
    }
  EXPECT(infini_fwd_workspace_bytes(NULL) == 0);
  EXPECT(infini_fwd_saved_bytes(&p) == (size_t)1 * 4 * 64 * 4);

  /* forward */
  EXPECT(infini_attn_fwd(NULL, FAKE(0), FAKE(1), FAKE(2), F, NULL, NULL, FAKE(3), Fo, Fo, NULL, NULL, 0, NULL) == INFINI_ERR_NULL);
  EXPECT(infini_attn_fwd(&p, NULL, FAKE(1), FAKE(2), F, NULL, NULL, FAKE(3), Fo, Fo, NULL, NULL, 0, NULL) == INFINI_ERR_NULL);
  EXPECT(infini_attn_fwd(&p, FAKE(0), FAKE(1), FAKE(2), F, (const float*)FAKE(5), NULL, FAKE(3), Fo, Fo, NULL, NULL, 0, NULL) == INFINI_ERR_NULL);
  EXPECT(infini_attn_fwd(&p, (char*)FAKE(0) + 2, FAKE(1), FAKE(2), F, NULL, NULL, FAKE(3), (float*)FAKE(4), (float*)FAKE(5), NULL, NULL, 0, NULL) == INFINI_ERR_UNSUPPORTED);
  EXPECT(infini_attn_fwd(&p, FAKE(0), FAKE(1), FAKE(2), F, NULL, NULL, FAKE(0), (float*)FAKE(4), (float*)FAKE(5), NULL, NULL, 0, NULL) == INFINI_ERR_ALIAS);
  infini_problem_t lp = {2, 8, 2, 1000, 128, 384, INFINI_BF16};
  EXPECT(infini_attn_fwd(&lp, FAKE(0), FAKE(1), FAKE(2), F, NULL, NULL, FAKE(3), (float*)FAKE(4), (float*)FAKE(5), NULL,
                         FAKE(6), infini_fwd_workspace_bytes(&lp) - 1, NULL) == INFINI_ERR_WORKSPACE);
  infini_problem_t bad = p;
  bad.q_heads = 3;
  EXPECT(infini_attn_fwd(&bad, FAKE(0), FAKE(1), FAKE(2), F, NULL, NULL, FAKE(3), Fo, Fo, NULL, NULL, 0, NULL) == INFINI_ERR_SHAPE);
  bad = p; bad.head_dim = 96;
  EXPECT(infini_attn_fwd(&bad, FAKE(0), FAKE(1), FAKE(2), F, NULL, NULL, FAKE(3), Fo, Fo, NULL, NULL, 0, NULL) == INFINI_ERR_UNSUPPORTED);
  bad = p; bad.dtype = 7;
  EXPECT(infini_attn_fwd(&bad, FAKE(0), FAKE(1), FAKE(2), F, NULL, NULL, FAKE(3), Fo, Fo, NULL, NULL, 0, NULL) == INFINI_ERR_UNSUPPORTED);
  bad = p; bad.batch = 2147483647; bad.q_heads = 2147483646; bad.kv_heads = 1;
  EXPECT(infini_attn_fwd(&bad, FAKE(0), FAKE(1), FAKE(2), F, NULL, NULL, FAKE(3), Fo, Fo, NULL, NULL, 0, NULL) == INFINI_ERR_SHAPE);
  bad = p; bad.seq_len = 2147483647; bad.seg_len = 1;   /* M_S and z_S given the same address */
  EXPECT(infini_attn_fwd(&bad, FAKE(0), FAKE(1), FAKE(2), F, NULL, NULL, FAKE(3), Fo, Fo, NULL, NULL, 0, NULL) == INFINI_ERR_ALIAS);

  /* phased forward */
  EXPECT(infini_fwd_memory(&lp, FAKE(1), FAKE(2), NULL, NULL, (float*)FAKE(4), (float*)FAKE(5), FAKE(6), 0, NULL) == INFINI_ERR_WORKSPACE);
  EXPECT(infini_fwd_attend(&lp, FAKE(0), FAKE(1), FAKE(2), NULL, FAKE(3), NULL, FAKE(6), 1u << 30, NULL) == INFINI_ERR_NULL);
  infini_problem_t longp = {1, 2, 2, 17 * 16, 64, 16, INFINI_BF16};
  EXPECT(infini_fwd_memory(&longp, FAKE(1), FAKE(2), NULL, NULL, (float*)FAKE(4), (float*)FAKE(5), FAKE(6), 1u << 30, NULL) == INFINI_ERR_SHAPE);

  /* backward */
  EXPECT(infini_attn_bwd(&p, FAKE(0), FAKE(1), FAKE(2), F, NULL, NULL, NULL, FAKE(3), NULL, NULL,
                         (char*)FAKE(1) + 64, FAKE(8), FAKE(9), Fo, NULL, NULL, FAKE(10), 1u << 30, NULL) == INFINI_ERR_ALIAS);
  EXPECT(infini_attn_bwd(&p, FAKE(0), FAKE(1), FAKE(2), F, NULL, NULL, NULL, FAKE(3), (const float*)FAKE(14), NULL,
                         FAKE(7), FAKE(8), FAKE(9), (float*)FAKE(11), NULL, NULL, FAKE(10), 1u << 30, NULL) == INFINI_ERR_NULL);
  EXPECT(infini_attn_bwd(&p, FAKE(0), FAKE(1), FAKE(2), F, NULL, NULL, NULL, FAKE(3), NULL, NULL,
                         FAKE(7), FAKE(8), FAKE(9), (float*)FAKE(11), (float*)FAKE(15), NULL, FAKE(10), 1u << 30, NULL) == INFINI_ERR_NULL);
  EXPECT(infini_attn_bwd(&p, FAKE(0), FAKE(1), FAKE(2), F, NULL, NULL, (const float*)FAKE(7), FAKE(3), NULL, NULL,
                         FAKE(7), FAKE(8), FAKE(9), (float*)FAKE(11), NULL, NULL, FAKE(10), 1u << 30, NULL) == INFINI_ERR_ALIAS);
  EXPECT(infini_attn_bwd(&lp, FAKE(0), FAKE(1), FAKE(2), F, NULL, NULL, NULL, FAKE(3), NULL, NULL,
                         FAKE(7), FAKE(8), FAKE(9), (float*)FAKE(11), NULL, NULL, FAKE(10), 64, NULL) == INFINI_ERR_WORKSPACE);

  /* streaming forward: pointer arrays with holes, overlaps and misalignment */
  infini_problem_t sp = {1, 2, 2, 16, 32, 16, INFINI_FP32};
  const void* Qs[3] = {FAKE(0), FAKE(1), FAKE(2)};
  const void* Ks[3] = {FAKE(3), FAKE(4), FAKE(5)};
  const void* Vs[3] = {FAKE(6), FAKE(7), FAKE(8)};
  void* Os[3] = {FAKE(9), FAKE(10), FAKE(11)};
  void* streams[2] = {FAKE(15), FAKE(16)};
  void* events[4] = {FAKE(17), FAKE(18), FAKE(19), FAKE(18)};
  size_t need = infini_fwd_stream_workspace_bytes(&sp, 2, 2);
  EXPECT(need > 0);
  EXPECT(infini_fwd_stream(&sp, 0, Qs, Ks, Vs, F, Fo, (float*)FAKE(14), Os, FAKE(20), need, 2, 2, NULL, streams, events) == INFINI_ERR_SHAPE);
  EXPECT(infini_fwd_stream(&sp, 3, Qs, Ks, Vs, F, Fo, (float*)FAKE(14), Os, FAKE(20), need - 1, 2, 2, NULL, streams, events) == INFINI_ERR_WORKSPACE);
  void* hole_streams[2] = {FAKE(15), NULL};
  EXPECT(infini_fwd_stream(&sp, 3, Qs, Ks, Vs, F, Fo, (float*)FAKE(14), Os, FAKE(20), need, 2, 2, NULL, hole_streams, events) == INFINI_ERR_NULL);
  const void* holeV[3] = {FAKE(6), NULL, FAKE(8)};
  EXPECT(infini_fwd_stream(&sp, 3, Qs, Ks, holeV, F, Fo, (float*)FAKE(14), Os, FAKE(20), need, 2, 2, NULL, streams, events) == INFINI_ERR_NULL);
  void* aliasO[3] = {FAKE(9), (char*)FAKE(4) + 64, FAKE(11)};
  EXPECT(infini_fwd_stream(&sp, 3, Qs, Ks, Vs, F, Fo, (float*)FAKE(14), aliasO, FAKE(20), need, 2, 2, NULL, streams, events) == INFINI_ERR_ALIAS);
  const void* misK[3] = {FAKE(3), (char*)FAKE(4) + 2, FAKE(5)};
  EXPECT(infini_fwd_stream(&sp, 3, Qs, misK, Vs, F, Fo, (float*)FAKE(14), Os, FAKE(20), need, 2, 2, NULL, streams, events) == INFINI_ERR_UNSUPPORTED);

  /* decode */
  infini_problem_t dp = {1, 4, 2, 3, 64, 16, INFINI_BF16};
  size_t dneed = infini_decode_workspace_bytes(&dp);
  EXPECT(dneed > 0);
  EXPECT(infini_decode(&dp, 14, FAKE(0), FAKE(1), FAKE(2), F, FAKE(3), FAKE(4), NULL, NULL, FAKE(5), NULL, NULL, FAKE(6), dneed, NULL) == INFINI_ERR_SHAPE);
  EXPECT(infini_decode(&dp, -1, FAKE(0), FAKE(1), FAKE(2), F, FAKE(3), FAKE(4), NULL, NULL, FAKE(5), NULL, NULL, FAKE(6), dneed, NULL) == INFINI_ERR_SHAPE);
  EXPECT(infini_decode(&dp, 13, FAKE(0), FAKE(1), FAKE(2), F, FAKE(3), FAKE(4), NULL, NULL, FAKE(5), NULL, NULL, FAKE(6), dneed, NULL) == INFINI_ERR_NULL);
  EXPECT(infini_decode(&dp, 0, FAKE(0), FAKE(1), FAKE(2), F, FAKE(3), FAKE(4), NULL, NULL, FAKE(3), NULL, NULL, FAKE(6), dneed, NULL) == INFINI_ERR_ALIAS);
  EXPECT(infini_decode(&dp, 0, FAKE(0), FAKE(1), FAKE(2), F, FAKE(3), FAKE(4), NULL, NULL, FAKE(5), NULL, NULL, FAKE(6), dneed - 1, NULL) == INFINI_ERR_WORKSPACE);

  for (int s = -1; s < 9; ++s) EXPECT(infini_status_string((infini_status_t)s) != NULL);
  if (fails) return 1;
  printf("ok\n");
  return 0;
}
"""


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout + r.stderr
    return r


def test_validation_paths_under_asan_and_ubsan():
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("hipcc / clang not found")
    work = os.path.join(ROOT, "_build", "sanitize")
    os.makedirs(work, exist_ok=True)
    common = ["-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", INCLUDE]
    objs = []
    for f in sorted(os.listdir(CSRC)):
        if not f.endswith((".hip", ".cpp")):
            continue
        obj = os.path.join(work, f + ".o")
        # the boundary code is sanitized; the kernel files only need to link
        extra = SAN if f == "api.cpp" else ["-O0"]
        _run([HIPCC, *common, *extra, "-c", os.path.join(CSRC, f), "-o", obj])
        objs.append(obj)
    lib = os.path.join(work, "libinfini_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN, "-o", lib, *objs])
    src = os.path.join(work, "driver.c")
    exe = os.path.join(work, "driver")
    with open(src, "w") as f:
        f.write(DRIVER)
    _run([CLANG, "-std=c99", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-I", INCLUDE, src, "-L", work, "-linfini_san", "-Wl,-rpath," + work, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
