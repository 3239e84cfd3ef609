"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Every source is compiled with the sanitizers on its host side (the device code as usual),
and linked with a C program that drives the entry points through every path that returns
before a HIP call: argument and alignment checks of each entry point, the split, per-row
and INT8 flag validation and the variant tables behind it, the factor choice over a range
of sizes, status strings, and the KQ_LOG debug lines. Any sanitizer report fails the run
(leak detection on, undefined behaviour fatal)."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kronecker_factored_transforms_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")

DRIVER = r"""
#include <math.h>
#include <stdio.h>
#include <string.h>
#include "kq.h"

static int fails = 0;
#define CHECK(c) do { if (!(c)) { printf("FAIL line %d: %s\n", __LINE__, #c); ++fails; } } while (0)
#define P(a) ((const void *)(a))

static kq_status create(int n1, int n2, kq_dtype xd, kq_dtype sd, const void *p1, const void *p2,
                        const float *c, float alpha, unsigned flags) {
  kq_plan *h = (kq_plan *)16;
  kq_status st = kq_create_ex(&h, n1, n2, xd, sd, p1, p2, c, alpha, NULL, flags);
  if (h != NULL) { printf("FAIL: plan left set on error\n"); ++fails; }
  return st;
}

static kq_status gemm(int64_t T, int64_t N, int64_t K, kq_dtype sd, kq_dtype od, const void *xq,
                      const void *sx, const void *wq, const void *sw, void *out, int64_t ldxq,
                      int64_t ldo) {
  return kq_int4_gemm((const uint8_t *)xq, ldxq, sx, T, (const uint8_t *)wq, K / 2, sw, N, K, sd,
                      od, out, ldo, NULL);
}

int main(void) {
  int a = 0, b = 0;
  for (int64_t n = 1; n <= 70000; ++n) {
    CHECK(kq_choose_factors(n, &a, &b) == KQ_OK && (int64_t)a * b == n && a <= b);
  }
  CHECK(kq_choose_factors(0, &a, &b) == KQ_ERR_INVALID_ARG);
  CHECK(kq_choose_factors(64, NULL, &b) == KQ_ERR_INVALID_ARG);
  for (int s = -2; s < 12; ++s) CHECK(strlen(kq_status_string((kq_status)s)) > 0);
  CHECK(kq_version() > 0);

  /* plan creation: rejected before any HIP call */
  CHECK(kq_create_ex(NULL, 8, 8, KQ_BF16, KQ_FP16, P(16), P(16), NULL, 1.f, NULL, 0) == KQ_ERR_INVALID_ARG);
  CHECK(create(0, 8, KQ_BF16, KQ_FP16, P(16), P(16), NULL, 1.f, 0) == KQ_ERR_INVALID_ARG);
  CHECK(create(3, 5, KQ_BF16, KQ_FP16, P(16), P(16), NULL, 1.f, 0) == KQ_ERR_INVALID_ARG);
  CHECK(create(1 << 13, 1 << 12, KQ_BF16, KQ_FP16, P(16), P(16), NULL, 1.f, 0) == KQ_ERR_INVALID_ARG);
  CHECK(create(8, 8, (kq_dtype)7, KQ_FP16, P(16), P(16), NULL, 1.f, 0) == KQ_ERR_INVALID_ARG);
  CHECK(create(8, 8, KQ_BF16, KQ_BF16, P(16), P(16), NULL, 1.f, 0) == KQ_ERR_INVALID_ARG);
  CHECK(create(8, 8, KQ_BF16, KQ_FP16, NULL, P(16), NULL, 1.f, 0) == KQ_ERR_INVALID_ARG);
  CHECK(create(8, 8, KQ_BF16, KQ_FP16, P(16), NULL, NULL, 1.f, 0) == KQ_ERR_INVALID_ARG);
  CHECK(create(8, 8, KQ_BF16, KQ_FP16, P(16), P(16), NULL, NAN, 0) == KQ_ERR_INVALID_ARG);
  CHECK(create(8, 8, KQ_BF16, KQ_FP16, P(16), P(16), NULL, 1.f, 0x8000u) == KQ_ERR_INVALID_ARG);
  CHECK(create(64, 128, KQ_BF16, KQ_FP16, P(16), P(16), NULL, 1.f,
               KQ_FLAG_SPLIT_REG1 | KQ_FLAG_SPLIT_COLS) == KQ_ERR_INVALID_ARG);
  CHECK(create(64, 128, KQ_FP32, KQ_FP16, P(16), P(16), NULL, 1.f, KQ_FLAG_SPLIT_REG1) == KQ_ERR_INVALID_ARG);
  CHECK(create(112, 128, KQ_BF16, KQ_FP16, P(16), P(16), NULL, 1.f, KQ_FLAG_SPLIT_REG2) == KQ_ERR_UNSUPPORTED);
  CHECK(create(8, 128, KQ_BF16, KQ_FP16, P(16), P(16), NULL, 1.f, KQ_FLAG_PER_ROW) == KQ_ERR_INVALID_ARG);
  CHECK(create(8, 128, KQ_BF16, KQ_FP16, NULL, P(16), (const float *)P(32), 1.f, KQ_FLAG_PER_ROW) == KQ_ERR_INVALID_ARG);
  CHECK(create(8, 32, KQ_BF16, KQ_FP16, NULL, P(16), NULL, 1.f, KQ_FLAG_PER_ROW | KQ_FLAG_INT8) == KQ_ERR_UNSUPPORTED);
  CHECK(create(64, 128, KQ_FP32, KQ_FP16, P(16), P(16), NULL, 1.f, KQ_FLAG_INT8) == KQ_ERR_INVALID_ARG);
  CHECK(create(64, 128, KQ_BF16, KQ_FP16, P(16), P(16), NULL, 1.f, KQ_FLAG_INT8 | KQ_FLAG_SPLIT_COLS) == KQ_ERR_UNSUPPORTED);
  CHECK(create(256, 128, KQ_FP32, KQ_FP16, P(16), P(16), NULL, 1.f, 0) == KQ_ERR_UNSUPPORTED);
  CHECK(create(208, 256, KQ_BF16, KQ_FP16, P(16), P(16), (const float *)P(32), 1.f, KQ_FLAG_SPLIT_PTILE) == KQ_ERR_UNSUPPORTED);

  /* calls on no plan, and the plan queries */
  size_t bytes = 7;
  CHECK(kq_workspace_size(NULL, 5, &bytes) == KQ_ERR_INVALID_ARG);
  CHECK(kq_transform_quant(NULL, P(16), 5, 8192, (uint8_t *)16, (void *)16, NULL, NULL) == KQ_ERR_INVALID_ARG);
  CHECK(kq_transform_quant_ws(NULL, P(16), 5, 8192, (uint8_t *)16, (void *)16, NULL, NULL, 0, NULL) == KQ_ERR_INVALID_ARG);
  CHECK(kq_transform_quant_noalloc(NULL, P(16), 5, 8192, (uint8_t *)16, (void *)16, NULL, NULL) == KQ_ERR_INVALID_ARG);
  CHECK(kq_destroy(NULL) == KQ_OK);
  CHECK(kq_plan_clip_ratio(NULL) == 0.f);
  CHECK(strlen(kq_plan_kernel_name(NULL)) == 0 && strlen(kq_plan_kernel_name_for(NULL, 3)) == 0);

  /* the INT4 GEMM and the weight-side factor */
  CHECK(gemm(0, 8, 256, KQ_FP16, KQ_FP32, P(16), P(16), P(16), P(16), (void *)16, 128, 8) == KQ_OK);
  CHECK(gemm(-1, 8, 256, KQ_FP16, KQ_FP32, P(16), P(16), P(16), P(16), (void *)16, 128, 8) == KQ_ERR_INVALID_ARG);
  CHECK(gemm(16, 8, 256, KQ_BF16, KQ_FP32, P(16), P(16), P(16), P(16), (void *)16, 128, 8) == KQ_ERR_INVALID_ARG);
  CHECK(gemm(16, 8, 256, KQ_FP16, KQ_FP32, NULL, P(16), P(16), P(16), (void *)16, 128, 8) == KQ_ERR_INVALID_ARG);
  CHECK(gemm(16, 8, 384, KQ_FP16, KQ_FP32, P(16), P(16), P(16), P(16), (void *)16, 192, 8) == KQ_ERR_UNSUPPORTED);
  CHECK(gemm(16, 6, 256, KQ_FP16, KQ_FP32, P(16), P(16), P(16), P(16), (void *)16, 128, 8) == KQ_ERR_UNSUPPORTED);
  CHECK(gemm(16, 8, 256, KQ_FP16, KQ_FP32, P(24), P(16), P(16), P(16), (void *)16, 128, 8) == KQ_ERR_ALIGNMENT);
  CHECK(kq_weight_factor(NULL, 4, KQ_BF16, (void *)16, NULL) == KQ_ERR_INVALID_ARG);
  CHECK(kq_weight_factor(P(16), 0, KQ_BF16, (void *)16, NULL) == KQ_ERR_INVALID_ARG);
  CHECK(kq_weight_factor(P(16), 4, KQ_FP16, (void *)16, NULL) == KQ_ERR_INVALID_ARG);
  CHECK(kq_weight_factor(P(17), 4, KQ_BF16, (void *)16, NULL) == KQ_ERR_ALIGNMENT);

  printf("host checks done, %d failed\n", fails);
  return fails != 0;
}
"""


def _host_sanitized_compile(src, obj):
    # the device code is compiled as usual (the host objects reference it); only the host
    # side carries the sanitizers
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
           "-fno-omit-frame-pointer", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    return obj


def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG) and os.path.exists(CLANGXX)):
        pytest.skip("ROCm compilers not available")
    from kronecker_factored_transforms_amd import build as Bd
    srcs = [os.path.join(CSRC, s) for s in Bd.SOURCES]
    objs = [str(tmp_path / (os.path.splitext(os.path.basename(s))[0] + ".o")) for s in srcs]
    with ThreadPoolExecutor(len(srcs)) as ex:
        list(ex.map(_host_sanitized_compile, srcs, objs))
    drv = tmp_path / "driver.c"
    drv.write_text(DRIVER)
    sanitize = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    r = subprocess.run([CLANG, "-std=c99", "-O1", "-g", "-Wall", "-Werror", *sanitize,
                        "-I", os.path.join(ROOT, "include"), "-c", str(drv),
                        "-o", str(tmp_path / "driver.o")], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    exe = str(tmp_path / "driver")
    r = subprocess.run([CLANGXX, *sanitize, str(tmp_path / "driver.o"), *objs, "-o", exe,
                        "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                        f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, KQ_LOG="1", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and "host checks done, 0 failed" in r.stdout, (r.stdout[-3000:], r.stderr[-3000:])
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
    # the debug log went to stderr, one line per call
    assert "[kq] create 3x5" in r.stderr and "[kq] int4_gemm" in r.stderr
