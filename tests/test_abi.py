"""The C-ABI library: it loads, exports every entry point include/kq.h declares, and its
host-only logic (status strings, factor choice, argument checks that fail before any
HIP call) behaves as documented. No compute calls: these run without a GPU."""
import ctypes
import math
import os
import re

import pytest

from kronecker_factored_transforms_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kq.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kq_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libkq.so not built")
    return B.lib()


def test_header_declares_the_binding_exports():
    assert _declared_functions() == sorted(B.EXPORTS)


def test_every_declared_symbol_is_exported(L):
    for name in _declared_functions():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_no_torch_types_in_the_abi():
    src = open(HEADER).read()
    assert "torch" not in src.lower() and "at::" not in src and "c10" not in src


def test_status_strings_and_version(L):
    assert B.kq_status_string(0) == "ok"
    msgs = {B.kq_status_string(s) for s in range(7)}
    assert len(msgs) == 7
    assert B.kq_status_string(99) == "unknown status"
    assert B.kq_version() >= 10100


def _brute_factors(n):
    best = None
    for a in range(1, n + 1):
        if n % a == 0 and a <= n // a:
            if best is None or a + n // a < best[0] + best[1]:
                best = (a, n // a)
    return best


def test_choose_factors_page_examples_and_brute_force(L):
    # the FlatQuant page's example: hidden 8192 -> (64, 128)
    assert B.kq_choose_factors(8192) == (64, 128)
    assert B.kq_choose_factors(4096) == (64, 64)
    assert B.kq_choose_factors(14336) == (112, 128)
    for n in list(range(1, 300)) + [11008, 5120, 6144, 13824, 28672]:
        assert B.kq_choose_factors(n) == _brute_factors(n), n
    with pytest.raises(B.KqError) as e:
        B.kq_choose_factors(0)
    assert e.value.status == B.KQ_ERR_INVALID_ARG


def _create_raw(L, n1, n2, xd=B.KQ_BF16, sd=B.KQ_FP16, p1=0x1000, p2=0x2000, c=None,
                alpha=math.inf, flags=0):
    h = ctypes.c_void_p(123)
    st = L.kq_create_ex(ctypes.byref(h), n1, n2, xd, sd, p1, p2, c, ctypes.c_float(alpha), None, flags)
    return st, h.value


def test_create_rejects_bad_arguments_before_touching_the_gpu(L):
    bad = [
        dict(n1=0, n2=8), dict(n1=8, n2=-1), dict(n1=3, n2=5),            # n odd
        dict(n1=8, n2=8, xd=7), dict(n1=8, n2=8, sd=B.KQ_BF16),
        dict(n1=8, n2=8, p1=None), dict(n1=8, n2=8, p2=None),
        dict(n1=8, n2=8, alpha=float("nan")), dict(n1=8, n2=8, flags=0x8000),
        dict(n1=1 << 13, n2=1 << 12),                                        # n too large
    ]
    for kw in bad:
        st, h = _create_raw(L, **kw)
        assert st == B.KQ_ERR_INVALID_ARG, kw
        assert h is None, kw
    assert L.kq_create_ex(None, 8, 8, 0, 2, 0x1000, 0x2000, None, ctypes.c_float(1.0), None, 0) \
        == B.KQ_ERR_INVALID_ARG


def test_split_flags_are_validated_on_the_host(L):
    two = B.KQ_FLAG_SPLIT_REG1 | B.KQ_FLAG_SPLIT_COLS
    for kw in (dict(flags=two), dict(flags=B.KQ_FLAG_SPLIT_REG2 | B.KQ_FLAG_FORCE_GENERIC),
               dict(flags=B.KQ_FLAG_SPLIT_REG1, xd=B.KQ_FP32)):
        st, h = _create_raw(L, 64, 128, **kw)
        assert st == B.KQ_ERR_INVALID_ARG and h is None, kw
    # a split that is not built for the shape
    st, h = _create_raw(L, 112, 128, flags=B.KQ_FLAG_SPLIT_REG2)
    assert st == B.KQ_ERR_UNSUPPORTED and h is None


def test_per_row_flag_is_validated_on_the_host(L):
    # P1 must be NULL with the flag, bf16 only, no c, no other flag
    for kw in (dict(flags=B.KQ_FLAG_PER_ROW),                              # P1 given
               dict(flags=B.KQ_FLAG_PER_ROW, p1=None, xd=B.KQ_FP32),
               dict(flags=B.KQ_FLAG_PER_ROW, p1=None, c=0x3000),
               dict(flags=B.KQ_FLAG_PER_ROW | B.KQ_FLAG_SPLIT_REG1, p1=None)):
        st, h = _create_raw(L, 8, 128, **kw)
        assert st == B.KQ_ERR_INVALID_ARG and h is None, kw


def test_int8_flag_is_validated_on_the_host(L):
    for kw in (dict(flags=B.KQ_FLAG_INT8, xd=B.KQ_FP32),
               dict(flags=B.KQ_FLAG_INT8 | B.KQ_FLAG_FORCE_GENERIC),
               dict(flags=B.KQ_FLAG_INT8 | B.KQ_FLAG_PER_ROW, p1=None, xd=B.KQ_FP32),
               dict(flags=B.KQ_FLAG_INT8 | B.KQ_FLAG_PER_ROW | B.KQ_FLAG_FORCE_GENERIC, p1=None)):
        st, h = _create_raw(L, 64, 128, **kw)
        assert st == B.KQ_ERR_INVALID_ARG and h is None, kw
    st, h = _create_raw(L, 64, 128, flags=B.KQ_FLAG_INT8 | B.KQ_FLAG_SPLIT_COLS)
    assert st == B.KQ_ERR_UNSUPPORTED and h is None
    # per-row INT8 exists for n2 in {64, 128} only
    st, h = _create_raw(L, 8, 32, p1=None, flags=B.KQ_FLAG_INT8 | B.KQ_FLAG_PER_ROW)
    assert st == B.KQ_ERR_UNSUPPORTED and h is None


def test_create_reports_unsupported_shapes(L):
    # fp32 beyond the generic kernel's on-chip limit and no MFMA variant for it
    st, h = _create_raw(L, 256, 128, xd=B.KQ_FP32)
    assert st == B.KQ_ERR_UNSUPPORTED and h is None


def test_null_plan_paths(L):
    assert L.kq_destroy(None) == B.KQ_OK
    assert L.kq_plan_clip_ratio(None) == 0.0
    assert L.kq_plan_kernel_name(None) == b""
    assert L.kq_plan_kernel_name_for(None, 5) == b""
    assert L.kq_transform_quant(None, None, 0, 0, None, None, None, None) == B.KQ_ERR_INVALID_ARG


def _gemm_raw(L, T=16, N=8, K=256, sd=B.KQ_FP16, od=B.KQ_FP32, xq=0x1000, wq=0x2000,
              sx=0x3000, sw=0x4000, out=0x5000, ldxq=None, ldwq=None, ldo=None):
    return L.kq_int4_gemm(xq, K // 2 if ldxq is None else ldxq, sx, T, wq,
                          K // 2 if ldwq is None else ldwq, sw, N, K, sd, od, out,
                          N if ldo is None else ldo, None)


def test_int4_gemm_rejects_bad_arguments_before_touching_the_gpu(L):
    assert _gemm_raw(L, T=0) == B.KQ_OK and _gemm_raw(L, N=0) == B.KQ_OK   # nothing to do
    for kw in (dict(T=-1), dict(K=0), dict(sd=B.KQ_BF16), dict(od=7), dict(xq=None),
               dict(sw=None), dict(out=None), dict(ldxq=64), dict(ldo=4)):
        assert _gemm_raw(L, **kw) == B.KQ_ERR_INVALID_ARG, kw
    for kw in (dict(K=384), dict(K=65536 + 256), dict(N=6)):
        assert _gemm_raw(L, **kw) == B.KQ_ERR_UNSUPPORTED, kw
    for kw in (dict(xq=0x1008), dict(ldxq=136), dict(out=0x5004), dict(ldo=10), dict(sd=B.KQ_FP32, sw=0x4004)):
        assert _gemm_raw(L, **kw) == B.KQ_ERR_ALIGNMENT, kw


def test_weight_factor_rejects_bad_arguments_before_touching_the_gpu(L):
    ok = dict(P=0x1000, m=64, dtype=B.KQ_BF16, out=0x2000)
    for kw in (dict(P=None), dict(out=None), dict(m=0), dict(m=1025), dict(dtype=B.KQ_FP16),
               dict(dtype=9)):
        a = {**ok, **kw}
        assert L.kq_weight_factor(a["P"], a["m"], a["dtype"], a["out"], None) == B.KQ_ERR_INVALID_ARG, kw
    for kw in (dict(P=0x1001), dict(dtype=B.KQ_FP32, out=0x2002)):
        a = {**ok, **kw}
        assert L.kq_weight_factor(a["P"], a["m"], a["dtype"], a["out"], None) == B.KQ_ERR_ALIGNMENT, kw


def test_host_tensors_are_refused_before_any_call():
    import torch
    with pytest.raises(ValueError):
        B._ptr(torch.zeros(4))
    assert B._ptr(None) is None and B._ptr(0x1000) == 0x1000


C_CONSUMER = r"""
#include <stdio.h>
#include <string.h>
#include "kq.h"

int main(void) {
  int n1 = 0, n2 = 0;
  kq_plan *plan = (kq_plan *)1;
  if (kq_choose_factors(8192, &n1, &n2) != KQ_OK || n1 != 64 || n2 != 128) return 1;
  if (strlen(kq_status_string(KQ_ERR_UNSUPPORTED)) == 0) return 2;
  if (kq_version() <= 0) return 3;
  /* rejected on the host, before any HIP call: n1 * n2 odd */
  if (kq_create(&plan, 3, 3, KQ_BF16, KQ_FP16, (const void *)16, (const void *)16, NULL,
                1.0f, NULL) != KQ_ERR_INVALID_ARG || plan != NULL) return 4;
  if (kq_destroy(NULL) != KQ_OK) return 5;
  if (kq_weight_factor(NULL, 4, KQ_BF16, NULL, NULL) != KQ_ERR_INVALID_ARG) return 6;
  printf("ok %d %d\n", n1, n2);
  return 0;
}
"""


def test_a_c99_program_builds_against_the_header_and_links_the_library(L, tmp_path):
    """The boundary is usable from plain C: a C99 program including only kq.h compiles
    with -Wall -Wextra -pedantic, links libkq.so and runs its host-only calls."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = tmp_path / "consumer.c"
    src.write_text(C_CONSUMER)
    exe = tmp_path / "consumer"
    libdir = os.path.dirname(B.LIB_PATH)
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                        "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                        "-L", libdir, "-lkq", f"-Wl,-rpath,{libdir}"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok 64 128", (r.returncode, r.stdout, r.stderr)


def test_plan_call_refuses_wrong_output_buffers():
    """Caller-provided (codes, scales) are checked before any pointer reaches the C ABI:
    a buffer of the wrong size, dtype, layout or device would be written past its end."""
    import torch
    p = B.Plan.__new__(B.Plan)
    p.handle, p.n1, p.n2, p.n, p.bits, p.per_row = None, 64, 128, 8192, 4, False
    p.x_dtype, p.scale_dtype = torch.bfloat16, torch.float16
    T = 5
    X = torch.zeros((T, 8192), dtype=torch.bfloat16)
    good_c = torch.empty((T, 4096), dtype=torch.uint8)
    good_s = torch.empty((T,), dtype=torch.float16)
    bad = [
        (torch.empty((T - 1, 4096), dtype=torch.uint8), good_s),          # short codes
        (torch.empty((T, 4096), dtype=torch.int8), good_s),               # dtype
        (torch.empty((4096, T), dtype=torch.uint8).t(), good_s),          # not contiguous
        (good_c, torch.empty((T - 1,), dtype=torch.float16)),             # short scales
        (good_c, torch.empty((T,), dtype=torch.float32)),                 # scale dtype
        (good_c, torch.empty((T, 64), dtype=torch.float16)),              # per-row shape
    ]
    for codes, scales in bad:
        with pytest.raises(ValueError):
            p(X, out=(codes, scales))
    p.per_row = True  # a per-row plan wants T x n1 scales
    with pytest.raises(ValueError):
        p(X, out=(good_c, good_s))
