// Internal declarations shared by the libkq translation units (host API + kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq.h"

// Kernel families a plan can dispatch to.
enum kq_kernel_kind {
  KQ_KIND_FUSED_MFMA = 0,  // bf16 X/P, two chained bf16 MFMA contractions, fused epilogue
  KQ_KIND_GENERIC = 1,     // any supported dtype/shape, fp32 FMA contractions
};

struct kq_plan;

// Launches one kq_transform_quant on a plan of the matching variant. Arguments are
// already validated by the host API.
typedef hipError_t (*kq_launch_fn)(const kq_plan *p, const void *X, int64_t T, int64_t ldx,
                                   uint8_t *codes, void *scales, float *y_debug,
                                   hipStream_t stream);

struct kq_plan {
  int n1, n2, n;
  kq_dtype x_dtype;
  kq_dtype scale_dtype;
  float clip;           // exact fp32 clip ratio
  int device;
  int kind;             // kq_kernel_kind
  const char *kname;    // static kernel variant name
  kq_launch_fn launch;
  int grid_cap;         // persistent-grid size (workgroups) for this device
  // fused MFMA variant: operand-ordered bf16 factor copies (see kq_fused.hip)
  void *p2op;
  void *p1op;
  // generic variant: fp32 row-major factor copies
  float *p1f;
  float *p2f;
  // per-channel scale (fp32, n) or nullptr
  float *c;
  // small-batch variant of the fused family, used when T < small_max_T: it spreads each
  // token over more waves (a different P2 operand layout, hence its own copy)
  kq_launch_fn small_launch;
  const char *small_kname;
  void *small_p2op;
  int small_grid_cap;
  int64_t small_max_T;
  // 1: identity left factor and one step per row of V (T * n1 scales)
  int per_row;
  int bits;             // code width: 4 or 8
};

// ---- fused MFMA family (kq_fused.hip) ----
// Work splits of the fused family: 1 or 2 waves per token with the token in registers
// ("deep": one wave per token and per SIMD, next token prefetched into registers), the
// column kernel (n2/32 waves per token, token staged in LDS), or the stream kernel (one
// wave per token, next token prefetched into an LDS slot by DMA).
enum { KQ_SPLIT_REG1 = 1, KQ_SPLIT_REG2 = 2, KQ_SPLIT_COLS = 3, KQ_SPLIT_DEEP = 4,
       KQ_SPLIT_STREAM = 5, KQ_SPLIT_PAIR = 6, KQ_SPLIT_ROWS = 7 };

struct kq_fused_variant {
  int n1, n2;
  bool has_c;
  int split;      // KQ_SPLIT_*
  int bits;       // code width: 4 (INT4, two per byte) or 8 (INT8)
  int p2_block;   // output columns per P2 operand block (kq_fused_arrange_p2)
  int threads;    // workgroup size
  kq_launch_fn launch;
  const void *kernel_symbol;
  const char *name;
};

// The variant for (n1, n2, has_c) with the given split (0: the default one) and code width,
// or nullptr.
const kq_fused_variant *kq_fused_lookup(int n1, int n2, bool has_c, int split, int bits = 4);
// The rows kernel (identity left factor, one step per row of V) for n2, or nullptr.
const kq_fused_variant *kq_fused_lookup_rows(int n2, int bits);
void kq_fused_arrange_p2_rows(const uint16_t *P2, int n2, uint16_t *out);
// Element counts of the operand-ordered bf16 copies of P1 / P2.
size_t kq_fused_p1op_elems(int n1);
size_t kq_fused_p2op_elems(int n2);
// Re-lay a row-major P1 (n1 x n1) / P2 (n2 x n2), given as bf16 bit patterns, into the
// order in which the fused kernels' lanes consume them as MFMA B operands.
void kq_fused_arrange_p1(const uint16_t *P1, int n1, uint16_t *out);
void kq_fused_arrange_p2(const uint16_t *P2, int n2, int cb, uint16_t *out);

// ---- generic family (kq_generic.hip) ----
kq_launch_fn kq_generic_launcher(const char **name, const void **kernel_symbol);
size_t kq_generic_lds_bytes(int n);
int kq_generic_threads();
int kq_generic_max_n();
