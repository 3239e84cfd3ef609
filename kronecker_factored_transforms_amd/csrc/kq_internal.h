// Internal declarations shared by the libkq translation units (host API + kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq.h"

// Kernel families a plan can dispatch to.
enum kq_kernel_kind {
  KQ_KIND_FUSED_MFMA = 0,  // bf16 X/P, two chained bf16 MFMA contractions, fused epilogue
  KQ_KIND_GENERIC = 1,     // any supported dtype/shape, fp32 FMA contractions
  KQ_KIND_FUSED_F32 = 2,   // fp32 X/P on bf16 MFMA (hi/lo operand pairs, three products)
};

struct kq_plan;

// Launches one kq_transform_quant on a plan of the matching variant. Arguments are
// already validated by the host API.
// `ws` is the call's device workspace (at least kq_ws_bytes(p, T) bytes, 256-byte aligned),
// or nullptr for the single-kernel designs, which need none.
typedef hipError_t (*kq_launch_fn)(const kq_plan *p, const void *X, int64_t T, int64_t ldx,
                                   uint8_t *codes, void *scales, float *y_debug, void *ws,
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
  int grid_cap2;        // the same for the second kernel of a two-kernel design
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
  int p1_exp;           // fp16 operands (variants with f16_ops): P1 * 2^-p1_exp and
  int p2_exp;           // P2 * 2^-p2_exp
  float c_absmax;       // max |c| (the bound of a token's x c, with max |x|)
  int c_f16;            // 1: every nonzero |c| lies in [2^-14, 2^15), so fp16(c) is a normal
                        // fp16 value (the column kernel with c may hold c in registers as fp16)
  // device workspace of the two-kernel designs for large factors: region A holds
  // ws_a_per_token bytes per token, region B (at a 256-byte aligned offset after A) holds
  // ws_b_per_token bytes per token; both 0 for the single-kernel designs
  size_t ws_a_per_token;
  size_t ws_b_per_token;
};

// Workspace of a call of T tokens: total bytes, and the offset of region B.
inline size_t kq_ws_offset_b(const kq_plan *p, int64_t T) {
  return ((size_t)T * p->ws_a_per_token + 255) / 256 * 256;
}
inline size_t kq_ws_bytes(const kq_plan *p, int64_t T) {
  if (!p->ws_a_per_token && !p->ws_b_per_token) return 0;
  return kq_ws_offset_b(p, T) + ((size_t)T * p->ws_b_per_token + 255) / 256 * 256;
}

// ---- fused MFMA family (kq_fused.hip) ----
// Work splits of the fused family: 1 or 2 waves per token with the token in registers
// ("deep": one wave per token and per SIMD, next token prefetched into registers), the
// column kernel (n2/32 waves per token, token staged in LDS), or the stream kernel (one
// wave per token, next token prefetched into an LDS slot by DMA).
// The two-kernel designs for large factors (kq_large.hip): Figure 8(c) (stage 1 writes Z
// to the workspace, stage 2 + quantizer reads it) and Figure 8(b) (P1 in tiles of its
// output dimension, Y through the workspace, a second kernel quantizes).
enum { KQ_SPLIT_REG1 = 1, KQ_SPLIT_REG2 = 2, KQ_SPLIT_COLS = 3, KQ_SPLIT_DEEP = 4,
       KQ_SPLIT_STREAM = 5, KQ_SPLIT_PAIR = 6, KQ_SPLIT_ROWS = 7, KQ_SPLIT_TWOSTAGE = 8,
       KQ_SPLIT_PTILE = 9, KQ_SPLIT_RSPLIT = 10 };

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
  // two-kernel designs only: the second kernel (for its occupancy) and the workspace
  const void *kernel_symbol2;
  int threads2;
  size_t ws_a_per_token;
  size_t ws_b_per_token;
  // both contractions on fp16 operands: the plan stores P1's and P2's operands as fp16
  // (scaled by 2^-p1_exp and 2^-p2_exp)
  bool f16_ops;
  // stage 1 only on fp16 operands (the two-kernel design of Figure 8(c) with a per-channel
  // scale): the plan stores P2's operands as fp16 (scaled by 2^-p2_exp), P1's as bf16
  bool f16_p2;
};

// The variant for (n1, n2, has_c) with the given split (0: the default one) and code width,
// or nullptr.
const kq_fused_variant *kq_fused_lookup(int n1, int n2, bool has_c, int split, int bits = 4);
// The two-kernel designs for large factors (kq_large.hip): the variant for (n1, n2,
// has_c) with split KQ_SPLIT_TWOSTAGE / KQ_SPLIT_PTILE (0: the shape's default), or nullptr.
const kq_fused_variant *kq_large_lookup(int n1, int n2, bool has_c, int split, int bits);
// The fp32 kernel (kq_f32.hip: fp32 values as bf16 hi/lo pairs on the bf16 MFMA) for
// (n1, n2, has_c), or nullptr. Its plan holds P2's and P1's operands twice, hi then lo.
const kq_fused_variant *kq_f32_lookup(int n1, int n2, bool has_c);
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

// ---- host-side debug log (kq_api.hip) ----
// KQ_LOG set to anything but "" or "0" in the environment: one line per plan, call and
// error on stderr, prefixed "[kq]". Read once; host code only.
bool kq_log_on();
void kq_logf(const char *fmt, ...) __attribute__((format(printf, 1, 2)));
