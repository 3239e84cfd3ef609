/*
 * kq.h -- C ABI of libkq: fused Kronecker-factored activation transform + per-token
 * symmetric INT4 quantization on AMD Instinct MI355X (gfx950).
 *
 * What one call computes, per token t (x_t = row t of X, n = n1*n2):
 *   1. x^_t = x_t * c                       (optional per-channel scale)
 *   2. V_t[i][k] = x^_t[i*n2 + k]           (row-major n1 x n2 view)
 *   3. Y_t = P1^T V_t P2  ==  x^_t (P1 (x) P2)
 *   4. a_t = max |Y_t|;  s32 = fp32(fp32(clip * a_t) / 7);  s_t = fp16_rne(s32) (or s32)
 *   5. q = clamp(rint(fp32(y * fp32(1/s_t))), -8, 7); s_t == 0 -> q = 0
 *   6. codes: element 2m in the low nibble of byte m, 2m+1 in the high nibble,
 *      4-bit two's complement, row-major Y order (index j*n2 + l).
 * Sources (web pages): "Kronecker Product" -- Definition (entry formula of A (x) B) and
 * Why It Matters for LLM Quantization (vec(V)(P1 (x) P2) = vec(P1^T V P2)); "FlatQuant:
 * Fast Learnable Affine Quantization" -- Symbol Map (X~ as k x n1 x n2, diag(c),
 * sigmoid-mapped clip alpha_a, Q(.) with step s), Deep Dive: Kronecker factorization
 * (P1^T x1 X~ x2 P2), Per-channel scaling and learnable clipping (c before the
 * transform, clip after it), The fused kernel / Figure 8a (P1, P2 resident on chip,
 * only the quantized tile written), Putting It Together step 3; "High-Rate Quantized
 * Matrix Multiplication I" -- absmax INT scaling.
 *
 * Conventions common to all calls
 *   - Device pointers are HIP device addresses on the current device. The library
 *     never frees caller memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the legacy default stream).
 *   - Every entry point returns a kq_status; nothing is thrown or printed across the
 *     ABI. Argument errors are detected before anything is enqueued.
 *   - A plan is immutable after kq_create: calls on one plan from several host threads
 *     or streams are safe. It belongs to the device that was current at kq_create, and
 *     kq_transform_quant returns KQ_ERR_INVALID_ARG when another device is current.
 *   - Debug log: with KQ_LOG set in the environment (to anything but "" or "0"), every
 *     plan creation (the kernel variant, grid, small-batch variant and workspace it
 *     chose), every call and every error prints one line on stderr, prefixed "[kq]".
 *     Host side only; the variable is read once per process.
 */
#ifndef KQ_H
#define KQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kq_plan kq_plan;

/* The enumerations are int-sized in C. Compiled as C++ (the library itself), they get int
 * as their fixed underlying type, so that any int a C caller passes (say, an unknown
 * status or dtype) is a valid value there too and is rejected by the checks rather than
 * being undefined. */
#ifdef __cplusplus
#define KQ_ENUM_INT : int
#else
#define KQ_ENUM_INT
#endif

typedef enum kq_status KQ_ENUM_INT {
  KQ_OK = 0,
  KQ_ERR_INVALID_ARG = 1,   /* bad size, NULL pointer, NaN alpha, ...          */
  KQ_ERR_UNSUPPORTED = 2,   /* valid, but the library has no kernel for it    */
  KQ_ERR_ALIGNMENT = 3,     /* a pointer or leading dimension is misaligned   */
  KQ_ERR_OUT_OF_MEMORY = 4, /* host or device allocation failed (kq_create)   */
  KQ_ERR_HIP = 5,           /* a HIP runtime call or kernel launch failed      */
  KQ_ERR_WORKSPACE = 6      /* the call needs a device workspace larger than   */
                            /* the one given (see kq_workspace_size)           */
} kq_status;

typedef enum kq_dtype KQ_ENUM_INT { KQ_BF16 = 0, KQ_FP32 = 1, KQ_FP16 = 2 } kq_dtype;

/* Flags for kq_create_ex. At most one KQ_FLAG_SPLIT_* may be given, only for bf16 plans
 * (KQ_ERR_UNSUPPORTED when that split is not built for the shape). All variants compute
 * Y within the plan dtype's tolerance of the exact transform (their operand roundings
 * differ where a per-channel scale is given, and their fp32 accumulation order always) and
 * quantize the Y they computed the same way. */
#define KQ_FLAG_FORCE_GENERIC 0x1u  /* fp32 FMA kernel even where an MFMA one applies   */
#define KQ_FLAG_SPLIT_REG1 0x10u    /* MFMA: one wave per token, token in registers     */
#define KQ_FLAG_SPLIT_REG2 0x20u    /* MFMA: two waves per token, token in registers    */
#define KQ_FLAG_SPLIT_COLS 0x40u    /* MFMA: n2/32 waves per token, token staged in LDS */
#define KQ_FLAG_SPLIT_DEEP 0x80u    /* MFMA: one wave per token and SIMD, next token     */
                                    /* prefetched into registers                          */
#define KQ_FLAG_SPLIT_STREAM 0x100u /* MFMA: one wave per token, next token prefetched   */
                                    /* into LDS by DMA (per-channel scale: n2 = 64 only)  */
#define KQ_FLAG_SPLIT_PAIR 0x200u   /* MFMA: two waves per token (one column half each),  */
                                    /* operands in registers, tokens double-buffered in   */
                                    /* LDS by DMA (no per-channel scale)                  */
/* The two designs for factors too large for one CU's on-chip memory ("FlatQuant" page,
 * Deep Dive: The fused kernel, Figure 8(b) and 8(c); Where It Breaks: on-chip memory
 * overflow). Both pass an intermediate through a device workspace that the caller gives
 * to kq_transform_quant_ws (kq_workspace_size says how large). */
#define KQ_FLAG_SPLIT_TWOSTAGE 0x1000u /* Figure 8(c): stage 1 (x c) P2 writes Z (bf16) to    */
                                       /* the workspace; stage 2 P1^T Z + quantization      */
                                       /* reads it back                                     */
#define KQ_FLAG_SPLIT_PTILE 0x2000u    /* Figure 8(b): Z stays on chip, P1 is applied one    */
                                       /* tile of its output (non-reduction) dimension at a */
                                       /* time, each tile of Y goes to the workspace (fp32) */
                                       /* with the token's absmax, and a second kernel      */
                                       /* quantizes it                                      */
#define KQ_FLAG_SPLIT_RSPLIT 0x4000u   /* MFMA, with a per-channel scale, n2 = 64, INT4: a   */
                                       /* token's 16-row blocks on n1/16 waves, Z passed    */
                                       /* between them through LDS (the small-batch split   */
                                       /* of those plans)                                   */

/* KQ_FLAG_PER_ROW: the left factor is the identity (pass P1 = NULL) and every row of V
 * (n2 values, e.g. one attention head of a token) gets its own step, so `scales` holds
 * T * n1 values (row i of token t at t * n1 + i) and codes keep the row-major Y order.
 * This is the per-head key/value transform ahead of a quantized KV cache ("FlatQuant"
 * page, Symbol Map: P_h, P_v; Transformer integration). bf16 only, n2 in {64, 128}, any
 * 1 <= n1 <= 2^20, no c, no other flag but KQ_FLAG_INT8 (KQ_ERR_INVALID_ARG /
 * KQ_ERR_UNSUPPORTED otherwise);
 * a call must have T * n1 < 2^31 rows (else KQ_ERR_UNSUPPORTED). */
#define KQ_FLAG_PER_ROW 0x400u

/* KQ_FLAG_INT8: INT8 codes instead of INT4 ("FlatQuant" page, How we know: beyond dense
 * W4A4 -- mixed precision, where some layers run at W8A8): step
 * s32 = fp32(fp32(clip * a) / 127), q = clamp(rint(fp32(y * inv)), -128, 127), one
 * two's-complement byte per value, so `codes` holds T x n bytes (row stride n). bf16
 * plans of the stream kernel's shapes: n2 in {64, 128} with n1 in {16, 32, 48, 64},
 * without c, or n2 = 64 with c; of the column kernel's shapes: n2 = 128 with n1 in {80,
 * 86, 96, 108, 112, 128}, with or without c, 64 x 128 with c, n1 = 128 with n2 in {144,
 * 160, 192, 224, 256} without c, and 32 x 48, 40 x 64, 56 x 64, 64 x 80, 64 x 88,
 * 64 x 96, 64 x 104, 64 x 112, 80 x 112 with or without c; and per-row plans
 * (KQ_FLAG_PER_ROW, one step per row of n2 values) with n2 in {64, 128}
 * (KQ_ERR_UNSUPPORTED otherwise, including the two-kernel designs and the fp32 MFMA
 * kernel); not with KQ_FLAG_FORCE_GENERIC. */
#define KQ_FLAG_INT8 0x800u

/*
 * kq_choose_factors -- factor a hidden size for the Kronecker transform.
 * Picks n1 <= n2 with n1*n2 == n minimising n1 + n2 ("FlatQuant" page, Deep Dive:
 * Kronecker factorization: the factor sizes minimise n1 + n2, e.g. 8192 -> (64, 128)).
 * n >= 1; writes *n1, *n2. Returns KQ_ERR_INVALID_ARG for n < 1 or NULL outputs.
 */
kq_status kq_choose_factors(int64_t n, int *n1, int *n2);

/*
 * kq_create -- build an immutable plan for one (P1, P2, c, alpha) set.
 *   out          receives the plan (set to NULL on error).
 *   n1, n2       factor sizes, n = n1*n2 must be even. n1, n2 >= 1.
 *   x_dtype      dtype of X, P1 and P2: KQ_BF16 or KQ_FP32 (P has the dtype of X).
 *   scale_dtype  KQ_FP16 (default in the bindings) or KQ_FP32 for the per-token scale.
 *   P1           device, n1 x n1 row-major, x_dtype ("left" factor, enters transposed);
 *                NULL (identity) exactly when KQ_FLAG_PER_ROW is given.
 *   P2           device, n2 x n2 row-major, x_dtype.
 *   c            device, n fp32 per-channel scale applied before the transform, or NULL
 *                (all ones).
 *   alpha        clip logit; clip = fp32(1 / (1 + exp(-alpha))) in double on the host.
 *                +INFINITY gives clip 1, -INFINITY gives clip 0. NaN -> INVALID_ARG.
 *   stream       stream used for the set-up copies. kq_create synchronizes it.
 * The plan owns device copies of P1, P2 (re-laid-out for the kernels) and c; the caller
 * may free its buffers when kq_create returns. Not a hot-path call: it allocates.
 * Errors: INVALID_ARG (sizes, NULLs, dtypes, NaN alpha), OUT_OF_MEMORY, HIP.
 */
kq_status kq_create(kq_plan **out, int n1, int n2, kq_dtype x_dtype, kq_dtype scale_dtype,
                    const void *P1, const void *P2, const float *c, float alpha,
                    void *stream);

/* Shapes with a kernel (anything else: KQ_ERR_UNSUPPORTED from kq_create):
 *   bf16 on the single-kernel MFMA designs ("FlatQuant" page, Deep Dive: The fused kernel,
 *     Figure 8(a)), with or without c: n2 = 32 with n1 in {16, 32}; n2 = 64 with n1 in
 *     {16, 32, 40, 48, 56, 64}; n2 = 128 with n1 in {16, 32, 48, 64, 80, 86, 96, 108, 112,
 *     128}; and 32 x 48, 64 x 80, 64 x 88, 64 x 96, 64 x 104, 64 x 112, 80 x 112. Factors
 *     that are not whole MFMA tiles are zero-padded inside the plan (results unchanged).
 *     Without c also n1 = 128 with n2 in {144, 160, 192, 224, 256}.
 *   bf16 on the two-kernel designs for factors beyond one CU's on-chip memory (Figure 8(b)
 *     and 8(c); these need a workspace, see kq_workspace_size): 160 x 160, 144 x 192,
 *     168 x 176, 208 x 256 and 256 x 256 with or without c, and 128 x n2 with c for n2 in
 *     {160, 192, 224, 256}.
 *   fp32 on the MFMA kernel (each value as a bf16 hi + lo pair, three products, Z in
 *     fp32): n2 = 64 with n1 in {16, 32, 48, 64}, without c.
 *   Every other fp32 shape, and bf16 shapes not listed above: the generic fp32 kernel,
 *     n <= 16384.
 */

/* kq_create with flags (KQ_FLAG_*); kq_create(...) == kq_create_ex(..., 0). */
kq_status kq_create_ex(kq_plan **out, int n1, int n2, kq_dtype x_dtype,
                       kq_dtype scale_dtype, const void *P1, const void *P2,
                       const float *c, float alpha, void *stream, unsigned flags);

/*
 * kq_transform_quant -- the hot path: transform + quantize T tokens, enqueued on
 * `stream`, asynchronous. No allocation, no synchronization, no host<->device copy, so a
 * call may be captured into a HIP graph and replayed (the buffers stay bound).
 *   plan     from kq_create.
 *   X        device, T rows of n elements of the plan's x_dtype; row t starts at
 *            X + t*ldx elements. 16-byte aligned; ldx >= n and ldx*sizeof(elem) a
 *            multiple of 16 bytes (else KQ_ERR_ALIGNMENT).
 *   T        number of tokens, >= 0. T == 0 returns KQ_OK and launches nothing.
 *   ldx      leading dimension of X in elements.
 *   codes    device, T x (n/2) bytes, row stride n/2, 16-byte aligned (written); T x n
 *            bytes, row stride n, for a KQ_FLAG_INT8 plan.
 *   scales   device, T scales of the plan's scale_dtype (written); T * n1 of them for a
 *            KQ_FLAG_PER_ROW plan.
 *   y_debug  device, T x n fp32, or NULL. When given, receives the exact fp32 Y that
 *            was quantized (for verification; adds 4n bytes of writes per token).
 * Caller owns X, codes, scales and y_debug. Outputs are written in full for every
 * token; inputs are not modified. Non-finite inputs give unspecified codes.
 * Errors: INVALID_ARG (NULL plan/pointers with T > 0, T < 0, ldx < n), ALIGNMENT,
 * HIP (launch failure; checked with hipGetLastError right after the launch).
 */
kq_status kq_transform_quant(const kq_plan *plan, const void *X, int64_t T, int64_t ldx,
                             uint8_t *codes, void *scales, float *y_debug, void *stream);

/*
 * kq_workspace_size -- device workspace (bytes) that a call of T tokens on `plan` needs:
 * 0 for the single-kernel designs; for the two-kernel designs (KQ_FLAG_SPLIT_TWOSTAGE,
 * KQ_FLAG_SPLIT_PTILE, and the plans of large factors that default to one of them) the
 * intermediate the two kernels pass through global memory. Writes *bytes. Errors:
 * INVALID_ARG (NULL plan or bytes, T < 0, T beyond 2^40 / n).
 */
kq_status kq_workspace_size(const kq_plan *plan, int64_t T, size_t *bytes);

/*
 * kq_transform_quant_ws -- kq_transform_quant with a caller-owned device workspace.
 *   workspace        device, at least kq_workspace_size(plan, T) bytes, 256-byte aligned;
 *                    may be NULL (with workspace_bytes 0) when that size is 0. Its contents
 *                    on entry do not matter; the call overwrites them. Calls that share a
 *                    workspace must be ordered (same stream), or they race on it.
 *   workspace_bytes  its size in bytes.
 * Everything else as kq_transform_quant, which is this call with (NULL, 0).
 * Errors: as kq_transform_quant, plus WORKSPACE (workspace missing or smaller than
 * needed) and ALIGNMENT (workspace not 256-byte aligned).
 */
kq_status kq_transform_quant_ws(const kq_plan *plan, const void *X, int64_t T, int64_t ldx,
                                uint8_t *codes, void *scales, float *y_debug, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * kq_transform_quant_noalloc -- kq_transform_quant_ws for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the workspace of the two-kernel designs comes from a scratch array inside
 * the library, KQ_NOALLOC_SCRATCH_BYTES per GPU, held from the library's load until the
 * process ends. The call itself allocates nothing. Arguments as kq_transform_quant.
 * Every call of this entry point on one GPU shares that GPU's scratch: calls that may
 * overlap on a GPU (different streams, or host threads without ordering) race on it and
 * must be ordered by the caller. Plans of the single-kernel designs need no workspace and
 * take any T. Errors: as kq_transform_quant_ws, with WORKSPACE when the call needs more
 * than KQ_NOALLOC_SCRATCH_BYTES (kq_workspace_size(plan, T) says how much), UNSUPPORTED
 * for a device ordinal of 64 or more.
 */
#define KQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
kq_status kq_transform_quant_noalloc(const kq_plan *plan, const void *X, int64_t T, int64_t ldx,
                                     uint8_t *codes, void *scales, float *y_debug, void *stream);

/*
 * kq_int4_gemm -- the INT4 x INT4 consumer of two kq_transform_quant outputs, on the int8
 * matrix cores ("FlatQuant" page, Putting It Together: the quantized activations feed an
 * INT4 GEMM; "High-Rate Quantized Matrix Multiplication I", Technical Summary: product of
 * two absmax-quantized matrices):
 *     out[t][j] = cvt( fp32( fp32( fp32(acc[t][j]) * sx[t] ) * sw[j] ) ),
 *     acc[t][j] = sum_k qx[t][k] * qw[j][k]  (exact, integer),
 * cvt = identity for KQ_FP32 output, round-to-nearest-even for KQ_BF16 / KQ_FP16.
 * The weight side is W's rows run through kq_transform_quant with the factors P1^-T and
 * P2^-T ((X P)(P^-1 W^T) = X W^T, "FlatQuant" page, Learning the affine transformation),
 * which for orthogonal factors are P1 and P2 themselves.
 *   xq     device, T rows of K/2 code bytes, row stride ldxq bytes (as kq_transform_quant
 *          writes them: ldxq = K/2), 16-byte aligned, ldxq a multiple of 16.
 *   sx     device, T per-token steps of scale_dtype (KQ_FP16 or KQ_FP32).
 *   wq     device, N rows of K/2 code bytes, row stride ldwq bytes, same rules as xq.
 *   sw     device, N per-row steps of scale_dtype (fp32: 16-byte aligned).
 *   K      codes per row: a multiple of 256, at most 65536 (the int32 accumulator range).
 *   N      a multiple of 4.
 *   out    device, T rows of N values of out_dtype (KQ_FP32, KQ_BF16, KQ_FP16), row stride
 *          ldo elements; out and each row start aligned to 4 elements.
 * T == 0 or N == 0 returns KQ_OK and launches nothing. Asynchronous on `stream`; no
 * allocation. Errors: INVALID_ARG (NULLs, negative sizes, strides too small, dtypes),
 * UNSUPPORTED (K or N not as above; T*ldxq or N*ldwq >= 4 GiB), ALIGNMENT, HIP.
 */
kq_status kq_int4_gemm(const uint8_t *xq, int64_t ldxq, const void *sx, int64_t T,
                       const uint8_t *wq, int64_t ldwq, const void *sw, int64_t N, int64_t K,
                       kq_dtype scale_dtype, kq_dtype out_dtype, void *out, int64_t ldo,
                       void *stream);

/*
 * kq_weight_factor -- the weight-side factor (P^-1)^T of one activation factor P, for the
 * weight rows of a W4A4 layer. The layer computes (X P)(P^-1 W^T) ("FlatQuant" page,
 * Learning the affine transformation); with P = P1 (x) P2 ("Kronecker Product" page: the
 * inverse and the transpose of a Kronecker product are the Kronecker products of the
 * factors' inverses and transposes), row j of W P^-T is w_j ((P1^-1)^T (x) (P2^-1)^T), so
 * kq_create with the factors kq_weight_factor(P1) and kq_weight_factor(P2), no c and clip
 * logit +INFINITY, quantizes W's rows for kq_int4_gemm. (A per-channel scale c of the
 * activations would be divided out of W's columns before that; the pages merge it into the
 * preceding weight instead.)
 *   P      device, m x m row-major, dtype KQ_BF16 or KQ_FP32 (aligned to its element).
 *   out    device, m x m row-major, same dtype; may be P itself.
 *   m      1 .. 1024.
 * Computed on the GPU in fp64 (Gauss-Jordan elimination with partial pivoting on
 * [P^T | I]) and rounded once, to nearest even, to dtype. A plan-time call like kq_create:
 * it allocates a 16 m^2-byte device workspace and frees it, and it synchronizes `stream`.
 * Errors: INVALID_ARG (NULL, m out of range, dtype, or P singular: a zero pivot),
 * ALIGNMENT, OUT_OF_MEMORY, HIP.
 */
kq_status kq_weight_factor(const void *P, int m, kq_dtype dtype, void *out, void *stream);

/* Free a plan and its device buffers. NULL is a no-op (returns KQ_OK). The caller must
 * make sure no enqueued kq_transform_quant on this plan is still running. */
kq_status kq_destroy(kq_plan *plan);

/* The exact fp32 clip ratio the kernels use (0 for a NULL plan). */
float kq_plan_clip_ratio(const kq_plan *plan);

/* Name of the kernel variant the plan dispatches to for large batches (static string;
 * "" for NULL). */
const char *kq_plan_kernel_name(const kq_plan *plan);

/* Name of the kernel variant a kq_transform_quant of T tokens runs on this plan. A plan
 * created without a KQ_FLAG_SPLIT_* flag may use a second work split for small batches
 * (fewer than about four tokens per compute unit), which spreads each token over more
 * waves; both compute the same Y and codes. "" for NULL. */
const char *kq_plan_kernel_name_for(const kq_plan *plan, int64_t T);

/* Static, human-readable description of a status code. */
const char *kq_status_string(kq_status s);

/* ABI version of this header (major * 10000 + minor * 100 + patch). */
int kq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KQ_H */
