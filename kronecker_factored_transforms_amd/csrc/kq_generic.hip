// Generic Kronecker transform + per-token INT4 quantization with fp32 FMA contractions.
//
// Used for fp32 inputs and for factor shapes the bf16 MFMA kernel does not cover. One
// workgroup handles one token at a time (grid-stride over tokens): the scaled token and
// the intermediate Z = V P2 live in LDS as fp32, then Y = P1^T Z, the absmax, and the
// same quantizer as the fused kernel ("FlatQuant: Fast Learnable Affine Quantization",
// Deep Dive: Kronecker factorization; Per-channel scaling and learnable clipping).
// Every dot product is a sequential fp32 FMA chain in index order, so results are
// deterministic for a given input.

#include "kq_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxN = 16384;  // LDS: two fp32 tiles of n values

__device__ __forceinline__ float load_elem(const void *X, int is_bf16, int64_t idx) {
  if (is_bf16) {
    const uint16_t b = static_cast<const uint16_t *>(X)[idx];
    return __uint_as_float((uint32_t)b << 16);
  }
  return static_cast<const float *>(X)[idx];
}

// Workgroup barrier ordering LDS only (no wait for in-flight global loads).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ uint32_t quant_nibble(float y, float inv) {
  float v = __fmul_rn(y, inv);
  v = rintf(v);
  v = fminf(fmaxf(v, -8.0f), 7.0f);
  return (uint32_t)((int)v) & 0xFu;
}

__global__ __launch_bounds__(kThreads) void kq_generic_kernel(
    const void *__restrict__ X, int x_is_bf16, int64_t T, int64_t ldx, int n1, int n2,
    const float *__restrict__ P1, const float *__restrict__ P2, const float *__restrict__ cvec,
    float clip, int scale_fp16, uint8_t *__restrict__ codes, void *__restrict__ scales,
    float *__restrict__ ydbg) {
  extern __shared__ float smem[];
  const int n = n1 * n2;
  float *V = smem;         // scaled token, then Y
  float *Z = smem + n;     // V P2
  __shared__ float s_red[kThreads / 64];
  const int tid = threadIdx.x;

  for (int64_t tok = blockIdx.x; tok < T; tok += gridDim.x) {
    for (int e = tid; e < n; e += kThreads) {
      float x = load_elem(X, x_is_bf16, tok * ldx + e);
      if (cvec != nullptr) x = __fmul_rn(x, cvec[e]);
      V[e] = x;
    }
    lds_barrier();
    // Z[i][l] = sum_k V[i][k] P2[k][l]
    for (int e = tid; e < n; e += kThreads) {
      const int i = e / n2, l = e % n2;
      float acc = 0.f;
      for (int k = 0; k < n2; ++k) acc = fmaf(V[i * n2 + k], P2[(size_t)k * n2 + l], acc);
      Z[e] = acc;
    }
    lds_barrier();
    // Y[j][l] = sum_i P1[i][j] Z[i][l]
    float m = 0.f;
    for (int e = tid; e < n; e += kThreads) {
      const int j = e / n2, l = e % n2;
      float acc = 0.f;
      for (int i = 0; i < n1; ++i) acc = fmaf(P1[(size_t)i * n1 + j], Z[i * n2 + l], acc);
      V[e] = acc;
      m = fmaxf(m, fabsf(acc));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if ((tid & 63) == 0) s_red[tid >> 6] = m;
    lds_barrier();
    float amax = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) amax = fmaxf(amax, s_red[w]);

    float s32 = __fdiv_rn(__fmul_rn(clip, amax), 7.0f);
    const _Float16 s16 = (_Float16)s32;
    const float sf = scale_fp16 ? (float)s16 : s32;
    float inv = (sf == 0.f) ? 0.f : __fdiv_rn(1.0f, sf);
    if (__builtin_isinf(inv)) {  // fp32 step <= 2^-128: stored as 0, codes 0 (underflow)
      s32 = 0.f;
      inv = 0.f;
    }

    uint8_t *crow = codes + tok * (int64_t)(n / 2);
    for (int mm = tid; mm < n / 2; mm += kThreads) {
      const float y0 = V[2 * mm], y1 = V[2 * mm + 1];
      crow[mm] = (uint8_t)(quant_nibble(y0, inv) | (quant_nibble(y1, inv) << 4));
      if (ydbg != nullptr) {
        ydbg[tok * (int64_t)n + 2 * mm] = y0;
        ydbg[tok * (int64_t)n + 2 * mm + 1] = y1;
      }
    }
    if (tid == 0) {
      if (scale_fp16) static_cast<_Float16 *>(scales)[tok] = s16;
      else static_cast<float *>(scales)[tok] = s32;
    }
    lds_barrier();
  }
}

hipError_t launch_generic(const kq_plan *p, const void *X, int64_t T, int64_t ldx, uint8_t *codes,
                          void *scales, float *y_debug, void *ws, hipStream_t stream) {
  const int grid = (int)(T < (int64_t)p->grid_cap ? T : (int64_t)p->grid_cap);
  const size_t lds = kq_generic_lds_bytes(p->n);
  hipLaunchKernelGGL(kq_generic_kernel, dim3(grid), dim3(kThreads), lds, stream, X,
                     p->x_dtype == KQ_BF16 ? 1 : 0, T, ldx, p->n1, p->n2, p->p1f, p->p2f, p->c,
                     p->clip, p->scale_dtype == KQ_FP16 ? 1 : 0, codes, scales, y_debug);
  return hipGetLastError();
}

}  // namespace

kq_launch_fn kq_generic_launcher(const char **name, const void **kernel_symbol) {
  if (name) *name = "generic_fp32_fma";
  if (kernel_symbol) *kernel_symbol = reinterpret_cast<const void *>(&kq_generic_kernel);
  return &launch_generic;
}

size_t kq_generic_lds_bytes(int n) { return (size_t)2 * (size_t)n * sizeof(float); }
int kq_generic_threads() { return kThreads; }
int kq_generic_max_n() { return kMaxN; }
