// kq_weight.hip -- the weight-side factor of a W4A4 linear layer, computed on the GPU.
//
// A linear layer X W^T with the activation transform P = P1 (x) P2 computes
// (X P)(P^-1 W^T) ("FlatQuant: Fast Learnable Affine Quantization", Learning the affine
// transformation). By the Kronecker product's inverse and transpose rules ("Kronecker
// Product", Definition and its properties: (A (x) B)^-1 = A^-1 (x) B^-1, (A (x) B)^T =
// A^T (x) B^T), row j of (P^-1 W^T)^T = W P^-T is w_j (P1^-T (x) P2^-T): the weight rows go
// through the same transform as tokens, with the factors (P1^-1)^T and (P2^-1)^T. This file
// forms one such factor, (P^-1)^T = (P^T)^-1, for an m x m factor P. It runs once per layer,
// offline, so it favours exactness over speed: one workgroup, fp64 Gauss-Jordan elimination
// with partial pivoting on [P^T | I], then one rounding of the right half to the factor's
// dtype.
#include "kq_internal.h"

#include <hip/hip_runtime.h>

namespace {

constexpr int kWThreads = 1024;
constexpr int kMaxM = 1024;

__device__ __forceinline__ double load_factor(const void *P, int is_bf16, int64_t i) {
  if (is_bf16) return (double)__uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(P)[i] << 16);
  return (double)reinterpret_cast<const float *>(P)[i];
}

// fp64 -> bf16 bits, round to nearest even, as one rounding. The conversion to fp32 rounds
// to nearest first; since every bf16 value and every midpoint between two of them is an
// fp32 value, that rounding can only mislead the second one when it lands exactly on a
// midpoint, and there the sign of the fp64 residual decides (zero residual: a true tie).
__device__ __forceinline__ uint16_t bf16_rne(double x) {
  const float f = (float)x;
  const uint32_t u = __float_as_uint(f);
  const uint32_t hi = u >> 16, low = u & 0xFFFFu;
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)(hi | (low ? 0x40u : 0u));  // inf / NaN
  bool up;
  if (low != 0x8000u) {
    up = low > 0x8000u;
  } else {
    const double r = fabs(x) - fabs((double)f);
    up = r > 0.0 ? true : (r < 0.0 ? false : (hi & 1u) != 0u);
  }
  return (uint16_t)(hi + (up ? 1u : 0u));
}

// A: m x 2m fp64 workspace, row-major. status: 0 done, 1 singular (a zero pivot).
__global__ __launch_bounds__(kWThreads) void kq_weight_factor_kernel(
    const void *__restrict__ P, int m, int is_bf16, double *__restrict__ A,
    void *__restrict__ out, int *__restrict__ status) {
  __shared__ double s_val[kWThreads];
  __shared__ int s_idx[kWThreads];
  __shared__ double s_col[kMaxM];  // column k of every row before step k's elimination
  const int tid = threadIdx.x;
  const int w = 2 * m;

  // [P^T | I]
  for (int64_t e = tid; e < (int64_t)m * w; e += kWThreads) {
    const int r = (int)(e / w), c = (int)(e % w);
    A[e] = c < m ? load_factor(P, is_bf16, (int64_t)c * m + r) : (c - m == r ? 1.0 : 0.0);
  }
  __syncthreads();

  for (int k = 0; k < m; ++k) {
    // pivot: the row r >= k with the largest |A[r][k]|, the first such row on ties
    double best = -1.0;
    int bi = -1;
    for (int r = k + tid; r < m; r += kWThreads) {
      const double v = fabs(A[(int64_t)r * w + k]);
      if (v > best) {
        best = v;
        bi = r;
      }
    }
    s_val[tid] = best;
    s_idx[tid] = bi;
    __syncthreads();
    for (int s = kWThreads / 2; s > 0; s >>= 1) {
      if (tid < s) {
        const double b = s_val[tid + s];
        const int ib = s_idx[tid + s];
        if (b > s_val[tid] || (b == s_val[tid] && ib >= 0 && (s_idx[tid] < 0 || ib < s_idx[tid]))) {
          s_val[tid] = b;
          s_idx[tid] = ib;
        }
      }
      __syncthreads();
    }
    const int p = s_idx[0];
    const double pv = s_val[0];
    if (!(pv > 0.0) || !(pv < __builtin_huge_val())) {  // the same decision in every thread
      if (tid == 0) *status = 1;
      return;
    }
    if (p != k) {
      for (int c = k + tid; c < w; c += kWThreads) {
        const double t = A[(int64_t)k * w + c];
        A[(int64_t)k * w + c] = A[(int64_t)p * w + c];
        A[(int64_t)p * w + c] = t;
      }
    }
    __syncthreads();
    for (int r = tid; r < m; r += kWThreads) s_col[r] = A[(int64_t)r * w + k];
    __syncthreads();
    // row k / pivot; then column k leaves every other row. Columns below k are already zero
    // in row k (exactly: each elimination step subtracts f * 1 from f), so they are skipped.
    const double piv = s_col[k];
    for (int c = k + tid; c < w; c += kWThreads) A[(int64_t)k * w + c] = A[(int64_t)k * w + c] / piv;
    __syncthreads();
    const int wk = w - k;
    for (int64_t e = tid; e < (int64_t)m * wk; e += kWThreads) {
      const int r = (int)(e / wk), c = k + (int)(e % wk);
      if (r != k) A[(int64_t)r * w + c] = fma(-s_col[r], A[(int64_t)k * w + c], A[(int64_t)r * w + c]);
    }
    __syncthreads();
  }

  // the right half, rounded once to the factor's dtype
  for (int64_t e = tid; e < (int64_t)m * m; e += kWThreads) {
    const double v = A[(e / m) * w + m + e % m];
    if (is_bf16) reinterpret_cast<uint16_t *>(out)[e] = bf16_rne(v);
    else reinterpret_cast<float *>(out)[e] = (float)v;
  }
  if (tid == 0) *status = 0;
}

}  // namespace

static kq_status weight_factor_impl(const void *P, int m, kq_dtype dtype, void *out, void *stream) {
  if (!P || !out || m < 1 || m > kMaxM) return KQ_ERR_INVALID_ARG;
  if (dtype != KQ_BF16 && dtype != KQ_FP32) return KQ_ERR_INVALID_ARG;
  const size_t es = dtype == KQ_BF16 ? 2 : 4;
  if ((uintptr_t)P % es != 0 || (uintptr_t)out % es != 0) return KQ_ERR_ALIGNMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t abytes = (size_t)m * 2 * m * sizeof(double);
  void *ws = nullptr;
  if (hipMalloc(&ws, abytes + 256) != hipSuccess) return KQ_ERR_OUT_OF_MEMORY;
  double *A = static_cast<double *>(ws);
  int *dstatus = reinterpret_cast<int *>(static_cast<char *>(ws) + abytes);
  int hstatus = -1;
  kq_status st = KQ_OK;
  hipLaunchKernelGGL(kq_weight_factor_kernel, dim3(1), dim3(kWThreads), 0, s, P, m,
                     dtype == KQ_BF16 ? 1 : 0, A, out, dstatus);
  if (hipGetLastError() != hipSuccess ||
      hipMemcpyAsync(&hstatus, dstatus, sizeof(int), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    st = KQ_ERR_HIP;
  else if (hstatus != 0)
    st = KQ_ERR_INVALID_ARG;  // singular P
  if (hipFree(ws) != hipSuccess && st == KQ_OK) st = KQ_ERR_HIP;
  return st;
}

extern "C" kq_status kq_weight_factor(const void *P, int m, kq_dtype dtype, void *out, void *stream) {
  const kq_status st = weight_factor_impl(P, m, dtype, out, stream);
  if (kq_log_on()) kq_logf("weight_factor m=%d: %s", m, kq_status_string(st));
  return st;
}
