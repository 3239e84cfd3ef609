// kq_gemm.hip -- INT4 x INT4 GEMM on the gfx950 int8 matrix cores: the consumer of two
// kq_transform_quant outputs (the transformed activations and the transformed weights).
//
//   out[t][j] = cvt( fp32( fp32( fp32(acc) * sx[t] ) * sw[j] ) ),
//   acc = sum_k qx[t][k] * qw[j][k]   (exact, int32)
//
// ("FlatQuant: Fast Learnable Affine Quantization", Putting It Together: both sides of a
// linear layer are quantized to INT4 and multiplied by an INT4 GEMM; "High-Rate Quantized
// Matrix Multiplication I", Technical Summary: the product of two absmax-quantized
// matrices is their integer product times the two scale vectors.)
//
// Codes are 4-bit two's complement, element 2m in the low nibble of byte m. A code moved
// into the high nibble of a byte is the int8 value 16 q, so unpacking is one shift and two
// masks per 8 codes and needs no sign extension; the MFMA then sums 256 q_x q_w and the
// accumulator is shifted right by 8 (exact). The order of the reduction index inside an
// MFMA operand is free as long as both operands use the same one (the instruction pairs
// byte b of A lane i+16g with byte b of B lane j+16g), so the even codes of a dword and
// then its odd codes go to consecutive operand bytes.
//
// Tiling: a workgroup of 8 waves computes 256 weight rows (output channels) x 256 tokens,
// over K in steps of 256 codes (128 bytes per row) double-buffered in LDS; every wave
// owns 128 x 64 outputs (8 x 4 MFMA 16x16x64 tiles). Each step's tiles arrive by DMA,
// 1 KiB of consecutive memory (8 rows x 128 bytes) per instruction, with the 16-byte
// pieces of row R stored at position p ^ ((R / 2) % 8): the 16 rows of one fragment read
// (16 bytes per lane, one piece) then spread evenly over the 8 bank groups of a row. The
// weight side is the MFMA A operand, so a lane ends with 4 consecutive output channels
// of one token (one vector store).
#include "kq_internal.h"
#include "kq_device.h"

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBM = 256;                   // weight rows (output channels) per workgroup
constexpr int kBN = 256;                   // tokens per workgroup
constexpr int kRowBytes = 128;             // code bytes per row and K step (256 codes)
constexpr int kGemmWaves = 8;              // 2 along weight rows x 4 along tokens
constexpr int kGemmThreads = kGemmWaves * 64;
constexpr int kMI = kBM / 2 / 16;          // 8 MFMA tiles along weight rows per wave
constexpr int kNI = kBN / 4 / 16;          // 4 MFMA tiles along tokens per wave
constexpr int kOpBytes = kBM * kRowBytes;  // 32 KiB per operand and stage (kBM == kBN)
constexpr int kLoads = kOpBytes / 1024 / kGemmWaves;  // DMA instructions per wave, operand, step
static_assert(kBM == kBN, "one DMA layout for both operands");
static_assert(kLoads * 1024 * kGemmWaves == kOpBytes, "tile splits evenly over the waves");

// 16 bytes of an operand fragment from one row's 8 code bytes (16 codes): the even codes
// of each dword, then its odd codes, each in the high nibble of a byte (= 16 q as int8).
__device__ __forceinline__ i32x4 unpack16(u32x2 c) {
  constexpr unsigned kHi = 0xF0F0F0F0u;
  return i32x4{(int)((c.x << 4) & kHi), (int)(c.x & kHi), (int)((c.y << 4) & kHi),
               (int)(c.y & kHi)};
}

template <int OUT>  // 0: fp32, 1: bf16 (RNE), 2: fp16 (RNE)
__global__ __launch_bounds__(kGemmThreads) void kq_int4_gemm_kernel(
    const uint8_t *__restrict__ xq, int64_t ldxq, const void *__restrict__ sx, int64_t T,
    const uint8_t *__restrict__ wq, int64_t ldwq, const void *__restrict__ sw, int64_t N,
    int ksteps, int scale_fp16, void *__restrict__ out, int64_t ldo, int tiles_m) {
  __shared__ __align__(16) unsigned char s_w[2][kOpBytes];
  __shared__ __align__(16) unsigned char s_x[2][kOpBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, lr = lane & 15;
  const int wm = wave & 1, wn = wave >> 1;  // this wave's 128 weight rows / 64 tokens
  const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int64_t n0 = (int64_t)tm * kBM, t0 = (int64_t)tn * kBN;

  // DMA: instruction J = wave kLoads + j of an operand fills tile rows 8J .. 8J+7; lane i
  // lands at row R = 8J + i/8, position i%8, i.e. reads piece (i%8) ^ ((R/2)%8) of that
  // row. Rows past the end of the matrix read its last row (their results are dropped).
  uint32_t voff_w[kLoads], voff_x[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int R = (wave * kLoads + j) * 8 + lane / 8;
    const int piece = (lane % 8) ^ ((R >> 1) & 7);
    const int64_t rw = n0 + R < N ? n0 + R : N - 1;
    const int64_t rx = t0 + R < T ? t0 + R : T - 1;
    voff_w[j] = (uint32_t)(rw * ldwq + piece * 16);
    voff_x[j] = (uint32_t)(rx * ldxq + piece * 16);
  }
  auto dma_step = [&](int ks, int b) {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const uint32_t lo = lds_addr(s_w[b] + (wave * kLoads + j) * 1024);
      dma16<false>(wq, voff_w[j] + (uint32_t)(ks * kRowBytes), lo);
    }
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const uint32_t lo = lds_addr(s_x[b] + (wave * kLoads + j) * 1024);
      dma16<false>(xq, voff_x[j] + (uint32_t)(ks * kRowBytes), lo);
    }
  };

  i32x4 acc[kMI][kNI];
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) acc[mi][ni] = i32x4{0, 0, 0, 0};

  // fragment rows: 16 mt + lr of this wave's block; (R/2)%8 == (lr/2)%8 for all of them
  const int sw8 = (lr >> 1) & 7;
  const int row_w = wm * (kBM / 2) + lr, row_x = wn * (kBN / 4) + lr;

  dma_step(0, 0);
  for (int ks = 0; ks < ksteps; ++ks) {
    const int b = ks & 1;
    // this step's tiles have landed (own DMAs), for every wave (barrier); every wave is
    // also done reading the other buffer, which the next DMA overwrites
    wait_and_fence<kWaitVm0>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    if (ks + 1 < ksteps) dma_step(ks + 1, b ^ 1);

#pragma unroll
    for (int q = 0; q < 2; ++q) {  // 128 codes (64 bytes) of the step: two MFMA steps
      // lane group g reads the whole piece 4 q + g (32 codes): its first 8 bytes feed the
      // first MFMA step, the last 8 bytes the second (for every row of both operands)
      const int off = ((4 * q + g) ^ sw8) * 16;
      u32x4_t pa[kMI], pb[kNI];
#pragma unroll
      for (int mi = 0; mi < kMI; ++mi)
        pa[mi] = *reinterpret_cast<const u32x4_t *>(s_w[b] + (row_w + mi * 16) * kRowBytes + off);
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni)
        pb[ni] = *reinterpret_cast<const u32x4_t *>(s_x[b] + (row_x + ni * 16) * kRowBytes + off);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        i32x4 a[kMI], bx[kNI];
#pragma unroll
        for (int mi = 0; mi < kMI; ++mi)
          a[mi] = unpack16(h ? u32x2{pa[mi].z, pa[mi].w} : u32x2{pa[mi].x, pa[mi].y});
#pragma unroll
        for (int ni = 0; ni < kNI; ++ni)
          bx[ni] = unpack16(h ? u32x2{pb[ni].z, pb[ni].w} : u32x2{pb[ni].x, pb[ni].y});
#pragma unroll
        for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
          for (int ni = 0; ni < kNI; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mi], bx[ni], acc[mi][ni], 0, 0, 0);
      }
    }
    wait_and_fence<kWaitLgkm0>();  // this wave's reads of buffer b have returned
  }

  // ---- epilogue: lane holds acc[mi][ni][r] = 256 x out channel n = n0 + wm 128 + 16 mi +
  // 4 g + r, token t = t0 + wn 64 + 16 ni + lr ----
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni) {
    const int64_t t = t0 + wn * (kBN / 4) + ni * 16 + lr;
    if (t >= T) continue;
    const float sxt = scale_fp16 ? (float)reinterpret_cast<const _Float16 *>(sx)[t]
                                 : reinterpret_cast<const float *>(sx)[t];
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi) {
      const int64_t n = n0 + wm * (kBM / 2) + mi * 16 + g * 4;
      if (n >= N) continue;  // N is a multiple of 4: the 4 channels are all in or all out
      float swn[4];
      if (scale_fp16) {
        const _Float16 *p = reinterpret_cast<const _Float16 *>(sw) + n;
#pragma unroll
        for (int r = 0; r < 4; ++r) swn[r] = (float)p[r];
      } else {
        const float4 v = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(sw) + n);
        swn[0] = v.x; swn[1] = v.y; swn[2] = v.z; swn[3] = v.w;
      }
      float o[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        o[r] = __fmul_rn(__fmul_rn((float)(acc[mi][ni][r] >> 8), sxt), swn[r]);
      if constexpr (OUT == 0) {
        *reinterpret_cast<float4 *>(reinterpret_cast<float *>(out) + t * ldo + n) =
            make_float4(o[0], o[1], o[2], o[3]);
      } else if constexpr (OUT == 1) {
        const __bf16 h[4] = {(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
        *reinterpret_cast<uint2 *>(reinterpret_cast<__bf16 *>(out) + t * ldo + n) =
            *reinterpret_cast<const uint2 *>(h);
      } else {
        const _Float16 h[4] = {(_Float16)o[0], (_Float16)o[1], (_Float16)o[2], (_Float16)o[3]};
        *reinterpret_cast<uint2 *>(reinterpret_cast<_Float16 *>(out) + t * ldo + n) =
            *reinterpret_cast<const uint2 *>(h);
      }
    }
  }
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

static kq_status int4_gemm_impl(const uint8_t *xq, int64_t ldxq, const void *sx, int64_t T,
                                const uint8_t *wq, int64_t ldwq, const void *sw, int64_t N,
                                int64_t K, kq_dtype scale_dtype, kq_dtype out_dtype, void *out,
                                int64_t ldo, void *stream) {
  if (T < 0 || N < 0 || K <= 0) return KQ_ERR_INVALID_ARG;
  if (scale_dtype != KQ_FP16 && scale_dtype != KQ_FP32) return KQ_ERR_INVALID_ARG;
  if (out_dtype != KQ_FP32 && out_dtype != KQ_BF16 && out_dtype != KQ_FP16)
    return KQ_ERR_INVALID_ARG;
  if (K % 256 != 0 || K > 65536 || N % 4 != 0) return KQ_ERR_UNSUPPORTED;
  if (T == 0 || N == 0) return KQ_OK;
  if (!xq || !wq || !sx || !sw || !out) return KQ_ERR_INVALID_ARG;
  if (ldxq < K / 2 || ldwq < K / 2 || ldo < N) return KQ_ERR_INVALID_ARG;
  const size_t oes = out_dtype == KQ_FP32 ? 4 : 2;
  if (!aligned(xq, 16) || !aligned(wq, 16) || ldxq % 16 != 0 || ldwq % 16 != 0)
    return KQ_ERR_ALIGNMENT;
  if (!aligned(sx, scale_dtype == KQ_FP16 ? 2 : 4) || !aligned(sw, scale_dtype == KQ_FP16 ? 2 : 16))
    return KQ_ERR_ALIGNMENT;
  if (!aligned(out, 4 * oes) || ((size_t)ldo * oes) % (4 * oes) != 0) return KQ_ERR_ALIGNMENT;
  // the DMA adds a 32-bit byte offset to the matrix base
  if ((uint64_t)T * (uint64_t)ldxq > 0xFFFFFFFFull || (uint64_t)N * (uint64_t)ldwq > 0xFFFFFFFFull)
    return KQ_ERR_UNSUPPORTED;
  const int64_t tiles_m = (N + kBM - 1) / kBM, tiles_n = (T + kBN - 1) / kBN;
  if (tiles_m * tiles_n > 0x7FFFFFFF) return KQ_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int fp16s = scale_dtype == KQ_FP16 ? 1 : 0;
  const int ks = (int)(K / 256);
  const dim3 grid((unsigned)(tiles_m * tiles_n)), block(kGemmThreads);
  switch (out_dtype) {
    case KQ_FP32:
      hipLaunchKernelGGL(kq_int4_gemm_kernel<0>, grid, block, 0, s, xq, ldxq, sx, T, wq, ldwq, sw,
                         N, ks, fp16s, out, ldo, (int)tiles_m);
      break;
    case KQ_BF16:
      hipLaunchKernelGGL(kq_int4_gemm_kernel<1>, grid, block, 0, s, xq, ldxq, sx, T, wq, ldwq, sw,
                         N, ks, fp16s, out, ldo, (int)tiles_m);
      break;
    default:
      hipLaunchKernelGGL(kq_int4_gemm_kernel<2>, grid, block, 0, s, xq, ldxq, sx, T, wq, ldwq, sw,
                         N, ks, fp16s, out, ldo, (int)tiles_m);
      break;
  }
  return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_HIP;
}

extern "C" kq_status kq_int4_gemm(const uint8_t *xq, int64_t ldxq, const void *sx, int64_t T,
                                  const uint8_t *wq, int64_t ldwq, const void *sw, int64_t N,
                                  int64_t K, kq_dtype scale_dtype, kq_dtype out_dtype, void *out,
                                  int64_t ldo, void *stream) {
  const kq_status st = int4_gemm_impl(xq, ldxq, sx, T, wq, ldwq, sw, N, K, scale_dtype, out_dtype,
                                      out, ldo, stream);
  if (kq_log_on())
    kq_logf("int4_gemm T=%lld N=%lld K=%lld: %s", (long long)T, (long long)N, (long long)K,
            kq_status_string(st));
  return st;
}
