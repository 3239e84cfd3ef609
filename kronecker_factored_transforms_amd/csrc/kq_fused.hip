// Fused Kronecker-factored transform + per-token INT4 quantization, bf16 MFMA, gfx950.
//
// Per token (n = n1*n2):  V = x (*c) viewed n1 x n2 row-major;  Z = V P2;  Y = P1^T Z;
// absmax -> clip -> fp16 step -> RTN -> clamp [-8, 7] -> two nibbles per byte.
// ("FlatQuant: Fast Learnable Affine Quantization", Deep Dive: Kronecker factorization
// and The fused kernel / Figure 8a; "Kronecker Product", Why It Matters: the identity
// vec(V)(P1 (x) P2) = vec(P1^T V P2).)
//
// What is kept from the page's fused design: both factors stay on chip for the kernel's
// lifetime, the token tile never leaves the CU between the two contractions, and only
// the packed INT4 tile (+ one scale per token) is written to HBM. What is different on
// gfx950: the two contractions run on 16x16x32 bf16 MFMA with fp32 accumulation and
// the intermediate Z is handed from stage 1 to stage 2 in registers (no LDS round trip):
// the stage-1 accumulator layout (4 consecutive rows of one column per lane) is exactly
// a stage-2 operand layout once the reduction index is re-ordered, and that re-ordering
// is absorbed by storing P1 pre-permuted in the plan. Quantization is done on the
// stage-2 accumulators with a wave reduction for the absmax.
//
// Work split: a workgroup has 4 waves; a token is shared by W = n2/32 waves, each of
// which owns 32 output columns (a column block of Y needs only the same column block
// of Z, which needs all of V and 32 columns of P2). The token tile V is staged in LDS
// (XOR-swizzled 16-byte chunks) and read by the W waves as MFMA A operands.
//
// MFMA operand layouts used below (wave64, 16x16x32 bf16; lane L, g = L/16):
//   A (16 x 32):  lane L holds row L%16, 8 reduction slots (g, v), v = 0..7
//   B (32 x 16):  lane L holds column L%16, the same 8 reduction slots (g, v)
//   D (16 x 16):  lane L holds rows 4g + r (r = 0..3) of column L%16
// Only the pairing of A's and B's slots matters for a reduction, so the kernel chooses
// which reduction index each slot carries and stores the factors in that order.

#include "kq_internal.h"

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

template <int N1, int N2, bool HAS_C>
struct Cfg {
  static_assert(N1 % 16 == 0 && N1 >= 16 && N1 <= 128, "n1 must be a multiple of 16 up to 128");
  static_assert(N2 == 32 || N2 == 64 || N2 == 128, "n2 must be 32, 64 or 128");
  static constexpr int W = N2 / 32;                 // waves per token
  static constexpr int TPI = kWaves / W;            // tokens per workgroup iteration
  static constexpr int MT = N1 / 16;                // 16-row tiles of V / Z
  static constexpr int KS = N2 / 32;                // stage-1 reduction steps
  static constexpr int KK = N1 / 32;                // stage-2 full reduction steps
  static constexpr bool KHALF = (N1 % 32) != 0;     // one trailing 16-wide stage-2 step
  static constexpr int CH = N2 / 8;                 // 16-byte chunks per V row
  static constexpr int TOK_CHUNKS = N1 * CH;
  static constexpr int CPT = TPI * TOK_CHUNKS / kThreads;  // chunks per thread per iter
  static_assert(CPT * kThreads == TPI * TOK_CHUNKS, "token tile must split evenly");
  static constexpr int V_BYTES = N1 * N2 * 2;
  static constexpr int P2_BYTES = N2 * N2 * 2;
  static constexpr int P1_BYTES = N1 * N1 * 2;
  static constexpr int VPLANES = HAS_C ? 2 : 1;     // hi (+ lo) bf16 planes of x*c
  static constexpr int VBUF = TPI * V_BYTES * VPLANES;
};

// byte offset of 16-byte chunk `cc` of row `r` of a token tile in LDS (XOR swizzle so
// that the 16 rows read by one A-operand load land in distinct banks)
template <int CH>
__device__ __forceinline__ int vchunk_off(int r, int cc) {
  return (r * CH + (cc ^ (r & (CH - 1)))) * 16;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ bf16x8 pack8(const f32x4 &a, const f32x4 &b) {
  bf16x8 r;
  r[0] = (__bf16)a[0]; r[1] = (__bf16)a[1]; r[2] = (__bf16)a[2]; r[3] = (__bf16)a[3];
  r[4] = (__bf16)b[0]; r[5] = (__bf16)b[1]; r[6] = (__bf16)b[2]; r[7] = (__bf16)b[3];
  return r;
}

__device__ __forceinline__ bf16x4 pack4(const f32x4 &a) {
  bf16x4 r;
  r[0] = (__bf16)a[0]; r[1] = (__bf16)a[1]; r[2] = (__bf16)a[2]; r[3] = (__bf16)a[3];
  return r;
}

// q = clamp(rint(fp32(y * inv)), -8, 7) as a 4-bit two's-complement nibble
__device__ __forceinline__ uint32_t quant_nibble(float y, float inv) {
  float v = __fmul_rn(y, inv);
  v = rintf(v);
  v = fminf(fmaxf(v, -8.0f), 7.0f);
  return (uint32_t)((int)v) & 0xFu;
}

template <int N1, int N2, bool HAS_C>
__global__ __launch_bounds__(kThreads) void kq_fused_kernel(
    const __bf16 *__restrict__ X, int64_t T, int64_t ldx,
    const bf16x8 *__restrict__ p2op, const bf16x8 *__restrict__ p1op,
    const float *__restrict__ cvec, float clip, int scale_fp16,
    uint8_t *__restrict__ codes, void *__restrict__ scales, float *__restrict__ ydbg) {
  using C = Cfg<N1, N2, HAS_C>;
  __shared__ __align__(16) unsigned char s_p2[C::P2_BYTES];
  __shared__ __align__(16) unsigned char s_p1[C::P1_BYTES];
  __shared__ __align__(16) unsigned char s_v[C::VBUF];
  __shared__ float s_red[kWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int lr = lane & 15;
  const int ts = wave / C::W;  // token slot within the iteration
  const int wt = wave % C::W;  // column block of this wave
  constexpr int n = N1 * N2;
  const int64_t ngroups = (T + C::TPI - 1) / C::TPI;

  // ---- factors -> LDS, once per workgroup (operand order, 16 B per lane) ----
  {
    const uint4 *src2 = reinterpret_cast<const uint4 *>(p2op);
    uint4 *dst2 = reinterpret_cast<uint4 *>(s_p2);
    for (int i = tid; i < C::P2_BYTES / 16; i += kThreads) dst2[i] = src2[i];
    const uint4 *src1 = reinterpret_cast<const uint4 *>(p1op);
    uint4 *dst1 = reinterpret_cast<uint4 *>(s_p1);
    for (int i = tid; i < C::P1_BYTES / 16; i += kThreads) dst1[i] = src1[i];
  }

  // per-thread chunk coordinates (fixed for the whole kernel)
  int c_ts[C::CPT], c_row[C::CPT], c_cc[C::CPT];
#pragma unroll
  for (int i = 0; i < C::CPT; ++i) {
    const int q = tid + kThreads * i;
    c_ts[i] = q / C::TOK_CHUNKS;
    const int qq = q % C::TOK_CHUNKS;
    c_row[i] = qq / C::CH;
    c_cc[i] = qq % C::CH;
  }
  // per-channel scale of this thread's chunks, kept in registers
  float creg[HAS_C ? C::CPT : 1][8];
  if constexpr (HAS_C) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const float4 *cp = reinterpret_cast<const float4 *>(cvec + c_row[i] * N2 + c_cc[i] * 8);
      const float4 a = cp[0], b = cp[1];
      creg[i][0] = a.x; creg[i][1] = a.y; creg[i][2] = a.z; creg[i][3] = a.w;
      creg[i][4] = b.x; creg[i][5] = b.y; creg[i][6] = b.z; creg[i][7] = b.w;
    }
  }

  uint4 pre[C::CPT];
  auto issue_loads = [&](int64_t grp) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int64_t tok = grp * C::TPI + c_ts[i];
      if (tok < T) {
        pre[i] = *reinterpret_cast<const uint4 *>(X + tok * ldx + c_row[i] * N2 + c_cc[i] * 8);
      } else {
        pre[i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };
  auto store_lds = [&]() {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int off = c_ts[i] * C::V_BYTES + vchunk_off<C::CH>(c_row[i], c_cc[i]);
      if constexpr (HAS_C) {
        const uint32_t w[4] = {pre[i].x, pre[i].y, pre[i].z, pre[i].w};
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = __uint_as_float(w[e] << 16);
          const float x1 = __uint_as_float(w[e] & 0xFFFF0000u);
          const float s0 = __fmul_rn(x0, creg[i][2 * e]);
          const float s1 = __fmul_rn(x1, creg[i][2 * e + 1]);
          const __bf16 h0 = (__bf16)s0, h1 = (__bf16)s1;
          const __bf16 l0 = (__bf16)__fsub_rn(s0, (float)h0);
          const __bf16 l1 = (__bf16)__fsub_rn(s1, (float)h1);
          hi[e] = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
                  ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
          lo[e] = (uint32_t)__builtin_bit_cast(uint16_t, l0) |
                  ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
        }
        *reinterpret_cast<uint4 *>(s_v + off) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        *reinterpret_cast<uint4 *>(s_v + C::TPI * C::V_BYTES + off) =
            make_uint4(lo[0], lo[1], lo[2], lo[3]);
      } else {
        *reinterpret_cast<uint4 *>(s_v + off) = pre[i];
      }
    }
  };

  int64_t grp = blockIdx.x;
  if (grp < ngroups) issue_loads(grp);
  __syncthreads();  // factors visible

  const bf16x8 *sp2 = reinterpret_cast<const bf16x8 *>(s_p2);
  const bf16x8 *sp1 = reinterpret_cast<const bf16x8 *>(s_p1);

  for (; grp < ngroups; grp += gridDim.x) {
    store_lds();
    __syncthreads();
    {
      const int64_t nxt = grp + gridDim.x;
      if (nxt < ngroups) issue_loads(nxt);  // in flight while this group computes
    }
    const int64_t tok = grp * C::TPI + ts;
    const unsigned char *vt = s_v + ts * C::V_BYTES;

    // ---- stage 1: Z[:, block] = V P2[:, block]  (M = n1 rows, K = n2, N = 32) ----
    f32x4 zacc[C::MT][2];
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) zacc[mt][0] = zacc[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const bf16x8 b0 = sp2[((wt * C::KS + ks) * 2 + 0) * 64 + lane];
      const bf16x8 b1 = sp2[((wt * C::KS + ks) * 2 + 1) * 64 + lane];
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) {
        const int r = mt * 16 + lr;
        const int off = vchunk_off<C::CH>(r, ks * 4 + g);
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(vt + off);
        zacc[mt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b0, zacc[mt][0], 0, 0, 0);
        zacc[mt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b1, zacc[mt][1], 0, 0, 0);
        if constexpr (HAS_C) {
          const bf16x8 al = *reinterpret_cast<const bf16x8 *>(vt + C::TPI * C::V_BYTES + off);
          zacc[mt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b0, zacc[mt][0], 0, 0, 0);
          zacc[mt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b1, zacc[mt][1], 0, 0, 0);
        }
      }
    }

    // ---- stage 2: Y^T[block, :] = Z[:, block]^T P1  (M = 32, K = n1, N = n1) ----
    // The stage-1 accumulators of row tiles (2kk, 2kk+1) form the A operand of
    // reduction step kk; P1 is stored in the matching reduction order.
    f32x4 yacc[2][C::MT];
#pragma unroll
    for (int nt = 0; nt < C::MT; ++nt) yacc[0][nt] = yacc[1][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      const bf16x8 za0 = pack8(zacc[2 * kk][0], zacc[2 * kk + 1][0]);
      const bf16x8 za1 = pack8(zacc[2 * kk][1], zacc[2 * kk + 1][1]);
#pragma unroll
      for (int nt = 0; nt < C::MT; ++nt) {
        const bf16x8 b = sp1[(kk * C::MT + nt) * 64 + lane];
        yacc[0][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(za0, b, yacc[0][nt], 0, 0, 0);
        yacc[1][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(za1, b, yacc[1][nt], 0, 0, 0);
      }
    }
    if constexpr (C::KHALF) {
      const bf16x4 za0 = pack4(zacc[2 * C::KK][0]);
      const bf16x4 za1 = pack4(zacc[2 * C::KK][1]);
      const bf16x4 *sp1h = reinterpret_cast<const bf16x4 *>(s_p1 + C::KK * C::MT * 1024);
#pragma unroll
      for (int nt = 0; nt < C::MT; ++nt) {
        const bf16x4 b = sp1h[nt * 64 + lane];
        yacc[0][nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(za0, b, yacc[0][nt], 0, 0, 0);
        yacc[1][nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(za1, b, yacc[1][nt], 0, 0, 0);
      }
    }

    // ---- epilogue: absmax over the token (wave, then the W waves sharing it) ----
    float m = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int nt = 0; nt < C::MT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(yacc[h][nt][r]));
    m = wave_max(m);
    if (lane == 0) s_red[wave] = m;
    __syncthreads();
    float amax = 0.f;
#pragma unroll
    for (int w = 0; w < C::W; ++w) amax = fmaxf(amax, s_red[ts * C::W + w]);

    // step s = fp16(fp32(fp32(clip * a) / 7)); codes use the stored step
    const float s32 = __fdiv_rn(__fmul_rn(clip, amax), 7.0f);
    float sf;
    _Float16 s16 = (_Float16)s32;
    if (scale_fp16) sf = (float)s16; else sf = s32;
    const float inv = (sf == 0.f) ? 0.f : __fdiv_rn(1.0f, sf);

    if (tok < T) {
      // lane holds Y[j = nt*16 + lr][wt*32 + 8g + 4h + r]: 8 consecutive codes -> 1 dword
      uint8_t *crow = codes + tok * (int64_t)(n / 2);
#pragma unroll
      for (int nt = 0; nt < C::MT; ++nt) {
        const int j = nt * 16 + lr;
        uint32_t word = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < 4; ++r) word |= quant_nibble(yacc[h][nt][r], inv) << (4 * (4 * h + r));
        *reinterpret_cast<uint32_t *>(crow + j * (N2 / 2) + wt * 16 + g * 4) = word;
        if (ydbg != nullptr) {
          float4 *yp = reinterpret_cast<float4 *>(ydbg + tok * (int64_t)n + j * N2 + wt * 32 + g * 8);
          yp[0] = make_float4(yacc[0][nt][0], yacc[0][nt][1], yacc[0][nt][2], yacc[0][nt][3]);
          yp[1] = make_float4(yacc[1][nt][0], yacc[1][nt][1], yacc[1][nt][2], yacc[1][nt][3]);
        }
      }
      if (wt == 0 && lane == 0) {
        if (scale_fp16) reinterpret_cast<_Float16 *>(scales)[tok] = s16;
        else reinterpret_cast<float *>(scales)[tok] = s32;
      }
    }
    __syncthreads();  // V tile and s_red are reused by the next iteration
  }
}

template <int N1, int N2, bool HAS_C>
hipError_t launch_fused(const kq_plan *p, const void *X, int64_t T, int64_t ldx, uint8_t *codes,
                        void *scales, float *y_debug, hipStream_t stream) {
  using C = Cfg<N1, N2, HAS_C>;
  const int64_t ngroups = (T + C::TPI - 1) / C::TPI;
  const int grid = (int)(ngroups < (int64_t)p->grid_cap ? ngroups : (int64_t)p->grid_cap);
  hipLaunchKernelGGL((kq_fused_kernel<N1, N2, HAS_C>), dim3(grid), dim3(kThreads), 0, stream,
                     static_cast<const __bf16 *>(X), T, ldx,
                     static_cast<const bf16x8 *>(p->p2op), static_cast<const bf16x8 *>(p->p1op),
                     p->c, p->clip, p->scale_dtype == KQ_FP16 ? 1 : 0, codes, scales, y_debug);
  return hipGetLastError();
}

struct Entry {
  int n1, n2;
  bool has_c;
  kq_launch_fn fn;
  const void *sym;
  const char *name;
};

#define KQ_FUSED_ENTRY(A, B)                                                           \
  {A, B, false, &launch_fused<A, B, false>,                                            \
   reinterpret_cast<const void *>(&kq_fused_kernel<A, B, false>),                      \
   "fused_mfma_bf16_" #A "x" #B},                                                      \
  {A, B, true, &launch_fused<A, B, true>,                                              \
   reinterpret_cast<const void *>(&kq_fused_kernel<A, B, true>),                       \
   "fused_mfma_bf16_" #A "x" #B "_c"}

const Entry kEntries[] = {
    KQ_FUSED_ENTRY(16, 32),  KQ_FUSED_ENTRY(32, 32),
    KQ_FUSED_ENTRY(16, 64),  KQ_FUSED_ENTRY(32, 64),  KQ_FUSED_ENTRY(48, 64),
    KQ_FUSED_ENTRY(64, 64),
    KQ_FUSED_ENTRY(16, 128), KQ_FUSED_ENTRY(32, 128), KQ_FUSED_ENTRY(48, 128),
    KQ_FUSED_ENTRY(64, 128), KQ_FUSED_ENTRY(80, 128), KQ_FUSED_ENTRY(96, 128),
    KQ_FUSED_ENTRY(112, 128), KQ_FUSED_ENTRY(128, 128),
};

}  // namespace

kq_launch_fn kq_fused_lookup(int n1, int n2, bool has_c, const char **name,
                             const void **kernel_symbol) {
  for (const Entry &e : kEntries) {
    if (e.n1 == n1 && e.n2 == n2 && e.has_c == has_c) {
      if (name) *name = e.name;
      if (kernel_symbol) *kernel_symbol = e.sym;
      return e.fn;
    }
  }
  return nullptr;
}

int kq_fused_threads() { return kThreads; }

size_t kq_fused_p1op_elems(int n1) { return (size_t)n1 * (size_t)n1; }
size_t kq_fused_p2op_elems(int n2) { return (size_t)n2 * (size_t)n2; }

// P2 as stage-1 B operands: [wave block wb][step ks][tile a][lane L][slot v] =
//   P2[32 ks + 8 g + v][32 wb + sigma(16 a + L%16)],  g = L/16,
// with sigma(16a + 4b + r) = 8b + 4a + r, so that after stage 2 every lane holds 8
// consecutive output columns (one packed dword of codes).
void kq_fused_arrange_p2(const uint16_t *P2, int n2, uint16_t *out) {
  const int W = n2 / 32, KS = n2 / 32;
  size_t o = 0;
  for (int wb = 0; wb < W; ++wb)
    for (int ks = 0; ks < KS; ++ks)
      for (int a = 0; a < 2; ++a)
        for (int L = 0; L < 64; ++L)
          for (int v = 0; v < 8; ++v) {
            const int g = L / 16, x = L % 16, b = x / 4, r = x % 4;
            const int k = 32 * ks + 8 * g + v;
            const int col = 32 * wb + 8 * b + 4 * a + r;
            out[o++] = P2[(size_t)k * n2 + col];
          }
}

// P1 as stage-2 B operands: full steps [kk][tile t][lane L][slot v] =
//   P1[32 kk + 16 (v/4) + 4 g + (v%4)][16 t + L%16]
// (slot order of the stage-1 accumulators of row tiles 2kk and 2kk+1), then, when n1 is
// an odd multiple of 16, one half step [t][L][v<4] = P1[32 KK + 4 g + v][16 t + L%16].
void kq_fused_arrange_p1(const uint16_t *P1, int n1, uint16_t *out) {
  const int MT = n1 / 16, KK = n1 / 32;
  size_t o = 0;
  for (int kk = 0; kk < KK; ++kk)
    for (int t = 0; t < MT; ++t)
      for (int L = 0; L < 64; ++L)
        for (int v = 0; v < 8; ++v) {
          const int g = L / 16;
          const int i = 32 * kk + 16 * (v / 4) + 4 * g + (v % 4);
          out[o++] = P1[(size_t)i * n1 + 16 * t + L % 16];
        }
  if (n1 % 32) {
    for (int t = 0; t < MT; ++t)
      for (int L = 0; L < 64; ++L)
        for (int v = 0; v < 4; ++v) {
          const int g = L / 16;
          const int i = 32 * KK + 4 * g + v;
          out[o++] = P1[(size_t)i * n1 + 16 * t + L % 16];
        }
  }
}
