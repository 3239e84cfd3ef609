// fp32 inputs on the bf16 matrix cores: the Kronecker transform + per-token quantization
// for plans whose X, P1 and P2 are fp32 ("Kronecker Product", Why It Matters: the
// identity vec(V)(P1 (x) P2) = vec(P1^T V P2); "FlatQuant: Fast Learnable Affine
// Quantization", Deep Dive: Kronecker factorization and The fused kernel).
//
// An fp32 value a is carried as two bf16 numbers, a_hi = bf16(a) and a_lo = bf16(a - a_hi),
// which hold about 16 of its 24 significant bits; a product a b is then formed from three
// bf16 MFMAs, a_hi b_hi + a_hi b_lo + a_lo b_hi, accumulated in fp32 (the dropped a_lo b_lo
// and the residual a - a_hi - a_lo are both below 2^-16 of a b). Both contractions run
// that way, and Z stays fp32 between them (split again for stage 2): no bf16 rounding of
// the intermediate, unlike the bf16 path. P1 and P2 are split once, in the plan.
//
// Work split (the stream kernel's, for fp32 tiles): one wave per token, eight waves per
// workgroup, persistent grid. Each wave owns a 16 KiB LDS slot for an n1 x 64 fp32 token;
// the next token arrives there by DMA (global_load_lds_dwordx4, 1 KiB of consecutive
// memory per instruction, non-temporal) as soon as stage 1 has read the slot. P2's and
// P1's hi / lo operands are shared in LDS. The 16-byte pieces of row R sit at position
// p ^ (R mod 16) of the row (256 bytes = one pass over the 64 LDS banks), so the 16 rows of
// an operand read hit 16 different bank groups.

#include "kq_internal.h"
#include "kq_device.h"
#include "kq_common.h"

namespace {

template <int N1>
struct F32Cfg {
  static_assert(N1 % 16 == 0 && N1 >= 16 && N1 <= 64, "fp32 kernel: n1 in {16, 32, 48, 64}");
  static constexpr int N2 = 64;
  static constexpr int WAVES = 8;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int MT = N1 / 16;            // row tiles of V / Z = column tiles of Y
  static constexpr int NT = N2 / 16;            // column tiles of Z / Y
  static constexpr int KS = N2 / 32;            // stage-1 reduction steps
  static constexpr int KK = (N1 + 31) / 32;     // stage-2 reduction steps
  static constexpr bool KHALF = (N1 % 32) != 0;
  static constexpr int RB = N2 * 4;             // bytes per row of V (256)
  static constexpr int TILE = N1 * RB;          // bytes of one token
  static constexpr int LOADS = TILE / 1024;     // DMA instructions per token (4 rows each)
  static constexpr int P2_OPS = N2 * N2 / 8;    // bf16x8 operands of P2 (hi or lo)
  static constexpr int P1_OPS = KK * MT * 64;   // bf16x8 operands of P1 (hi or lo)
  static_assert(WAVES * TILE + 2 * (P2_OPS + P1_OPS) * 16 <= 160 * 1024, "LDS budget");
};

// 8 fp32 values -> hi = bf16(v), lo = bf16(v - float(hi)), both round to nearest even;
// per pair: one paired conversion for hi, two unpacks, two subtractions, one paired
// conversion for lo
__device__ __forceinline__ void split8(const float (&v)[8], bf16x8 &hi, bf16x8 &lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bf16x2_t hv = {(__bf16)v[2 * e], (__bf16)v[2 * e + 1]};  // v_cvt_pk_bf16_f32
    h[e] = __builtin_bit_cast(uint32_t, hv);
    asm("" : "+v"(h[e]));  // unpack hi from this word, not by converting v again
    const float r0 = __fsub_rn(v[2 * e], __uint_as_float(h[e] << 16));
    const float r1 = __fsub_rn(v[2 * e + 1], __uint_as_float(h[e] & 0xFFFF0000u));
    const bf16x2_t lv = {(__bf16)r0, (__bf16)r1};
    l[e] = __builtin_bit_cast(uint32_t, lv);
  }
  hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
}

// a_hi b_hi + a_hi b_lo + a_lo b_hi
__device__ __forceinline__ f32x4 mfma3(const bf16x8 &ah, const bf16x8 &al, const bf16x8 &bh,
                                       const bf16x8 &bl, f32x4 c) {
  c = mfma(ah, bh, c);
  c = mfma(ah, bl, c);
  return mfma(al, bh, c);
}

template <int N1, bool YDBG>
__global__ __launch_bounds__(512) void kq_f32_kernel(
    const float *__restrict__ X, int64_t T, int64_t ldx, const bf16x8 *__restrict__ p2op,
    const bf16x8 *__restrict__ p1op, float clip, int scale_fp16, int clip_allows_no_clamp,
    uint8_t *__restrict__ codes, void *__restrict__ scales, float *__restrict__ ydbg) {
  using C = F32Cfg<N1>;
  constexpr int N2 = C::N2;
  constexpr int n = N1 * N2;
  // P2 hi, P2 lo, P1 hi, P1 lo operands, then one token slot per wave
  __shared__ __align__(16) bf16x8 s_ops[2 * (C::P2_OPS + C::P1_OPS)];
  __shared__ __align__(16) unsigned char s_tile[C::WAVES][C::TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, lr = lane & 15;
  unsigned char *slot = s_tile[wave];

  // DMA of token `tok` into the slot: instruction j fills rows 4 j .. 4 j + 3; lane i lands
  // at row R = 4 j + i / 16, position i % 16, so it reads piece (i % 16) ^ (R % 16). The
  // lane's offset within the instruction's 1 KiB repeats every 4 instructions.
  uint32_t voff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int R = 4 * j + lane / 16;
    voff[j] = (uint32_t)((lane / 16) * C::RB + (((lane % 16) ^ (R % 16)) * 16));
  }
  auto dma_tile = [&](int64_t tok) {
    const unsigned char *xt = reinterpret_cast<const unsigned char *>(X + tok * ldx);
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j) dma16_nt(xt + j * 1024, voff[j % 4], lds_addr(slot + j * 1024));
  };

  const int64_t stride = (int64_t)gridDim.x * C::WAVES;
  int64_t tok = (int64_t)blockIdx.x * C::WAVES + wave;
  // the factor operands reach LDS by DMA, each wave copying its share, before any token
  dma_copy(p2op, s_ops, 2 * C::P2_OPS * 16, wave, C::WAVES, lane);
  dma_copy(p1op, s_ops + 2 * C::P2_OPS, 2 * C::P1_OPS * 16, wave, C::WAVES, lane);
  // The first half of the waves issues its token's DMA at once and waits for it before the
  // barrier; the second half issues its own only after the barrier, i.e. once the first
  // half's tokens have landed. The first tokens then arrive sooner and half the CU computes
  // while the rest load (measured on MI355X: 6 % on 2048 fp32 tokens of 64x64, 0.5 % on
  // 16384 tokens of 64x128, neutral on 2048 tokens with c).
  if (wave < C::WAVES / 2) {
    if (tok < T) dma_tile(tok);
    wait_and_fence<kWaitVm0>();
    lds_barrier();  // operands visible to every wave
  } else {
    wait_and_fence<kWaitVm0>();
    lds_barrier();  // operands visible to every wave
    if (tok < T) dma_tile(tok);
  }
  const bf16x8 *p2h = s_ops, *p2l = s_ops + C::P2_OPS;
  const bf16x8 *p1h = s_ops + 2 * C::P2_OPS, *p1l = p1h + C::P1_OPS;

  uint32_t pend[C::MT][C::NT / 2];
  TokenScale pend_s{0.f, (_Float16)0.f, 0.f};
  int64_t pend_tok = -1;
  auto store_pending = [&]() {
    store_codes<N1, N2>(codes, pend_tok, pend, lr, g);
    if (lane == 0) store_scale(scales, pend_tok, pend_s, scale_fp16);
  };

  for (; tok < T; tok += stride) {
    wait_and_fence<kWaitVm0>();  // this token's tile (and older stores) have landed
    if (pend_tok >= 0) store_pending();

    // ---- stage 1: Z = V P2 (fp32 accumulators, all column tiles) ----
    f32x4 zacc[C::MT][C::NT];
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) zacc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      // A operand (mt, ks) of lane L: V[16 mt + lr][32 ks + 8 g + v], pieces 2 (4 ks + g)
      // and 2 (4 ks + g) + 1 of row 16 mt + lr
      bf16x8 ah[C::MT], al[C::MT];
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) {
        const unsigned char *row = slot + (mt * 16 + lr) * C::RB;
        const int p0 = 2 * (4 * ks + g);
        const float4 a = *reinterpret_cast<const float4 *>(row + ((p0 ^ lr) * 16));
        const float4 b = *reinterpret_cast<const float4 *>(row + (((p0 + 1) ^ lr) * 16));
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        split8(v, ah[mt], al[mt]);
      }
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) {
        const bf16x8 bh = p2h[(ks * C::NT + nt) * 64 + lane], bl = p2l[(ks * C::NT + nt) * 64 + lane];
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt) zacc[mt][nt] = mfma3(ah[mt], al[mt], bh, bl, zacc[mt][nt]);
      }
    }
    wait_and_fence<kWaitLgkm0>();  // every slot read has returned: the slot is free again
    if (tok + stride < T) dma_tile(tok + stride);

    // ---- stage 2: Y^T = Z^T P1, Z split into hi / lo operands ----
    f32x4 yacc[C::NT][C::MT];
#pragma unroll
    for (int m2 = 0; m2 < C::NT; ++m2)
#pragma unroll
      for (int nt = 0; nt < C::MT; ++nt) yacc[m2][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      const bool pad = C::KHALF && kk == C::KK - 1;
      bf16x8 zh[C::NT], zl[C::NT];
#pragma unroll
      for (int m2 = 0; m2 < C::NT; ++m2) {
        const f32x4 z0 = zacc[2 * kk][m2];
        const f32x4 z1 = pad ? zero : zacc[(2 * kk + 1) % C::MT][m2];
        const float v[8] = {z0[0], z0[1], z0[2], z0[3], z1[0], z1[1], z1[2], z1[3]};
        split8(v, zh[m2], zl[m2]);
      }
#pragma unroll
      for (int nt = 0; nt < C::MT; ++nt) {
        const bf16x8 bh = p1h[(kk * C::MT + nt) * 64 + lane], bl = p1l[(kk * C::MT + nt) * 64 + lane];
#pragma unroll
        for (int m2 = 0; m2 < C::NT; ++m2) yacc[m2][nt] = mfma3(zh[m2], zl[m2], bh, bl, yacc[m2][nt]);
      }
    }

    // ---- epilogue: lane holds Y[16 nt + lr][16 g + 4 m2 + r] ----
    float m = 0.f;
#pragma unroll
    for (int m2 = 0; m2 < C::NT; ++m2)
#pragma unroll
      for (int nt = 0; nt < C::MT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(yacc[m2][nt][r]));
    const float amax = wave_max_uniform(m);
    const TokenScale ts = token_scale(amax, clip, scale_fp16);
    if (__builtin_amdgcn_readfirstlane(clamp_needed(clip_allows_no_clamp, ts.s32) ? 1 : 0))
      quant_tile<true, C::MT, C::NT>(yacc, ts.inv, pend);
    else
      quant_tile<false, C::MT, C::NT>(yacc, ts.inv, pend);
    pend_s = ts;
    pend_tok = tok;
    if constexpr (YDBG) {
#pragma unroll
      for (int nt = 0; nt < C::MT; ++nt) {
        float4 *yp = reinterpret_cast<float4 *>(ydbg + tok * (int64_t)n + (nt * 16 + lr) * N2 + g * 16);
#pragma unroll
        for (int m2 = 0; m2 < C::NT; ++m2)
          yp[m2] = make_float4(yacc[m2][nt][0], yacc[m2][nt][1], yacc[m2][nt][2], yacc[m2][nt][3]);
      }
    }
  }
  if (pend_tok >= 0) store_pending();
}

template <int N1>
hipError_t launch_f32(const kq_plan *p, const void *X, int64_t T, int64_t ldx, uint8_t *codes,
                      void *scales, float *y_debug, void *, hipStream_t stream) {
  using C = F32Cfg<N1>;
  const int64_t ngroups = (T + C::WAVES - 1) / C::WAVES;
  const int grid = (int)(ngroups < (int64_t)p->grid_cap ? ngroups : (int64_t)p->grid_cap);
  auto k = y_debug ? &kq_f32_kernel<N1, true> : &kq_f32_kernel<N1, false>;
  hipLaunchKernelGGL(k, dim3(grid), dim3(C::THREADS), 0, stream, static_cast<const float *>(X), T, ldx,
                     static_cast<const bf16x8 *>(p->p2op), static_cast<const bf16x8 *>(p->p1op),
                     p->clip, p->scale_dtype == KQ_FP16 ? 1 : 0, p->clip >= 0.935f ? 1 : 0, codes,
                     scales, y_debug);
  return hipGetLastError();
}

#define KQ_F32(A)                                                                       \
  kq_fused_variant{A, 64, false, KQ_SPLIT_STREAM, 4, 64, F32Cfg<A>::THREADS, &launch_f32<A>, \
                   reinterpret_cast<const void *>(&kq_f32_kernel<A, false>),              \
                   "fused_mfma_f32x3_stream_" #A "x64"}
const kq_fused_variant kF32Variants[] = {KQ_F32(16), KQ_F32(32), KQ_F32(48), KQ_F32(64)};

}  // namespace

const kq_fused_variant *kq_f32_lookup(int n1, int n2, bool has_c) {
  if (has_c) return nullptr;
  for (const kq_fused_variant &e : kF32Variants)
    if (e.n1 == n1 && e.n2 == n2) return &e;
  return nullptr;
}
