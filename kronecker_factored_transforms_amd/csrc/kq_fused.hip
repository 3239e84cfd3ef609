// Fused Kronecker-factored transform + per-token INT4 (or INT8) quantization, bf16 MFMA,
// gfx950.
//
// Per token (n = n1*n2):  V = x (*c) viewed n1 x n2 row-major;  Z = V P2;  Y = P1^T Z;
// absmax -> clip -> fp16 step -> RTN -> clamp [-8, 7] -> two nibbles per byte.
// ("FlatQuant: Fast Learnable Affine Quantization", Deep Dive: Kronecker factorization
// and The fused kernel / Figure 8a; "Kronecker Product", Why It Matters: the identity
// vec(V)(P1 (x) P2) = vec(P1^T V P2).)
//
// What is kept from the page's fused design: both factors stay on chip for the kernel's
// lifetime, the token tile never leaves the CU between the two contractions, and only
// the packed codes (+ one scale per token) are written to HBM. What is different on
// gfx950: the two contractions run on 16x16x32 bf16 MFMA with fp32 accumulation and
// the intermediate Z is handed from stage 1 to stage 2 in registers (no LDS round trip):
// the stage-1 accumulator layout (4 consecutive rows of one column per lane) is exactly
// a stage-2 operand layout once the reduction index is re-ordered, and that re-ordering
// is absorbed by storing P1 pre-permuted in the plan. Quantization runs on the stage-2
// accumulators with a wave reduction for the absmax.
//
// Work splits (each a kernel below; the plan picks one per shape, see the variant table):
//  * register kernel: 1 or 2 waves per token, the token loaded straight from HBM into
//    MFMA A-operand registers ("deep": one wave per SIMD, next token prefetched);
//  * stream kernel: one wave per token, the next token brought into an LDS slot by DMA
//    while the current one is computed (also rows of 112 values in the 128 layout);
//  * pair kernel: two waves per token, one column half each (small batches);
//  * rows kernel: identity left factor, one step per row of V (per-head transforms);
//  * column kernel: a token shared by n2/32 waves of a workgroup, each owning 32 output
//    columns, the tile staged in LDS (larger factors, n1 not a multiple of 16, n2 an odd
//    multiple of 16, and the shapes with a per-channel scale beyond the stream kernel's).
// The stream, pair, column and rows kernels also write INT8 codes (one byte per value).
//
// MFMA operand layouts used below (wave64, 16x16x32 bf16; lane L, g = L/16):
//   A (16 x 32):  lane L holds row L%16, 8 reduction slots (g, v), v = 0..7
//   B (32 x 16):  lane L holds column L%16, the same 8 reduction slots (g, v)
//   D (16 x 16):  lane L holds rows 4g + r (r = 0..3) of column L%16
// Only the pairing of A's and B's slots matters for a reduction, so the kernels choose
// which reduction index each slot carries and the plan stores the factors in that order.

#include "kq_internal.h"
#include "kq_device.h"
#include "kq_common.h"


namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ void copy_to_lds(unsigned char *dst, const void *src, int bytes,
                                            int tid, int nthreads = kThreads) {
  const uint4 *s = reinterpret_cast<const uint4 *>(src);
  uint4 *d = reinterpret_cast<uint4 *>(dst);
  for (int i = tid; i < bytes / 16; i += nthreads) d[i] = s[i];
}

// ------------------------------------------------------------------------------------
// register kernel: WPT (1 or 2) waves per token, the token loaded straight into registers
// ------------------------------------------------------------------------------------
template <int N1, int N2, int WPT, bool HAS_C, bool DEEP = false>
struct RegCfg {
  static_assert(N1 % 16 == 0 && N1 >= 16 && N1 <= 64, "register kernel: n1 in {16, 32, 48, 64}");
  static_assert(N2 == 32 || N2 == 64 || N2 == 128, "n2 must be 32, 64 or 128");
  static_assert(WPT == 1 || WPT == 2, "one or two waves per token");
  static_assert(N2 / WPT >= 32, "a wave owns at least 32 output columns");
  static constexpr int MT = N1 / 16;            // row tiles of V/Z = column tiles (j) of Y
  static constexpr int NT = N2 / 16 / WPT;      // column tiles (l) of this wave's block
  static constexpr int CB = N2 / WPT;           // output columns owned by a wave
  static constexpr int KS = N2 / 32;            // stage-1 reduction steps
  static constexpr int KK = (N1 + 31) / 32;     // stage-2 reduction steps
  static constexpr bool KHALF = (N1 % 32) != 0;
  static constexpr int LPL = CB / 4;            // consecutive output columns per lane and row
  static constexpr int TPI = kWaves / WPT;      // tokens per workgroup iteration
  // prefetch the next token's tile while this one is computed: always with two waves
  // per token; with one wave per token only in the deep variant, which runs one wave
  // per SIMD so that the whole register file (VGPRs + AGPRs) is available
  static constexpr bool PREFETCH = WPT > 1 || DEEP;
  static constexpr int P2_BYTES = N2 * N2 * 2;
  static constexpr int P1_BYTES = KK * MT * 1024;
};

template <int N1, int N2, int WPT, bool HAS_C, bool DEEP>
__global__ __launch_bounds__(kThreads, DEEP ? 1 : 2) void kq_reg_kernel(
    const __bf16 *__restrict__ X, int64_t T, int64_t ldx,
    const bf16x8 *__restrict__ p2op, const bf16x8 *__restrict__ p1op,
    const float *__restrict__ cvec, float clip, int scale_fp16, int clip_allows_no_clamp,
    uint8_t *__restrict__ codes, void *__restrict__ scales, float *__restrict__ ydbg) {
  using C = RegCfg<N1, N2, WPT, HAS_C, DEEP>;
  constexpr int n = N1 * N2;
  __shared__ __align__(16) unsigned char s_p2[C::P2_BYTES];
  __shared__ __align__(16) unsigned char s_p1[C::P1_BYTES];
  __shared__ float s_red[2][kWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int lr = lane & 15;
  const int slot = wave / WPT;  // token slot within the iteration
  const int wb = wave % WPT;    // column block of this wave

  copy_to_lds(s_p2, p2op, C::P2_BYTES, tid);
  copy_to_lds(s_p1, p1op, C::P1_BYTES, tid);
  lds_barrier();
  const bf16x8 *sp2 = reinterpret_cast<const bf16x8 *>(s_p2) + wb * (C::KS * C::NT * 64);
  const bf16x8 *sp1 = reinterpret_cast<const bf16x8 *>(s_p1);

  // token tile as A operands: lane holds V[16 mt + lr][32 ks + 8 g + v] (raw bf16)
  uint4 a[C::MT][C::KS];
  auto load_tile = [&](int64_t tok) {
    const __bf16 *xt = X + tok * ldx;
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
        a[mt][ks] = tok < T ? *reinterpret_cast<const uint4 *>(xt + (mt * 16 + lr) * N2 + ks * 32 + g * 8)
                            : make_uint4(0u, 0u, 0u, 0u);
  };

  const int64_t ngroups = (T + C::TPI - 1) / C::TPI;
  int64_t grp = blockIdx.x;
  if (C::PREFETCH && grp < ngroups) load_tile(grp * C::TPI + slot);
  for (int it = 0; grp < ngroups; grp += gridDim.x, ++it) {
    const int64_t tok = grp * C::TPI + slot;
    if constexpr (!C::PREFETCH) load_tile(tok);
    // deep variant: the next tile goes to a second register set right away
    uint4 an[DEEP ? C::MT : 1][DEEP ? C::KS : 1];
    if constexpr (DEEP) {
      const int64_t nt_ = (grp + gridDim.x) * C::TPI + slot;
      const __bf16 *xt = X + nt_ * ldx;
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
          an[mt][ks] = nt_ < T ? *reinterpret_cast<const uint4 *>(xt + (mt * 16 + lr) * N2 + ks * 32 + g * 8)
                               : make_uint4(0u, 0u, 0u, 0u);
    }

    // ---- stage 1: Z[:, block] = V P2[:, block] (columns in the plan's permuted order) ----
    f32x4 zacc[C::MT][C::NT];
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) zacc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      bf16x8 ahi[C::MT], alo[HAS_C ? C::MT : 1];
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) {
        if constexpr (HAS_C) {
          const float *cp = cvec + (mt * 16 + lr) * N2 + ks * 32 + g * 8;
          const float4 c0 = *reinterpret_cast<const float4 *>(cp);
          const float4 c1 = *reinterpret_cast<const float4 *>(cp + 4);
          const float cc[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
          uint4 hi, lo;
          split_scaled(a[mt][ks], cc, hi, lo);
          ahi[mt] = __builtin_bit_cast(bf16x8, hi);
          alo[mt] = __builtin_bit_cast(bf16x8, lo);
        } else {
          ahi[mt] = __builtin_bit_cast(bf16x8, a[mt][ks]);
        }
      }
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) {
        const bf16x8 b = sp2[(ks * C::NT + nt) * 64 + lane];
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt) {
          zacc[mt][nt] = mfma(ahi[mt], b, zacc[mt][nt]);
          if constexpr (HAS_C) zacc[mt][nt] = mfma(alo[mt], b, zacc[mt][nt]);
        }
      }
    }
    // the tile is consumed: fetch the next one while this token finishes
    if constexpr (DEEP) {
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) a[mt][ks] = an[mt][ks];
    } else if constexpr (C::PREFETCH) {
      const int64_t nxt = grp + gridDim.x;
      if (nxt < ngroups) load_tile(nxt * C::TPI + slot);
    }

    // ---- stage 2: Y^T[block, :] = Z[:, block]^T P1 (M = CB, K = n1, N = n1) ----
    f32x4 yacc[C::NT][C::MT];
#pragma unroll
    for (int m2 = 0; m2 < C::NT; ++m2)
#pragma unroll
      for (int nt = 0; nt < C::MT; ++nt) yacc[m2][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      const bool pad = C::KHALF && kk == C::KK - 1;
      bf16x8 za[C::NT];
#pragma unroll
      for (int m2 = 0; m2 < C::NT; ++m2)
        za[m2] = pack8(zacc[2 * kk][m2], pad ? zero : zacc[(2 * kk + 1) % C::MT][m2]);
#pragma unroll
      for (int nt = 0; nt < C::MT; ++nt) {
        const bf16x8 b = sp1[(kk * C::MT + nt) * 64 + lane];
#pragma unroll
        for (int m2 = 0; m2 < C::NT; ++m2) yacc[m2][nt] = mfma(za[m2], b, yacc[m2][nt]);
      }
    }

    // ---- epilogue: lane holds Y[16 nt + lr][CB wb + LPL g + 4 m2 + r] ----
    float m = 0.f;
#pragma unroll
    for (int m2 = 0; m2 < C::NT; ++m2)
#pragma unroll
      for (int nt = 0; nt < C::MT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(yacc[m2][nt][r]));
    m = wave_max_uniform(m);
    if constexpr (WPT > 1) {
      // combine the partial absmax of the waves sharing the token (slots alternate per
      // iteration, so one barrier per token is enough)
      if (lane == 0) s_red[it & 1][wave] = m;
      lds_barrier();
#pragma unroll
      for (int w = 0; w < WPT; ++w) m = fmaxf(m, s_red[it & 1][slot * WPT + w]);
    }
    const TokenScale ts = token_scale(m, clip, scale_fp16);
    const bool clamp = __builtin_amdgcn_readfirstlane(clamp_needed(clip_allows_no_clamp, ts.s32) ? 1 : 0);

    if (tok < T) {
      uint8_t *crow = codes + tok * (int64_t)(n / 2);
#pragma unroll
      for (int nt = 0; nt < C::MT; ++nt) {
        const int j = nt * 16 + lr;
        uint32_t w[C::NT / 2];
#pragma unroll
        for (int q = 0; q < C::NT / 2; ++q) {
          const float yv[8] = {yacc[2 * q][nt][0],     yacc[2 * q][nt][1],
                               yacc[2 * q][nt][2],     yacc[2 * q][nt][3],
                               yacc[2 * q + 1][nt][0], yacc[2 * q + 1][nt][1],
                               yacc[2 * q + 1][nt][2], yacc[2 * q + 1][nt][3]};
          w[q] = clamp ? quant8<true>(yv, ts.inv) : quant8<false>(yv, ts.inv);
        }
        uint8_t *dst = crow + j * (N2 / 2) + wb * (C::CB / 2) + g * (C::LPL / 2);
        if constexpr (C::NT == 8) {
          *reinterpret_cast<uint4 *>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
        } else if constexpr (C::NT == 4) {
          *reinterpret_cast<uint2 *>(dst) = make_uint2(w[0], w[1]);
        } else {
          *reinterpret_cast<uint32_t *>(dst) = w[0];
        }
        if (ydbg != nullptr) {
          float4 *yp = reinterpret_cast<float4 *>(ydbg + tok * (int64_t)n + j * N2 + wb * C::CB +
                                                  g * C::LPL);
#pragma unroll
          for (int m2 = 0; m2 < C::NT; ++m2)
            yp[m2] = make_float4(yacc[m2][nt][0], yacc[m2][nt][1], yacc[m2][nt][2], yacc[m2][nt][3]);
        }
      }
      if (wb == 0 && lane == 0) store_scale(scales, tok, ts, scale_fp16);
    }
  }
}

// ------------------------------------------------------------------------------------
// stream kernel: one wave per token, next token prefetched into LDS by DMA
// ------------------------------------------------------------------------------------
// Eight waves per workgroup (two per SIMD, one workgroup per CU). Each wave owns an LDS
// slot of one token tile; while it computes token t, a global->LDS DMA
// (global_load_lds_dwordx4: lane i's 16 bytes land at slot + 16 i) brings its next token
// into the slot, so the load costs no registers and no barrier: a wave only ever waits
// for its own DMA. Every DMA instruction reads 1 KiB of contiguous global memory (whole
// rows of V); the 16-byte pieces of row R are permuted within the row (piece P stored
// at position P ^ swz(R)), which makes the A-operand reads of a 16-row tile hit 16
// different bank groups. The next token's DMA is issued as soon as stage 1 has read the
// slot. P2 operands stay in LDS (shared, read-only), P1 operands in registers. The code
// stores of a token are issued after the wait for the next token's tile, so that wait
// never covers a just-issued store.
template <int N1, int N2, bool HAS_C = false>
struct StreamCfg {
  static_assert(N1 % 16 == 0 && N1 >= 16 && N1 <= 64, "stream kernel: n1 in {16, 32, 48, 64}");
  static_assert(N2 == 64 || N2 == 128, "stream kernel: n2 in {64, 128}");
  // with a per-channel scale the A operands are split into bf16 hi + lo words, which
  // only leaves registers for it when a token's Y tile is at most 64 x 64
  static_assert(!HAS_C || N2 == 64, "stream kernel with c: n2 = 64");
  static constexpr int WAVES = 8;
  static constexpr int THREADS = WAVES * 64;  // the kernel's launch bound
  static constexpr int MT = N1 / 16;
  static constexpr int NT = N2 / 16;
  static constexpr int KS = N2 / 32;
  static constexpr int KK = (N1 + 31) / 32;
  static constexpr bool KHALF = (N1 % 32) != 0;
  static constexpr int LPL = N2 / 4;            // consecutive output columns per lane and row
  static constexpr int TILE = N1 * N2 * 2;      // bytes of one token
  static constexpr int P2_BYTES = N2 * N2 * 2;
  static constexpr int C_BYTES = HAS_C ? N1 * N2 * 4 : 0;  // c (fp32), swizzled rows
  // with c, P1's operands live in LDS too (one copy per CU instead of one per wave: with
  // one token per wave, the per-wave copies would cost as much L2 traffic as the tokens)
  static constexpr int P1_BYTES = HAS_C ? KK * MT * 1024 : 0;
  static_assert(P2_BYTES + C_BYTES + P1_BYTES + WAVES * TILE <= 160 * 1024, "LDS budget");
  static constexpr int RB = N2 * 2;             // bytes per row of V
  static constexpr int PPR = RB / 16;           // 16-byte pieces per row
  static constexpr int RPB = 256 / RB;          // rows per 256-byte bank row
  static constexpr int RPI = 1024 / RB;         // rows per DMA instruction
  static constexpr int LOADS = TILE / 1024;     // DMA instructions per token
  // position permutation of row R's pieces (an xor, so its own inverse)
  __device__ static constexpr int swz(int R) { return (R / RPB) % PPR; }
};

// Cache policy of the streaming accesses: every input byte is read once and every code
// byte written once, so both go non-temporal ("nt"), which keeps them from displacing
// each other in the caches (measured on MI355X: read 16 KiB + write 4 KiB per token
// streams about 12% faster than with the default policy).

// INT8 codes of a wave's Y tile (lane holds yacc[m2][nt] = 4 consecutive columns of row
// 16 nt + lr): w[nt][m2] holds those 4 values as bytes.
template <int MT, int NT>
__device__ __forceinline__ void quant_tile8(const f32x4 (&yacc)[NT][MT], float inv,
                                            uint32_t (&w)[MT][NT]) {
#pragma unroll
  for (int nt = 0; nt < MT; ++nt)
#pragma unroll
    for (int m2 = 0; m2 < NT; ++m2)
      w[nt][m2] = quant4x8(yacc[m2][nt][0], yacc[m2][nt][1], yacc[m2][nt][2], yacc[m2][nt][3], inv);
}

// INT8 code rows: lane stores 4 NT bytes (its LPL consecutive columns) of row 16 nt + lr.
// Each store instruction fills half of every 32-byte piece of a row and the next one the
// other half; plain stores let L2 merge the halves before they go to HBM (non-temporal
// stores wrote 14 % more bytes than the codes hold).
template <int N1, int N2>
__device__ __forceinline__ void store_codes8(uint8_t *codes, int64_t tok,
                                             const uint32_t (*w)[N2 / 16], int lr, int g) {
  uint8_t *crow = codes + tok * (int64_t)(N1 * N2);
#pragma unroll
  for (int nt = 0; nt < N1 / 16; ++nt) {
    uint8_t *dst = crow + (nt * 16 + lr) * N2 + g * (N2 / 4);
#pragma unroll
    for (int q = 0; q < N2 / 64; ++q) {
      const u32x4_t v = {w[nt][4 * q], w[nt][4 * q + 1], w[nt][4 * q + 2], w[nt][4 * q + 3]};
      *reinterpret_cast<u32x4_t *>(dst + 16 * q) = v;
    }
  }
}

// N2R < N2: rows of X (and of Y and the codes) hold N2R values; the tile in LDS keeps the
// N2 layout, its padding pieces meet P2's zero rows (see dma_tile) and padded columns of
// Y are zero and not stored
// With c (HAS_C), both contractions run on fp16 operands: x^ = fp16(fp32(x c) 2^sx), where
// the token's bound max|x| max|c| picks sx (f16_scale_exp; 0 for ordinary tokens); P2 and
// P1 come from the plan as fp16 operands scaled by 2^-f2 and 2^-f1 (f_exp = f1 + f2); the
// token's largest |Z| picks sz for Z's conversion; Y = Y' 2^(f_exp - sx - sz) exactly.
template <int N1, int N2, bool HAS_C, bool YDBG, int BITS = 4, int N2R = N2>
__global__ __launch_bounds__(512) void kq_stream_kernel(
    const __bf16 *__restrict__ X, int64_t T, int64_t ldx,
    const bf16x8 *__restrict__ p2op, const bf16x8 *__restrict__ p1op,
    const float *__restrict__ cvec, int f_exp, float cmax, float clip, int scale_fp16,
    int clip_allows_no_clamp, uint8_t *__restrict__ codes, void *__restrict__ scales,
    float *__restrict__ ydbg) {
  using C = StreamCfg<N1, N2, HAS_C>;
  static_assert(N2R == N2 || (N2 == 128 && N2R == 112 && !HAS_C && BITS == 4), "padded rows");
  constexpr int n = N1 * N2R;
  // P2 operands, then (with c) c as 16-byte units of 4 channels: unit u of row R at
  // R * 4 N2 + ((u ^ (R % 16)) * 16), so that the 16 rows of one A-operand read hit 16
  // different bank groups
  __shared__ __align__(16) unsigned char s_p2[C::P2_BYTES + C::C_BYTES + C::P1_BYTES];
  unsigned char *const s_c = s_p2 + C::P2_BYTES;
  unsigned char *const s_p1 = s_c + C::C_BYTES;
  __shared__ __align__(16) unsigned char s_tile[C::WAVES][C::TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g = lane >> 4;
  const int lr = lane & 15;

  unsigned char *slot = s_tile[wave];

  // DMA token `tok` into this wave's slot: instruction j fills slot bytes [1024 j, 1024 j
  // + 1024) = rows [RPI j, RPI j + RPI); lane i lands at row R = RPI j + i / PPR, position
  // i % PPR, so it reads piece (i % PPR) ^ swz(R) of that row.
  // The lane's byte offset within instruction j's 1 KiB depends on j only through
  // swz(R), which repeats every SWP instructions: SWP offsets per lane.
  constexpr int SWP = C::PPR * C::RPB / C::RPI;  // swz period in instructions
  static_assert(SWP >= 1 && C::LOADS % SWP == 0, "swizzle period");
  uint32_t voff[SWP];
  {
    const int r0 = lane / C::PPR, pos0 = lane % C::PPR;
#pragma unroll
    for (int j = 0; j < SWP; ++j) {
      const int R = j * C::RPI + r0;
      // rows of X hold N2R values: a padding piece (>= N2R / 8) reads the row's first
      // piece instead, finite values that meet P2's zero rows
      const int piece = pos0 ^ C::swz(R);
      voff[j] = (uint32_t)((r0 * N2R + ((piece < N2R / 8 ? piece : 0) * 8)) * 2);
    }
  }
  auto dma_tile = [&](int64_t tok) {
    const unsigned char *xt = reinterpret_cast<const unsigned char *>(X + tok * ldx);
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j)  // swz(R + SWP RPI) == swz(R)
      dma16_nt(xt + j * (C::RPI * N2R * 2), voff[j % SWP], lds_addr(slot + j * 1024));
  };

  const int64_t stride = (int64_t)gridDim.x * C::WAVES;
  int64_t tok = (int64_t)blockIdx.x * C::WAVES + wave;
  bf16x8 p1r[HAS_C ? 1 : C::KK][HAS_C ? 1 : C::MT];  // stage-2 B operands, resident (no c)
  if constexpr (!HAS_C) {
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk)
#pragma unroll
      for (int nt = 0; nt < C::MT; ++nt) p1r[kk][nt] = p1op[(kk * C::MT + nt) * 64 + lane];
  } else {
    dma_copy(p1op, s_p1, C::P1_BYTES, wave, C::WAVES, lane);
  }
  // P2's operands (and c) reach LDS by DMA, each wave copying its share, before any token
  dma_copy(p2op, s_p2, C::P2_BYTES, wave, C::WAVES, lane);
  if constexpr (HAS_C) {
    // c in 16-byte units of 4 channels, unit u of row R at R * 4 N2 + ((u ^ (R % 16)) * 16):
    // lane i of instruction j lands at LDS byte b = 1024 j + 16 i of that layout, i.e. row
    // b / (4 N2), position p = (b % (4 N2)) / 16, and reads unit p ^ (row % 16)
    const unsigned char *csrc = reinterpret_cast<const unsigned char *>(cvec);
    for (int j = wave; j < C::C_BYTES / 1024; j += C::WAVES) {
      const int b = j * 1024 + lane * 16;
      const int R = b / (4 * N2), pos = (b % (4 * N2)) / 16;
      dma16<false>(csrc, (uint32_t)(R * 4 * N2 + ((pos ^ (R % 16)) * 16)), lds_addr(s_c + j * 1024));
    }
  }
  // The first half of the waves issues its token's DMA at once and waits for it before the
  // barrier; the second half issues its own only after the barrier, i.e. once the first
  // half's tokens have landed. The first tokens then arrive sooner and half the CU computes
  // while the rest load (measured on MI355X: 6 % on 2048 fp32 tokens of 64x64, 0.5 % on
  // 16384 tokens of 64x128, neutral on 2048 tokens with c).
  if (wave < C::WAVES / 2) {
    if (tok < T) dma_tile(tok);
    wait_and_fence<kWaitVm0>();
    lds_barrier();  // P2 (and c) visible to every wave
  } else {
    wait_and_fence<kWaitVm0>();
    lds_barrier();  // P2 (and c) visible to every wave
    if (tok < T) dma_tile(tok);
  }
  const bf16x8 *sp2 = reinterpret_cast<const bf16x8 *>(s_p2);

  // codes of the previous token, stored one step late (8 or 4 values per dword)
  uint32_t pend[C::MT][BITS == 4 ? C::NT / 2 : C::NT];
  TokenScale pend_s{0.f, (_Float16)0.f, 0.f};
  int64_t pend_tok = -1;
  auto store_pending = [&]() {
    if constexpr (BITS == 4) store_codes<N1, N2, N2R>(codes, pend_tok, pend, lr, g);
    else store_codes8<N1, N2>(codes, pend_tok, pend, lr, g);
    if (lane == 0) store_scale(scales, pend_tok, pend_s, scale_fp16);
  };

  for (; tok < T; tok += stride) {
    wait_and_fence<kWaitVm0>();  // this token's tile (and older stores) have landed
    if (pend_tok >= 0) store_pending();
    // The two waves of a SIMD alternate between MFMA-heavy stages and the VALU-heavy
    // quantizer: a higher issue priority for the MFMA phase keeps the matrix core fed
    // while the other wave's VALU work fills the gaps (measured on MI355X: about 2 %).
    __builtin_amdgcn_s_setprio(1);
    constexpr int NH = C::NT / 2;  // column tiles per half
    f32x4 yacc[C::NT][C::MT];
    float pm[C::NT];
    int ty = 0;  // with c: Y = yacc 2^ty
    if constexpr (HAS_C) {
      // ---- the token's x, its bound max|x| max|c| and the scale of x^ ----
      uint4 raw[C::KS][C::MT];
      uint32_t xm = 0;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const unsigned char *arow = slot + lr * C::RB + (((ks * 4 + g) ^ C::swz(lr)) * 16);
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt) {
          raw[ks][mt] = *reinterpret_cast<const uint4 *>(arow + mt * 16 * C::RB);
          xm = absmax_bf16(raw[ks][mt], xm);
        }
      }
      const float xmax = wave_max_uniform(__uint_as_float(xm << 16));
      const int sx = __builtin_amdgcn_readfirstlane(f16_scale_exp(__fmul_rn(xmax, cmax)));
      // ---- stage 1 over all column tiles: Z' = x^ P2' on fp16 operands ----
      f32x4 zacc[C::MT][C::NT];
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) zacc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      // sx is wave-uniform: tokens that need no scaling (the usual case) take the
      // branch without the ldexp
      auto stage1 = [&](auto scale) {
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          f16x8 av[C::MT];
#pragma unroll
          for (int mt = 0; mt < C::MT; ++mt) {
            const unsigned char *crow = s_c + (mt * 16 + lr) * (N2 * 4);
            const int u0 = (ks * 4 + g) * 2;
            const float4 c0 = *reinterpret_cast<const float4 *>(crow + ((u0 ^ lr) * 16));
            const float4 c1 = *reinterpret_cast<const float4 *>(crow + (((u0 + 1) ^ lr) * 16));
            const float cc[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
            av[mt] = scale_round_f16<decltype(scale)::value>(raw[ks][mt], cc, sx);
          }
#pragma unroll
          for (int nt = 0; nt < C::NT; ++nt) {
            const f16x8 bv = reinterpret_cast<const f16x8 *>(sp2)[(ks * C::NT + nt) * 64 + lane];
#pragma unroll
            for (int mt = 0; mt < C::MT; ++mt) zacc[mt][nt] = mfma_f16(av[mt], bv, zacc[mt][nt]);
          }
        }
      };
      if (sx == 0) stage1(std::false_type{});
      else stage1(std::true_type{});
      wait_and_fence<kWaitLgkm0>();  // every slot read has returned: the slot is free again
      if (tok + stride < T) dma_tile(tok + stride);
      float zm = 0.f;
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) zm = absmax_acc(zacc[mt], zm);
      const int zs = __builtin_amdgcn_readfirstlane(f16_scale_exp(wave_max_uniform(zm)));
      // ---- stage 2 on fp16 operands: Y^T = Z^T P1 ----
#pragma unroll
      for (int m2 = 0; m2 < C::NT; ++m2)
#pragma unroll
        for (int nt = 0; nt < C::MT; ++nt) yacc[m2][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk) {
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        const bool pad = C::KHALF && kk == C::KK - 1;
        f16x8 za[C::NT];
#pragma unroll
        for (int m2 = 0; m2 < C::NT; ++m2)
          za[m2] = pack8_f16(zacc[2 * kk][m2], pad ? zero : zacc[(2 * kk + 1) % C::MT][m2], zs);
#pragma unroll
        for (int nt = 0; nt < C::MT; ++nt) {
          const f16x8 b = reinterpret_cast<const f16x8 *>(s_p1)[(kk * C::MT + nt) * 64 + lane];
#pragma unroll
          for (int m2 = 0; m2 < C::NT; ++m2) yacc[m2][nt] = mfma_f16(za[m2], b, yacc[m2][nt]);
        }
      }
      ty = f_exp - sx - zs;  // Y = Y' 2^(f1 + f2 - sx - sz), exact
      // maxima of |Y'|: ldexp is monotone, so max|Y| is the scaled maximum
#pragma unroll
      for (int m2 = 0; m2 < C::NT; ++m2) pm[m2] = absmax_acc(yacc[m2], 0.f);
    } else {
    // ---- stages 1 and 2 per half of the output columns ----
    // A column tile of Y needs only the same column tile of Z, so each half runs stage 1
    // (Z = V P2 for its columns) and stage 2 (Y^T = Z^T P1) on its own: only half of
    // the stage-1 accumulators are ever live, which leaves registers to fetch operands
    // ahead, and the first half's absmax overlaps the second half's MFMAs.
    // A operand (mt, ks) of lane L: V[16 mt + lr][32 ks + 8 g + v], i.e. piece 4 ks + g
    // of row 16 mt + lr.
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 zacc[C::MT][NH];
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NH; ++nt) zacc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const unsigned char *arow = slot + lr * C::RB + (((ks * 4 + g) ^ C::swz(lr)) * 16);
        bf16x8 av[C::MT], bv[NH];
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)  // swz(16 mt + lr) == swz(lr)
          av[mt] = *reinterpret_cast<const bf16x8 *>(arow + mt * 16 * C::RB);
#pragma unroll
        for (int nt = 0; nt < NH; ++nt) bv[nt] = sp2[(ks * C::NT + h * NH + nt) * 64 + lane];
#pragma unroll
        for (int nt = 0; nt < NH; ++nt)
#pragma unroll
          for (int mt = 0; mt < C::MT; ++mt) zacc[mt][nt] = mfma(av[mt], bv[nt], zacc[mt][nt]);
      }
      if (h == 1) {
        wait_and_fence<kWaitLgkm0>();  // every slot read has returned: the slot is free again
        if (tok + stride < T) dma_tile(tok + stride);
      }
      bf16x8 za[C::KK][NH];
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk) {
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        const bool pad = C::KHALF && kk == C::KK - 1;
#pragma unroll
        for (int m2 = 0; m2 < NH; ++m2)
          za[kk][m2] = pack8(zacc[2 * kk][m2], pad ? zero : zacc[(2 * kk + 1) % C::MT][m2]);
      }
#pragma unroll
      for (int m2 = 0; m2 < NH; ++m2)
#pragma unroll
        for (int nt = 0; nt < C::MT; ++nt) yacc[h * NH + m2][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk)
#pragma unroll
        for (int nt = 0; nt < C::MT; ++nt)
#pragma unroll
          for (int m2 = 0; m2 < NH; ++m2)
            yacc[h * NH + m2][nt] = mfma(za[kk][m2], p1r[kk][nt], yacc[h * NH + m2][nt]);
      // partial absmax of this half (independent chains, one per column tile)
#pragma unroll
      for (int m2 = h * NH; m2 < (h + 1) * NH; ++m2) pm[m2] = absmax_acc(yacc[m2], 0.f);
    }
    }  // !HAS_C

    __builtin_amdgcn_s_setprio(0);
    // ---- epilogue: lane holds Y[16 nt + lr][LPL g + 4 m2 + r] ----
#pragma unroll
    for (int w = C::NT / 2; w >= 1; w /= 2)
#pragma unroll
      for (int i = 0; i < w; ++i) pm[i] = max_nn(pm[i], pm[i + w]);
    const float m = pm[0];
    // the absmax and the clamp decision are wave-uniform: broadcast them so that the
    // choice below is one scalar branch, not a per-lane select
    const float amax = HAS_C ? __builtin_ldexpf(wave_max_uniform(m), ty) : wave_max_uniform(m);
    const TokenScale ts = token_scale(amax, clip, scale_fp16, BITS == 4 ? 7.0f : 127.0f);
    // with c: codes straight from Y' with the reciprocal scaled by 2^ty where that is
    // exact, else from Y = ldexp(Y', ty) (then ty = 0: yacc holds Y)
    float inv = ts.inv;
    if constexpr (HAS_C) {
      if (!__builtin_amdgcn_readfirstlane(fold_scale(ts.inv, ty, amax, inv) ? 1 : 0)) {
#pragma unroll
        for (int m2 = 0; m2 < C::NT; ++m2)
#pragma unroll
          for (int nt = 0; nt < C::MT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) yacc[m2][nt][r] = __builtin_ldexpf(yacc[m2][nt][r], ty);
        inv = ts.inv;
        ty = 0;
      }
    }
    if constexpr (BITS == 8) {
      quant_tile8<C::MT, C::NT>(yacc, inv, pend);
    } else if (__builtin_amdgcn_readfirstlane(clamp_needed(clip_allows_no_clamp, ts.s32) ? 1 : 0)) {
      quant_tile<true, C::MT, C::NT>(yacc, inv, pend);
    } else {
      quant_tile<false, C::MT, C::NT>(yacc, inv, pend);
    }
    pend_s = ts;
    pend_tok = tok;
    if constexpr (YDBG) {
#pragma unroll
      for (int nt = 0; nt < C::MT; ++nt) {
        float4 *yp = reinterpret_cast<float4 *>(ydbg + tok * (int64_t)n + (nt * 16 + lr) * N2R + g * C::LPL);
#pragma unroll
        for (int m2 = 0; m2 < C::NT; ++m2)
          if (g * C::LPL + 4 * m2 < N2R)  // padded columns are not written
            yp[m2] = make_float4(__builtin_ldexpf(yacc[m2][nt][0], ty), __builtin_ldexpf(yacc[m2][nt][1], ty),
                                 __builtin_ldexpf(yacc[m2][nt][2], ty), __builtin_ldexpf(yacc[m2][nt][3], ty));
      }
    }
  }
  if (pend_tok >= 0) store_pending();
}

// ------------------------------------------------------------------------------------
// row-split kernel with c (n2 = 64): a token's rows spread over n1/16 waves
// ------------------------------------------------------------------------------------
// For batches of a few thousand tokens the stream kernel has one token per wave, and the
// token's whole conversion, both contractions and the quantizer run as one serial chain
// in that wave. Here a workgroup of MT = n1/16 waves takes a token, wave w its rows
// 16 w .. 16 w + 15:
//  * stage 1 is row-wise: the wave converts and multiplies only its own rows, with c for
//    those rows held in registers; the token's bound max|x| max|c| (for x^'s scale 2^sx)
//    meets at barrier 0;
//  * Z crosses the waves through LDS, rounded to fp16 after the scale 2^zs from the
//    token's largest |Z'| (barrier 1); stage 2 starts after barrier 2;
//  * stage 2 gives wave w rows 16 w .. 16 w + 15 of Y; the absmax meets at barrier 3
//    and every wave quantizes and stores its rows.
// The roundings, scales and MFMA order are the stream kernel's, so a token gets the same
// codes from both (a plan may use either, by batch size). Each wave DMAs its own rows of
// the next token into its part of the slot as soon as it has read the current ones (no
// other wave reads them), so the loads overlap the rest of the token.
template <int N1>
struct RsplitCfg {
  static_assert(N1 % 16 == 0 && N1 >= 16 && N1 <= 64, "row-split kernel: n1 in {16, 32, 48, 64}");
  static constexpr int N2 = 64;
  static constexpr int MT = N1 / 16;            // waves per token (16-row blocks)
  static constexpr int THREADS = MT * 64;
  static constexpr int KS = N2 / 32;            // stage-1 reduction steps
  static constexpr int NT = N2 / 16;            // column tiles
  static constexpr int KK = (MT + 1) / 2;       // stage-2 reduction steps (32 rows each)
  static constexpr int RB = N2 * 2;             // bytes per row of X
  static constexpr int WROWS = 16 * RB;         // bytes of a wave's rows (2 KiB)
  static constexpr int ZBYTES = NT * KK * 64 * 16;  // Z exchange: [a][kk][lane] 16 bytes
};

template <int N1, bool YDBG = false>
__global__ __launch_bounds__(RsplitCfg<N1>::THREADS) void kq_rsplit_kernel(
    const __bf16 *__restrict__ X, int64_t T, int64_t ldx,
    const f16x8 *__restrict__ p2op, const f16x8 *__restrict__ p1op,
    const float *__restrict__ cvec, int f_exp, float cmax, float clip, int scale_fp16,
    int clip_allows_no_clamp, uint8_t *__restrict__ codes, void *__restrict__ scales,
    float *__restrict__ ydbg) {
  using C = RsplitCfg<N1>;
  constexpr int N2 = C::N2;
  constexpr int n = N1 * N2;
  // the token's rows (each wave DMAs and reads only its own 16), and Z's exchange area:
  // for stage-2 step kk and column tile a, lane L's 16 bytes are the 4 fp16 values of
  // lane L of wave 2 kk (rows 32 kk + 4 g + r) then those of wave 2 kk + 1 (rows + 16):
  // exactly the stage-2 A operand of lane L, in the slot order of P1's operands
  __shared__ __align__(16) unsigned char s_tile[C::MT * C::WROWS];
  __shared__ __align__(16) unsigned char s_z[C::ZBYTES];
  __shared__ float s_xm[2][C::MT];
  __shared__ float s_zm[2][C::MT];
  __shared__ float s_ym[2][C::MT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // this wave's 16-row block
  const int g = lane >> 4;
  const int lr = lane & 15;
  unsigned char *rows = s_tile + w * C::WROWS;

  // DMA of the wave's rows of token `tok`: instruction j fills rows 8 j .. 8 j + 7 of the
  // block; lane i lands at row R = 8 j + i / 8, position i % 8 of that row, so it reads
  // piece (i % 8) ^ ((R / 2) % 8): the 16 rows of an operand read then fall in 16
  // different bank groups
  uint32_t voff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int R = 8 * j + lane / 8;
    voff[j] = (uint32_t)(((16 * w + R) * N2 + (((lane % 8) ^ ((R / 2) % 8)) * 8)) * 2);
  }
  auto dma_rows = [&](int64_t tok) {
    const unsigned char *xt = reinterpret_cast<const unsigned char *>(X + tok * ldx);
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16_nt(xt, voff[j], lds_addr(rows + j * 1024));
  };
  int64_t tok = blockIdx.x;
  if (tok < T) dma_rows(tok);

  // operands in registers for the whole kernel: P2 (stage-1 B, all column tiles), P1
  // (stage-2 B, this wave's output rows), and c for the lane's 16 channels
  f16x8 p2w[C::KS][C::NT], p1w[C::KK];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
    for (int a = 0; a < C::NT; ++a) p2w[ks][a] = p2op[(ks * C::NT + a) * 64 + lane];
#pragma unroll
  for (int kk = 0; kk < C::KK; ++kk) p1w[kk] = p1op[(kk * C::MT + w) * 64 + lane];
  float cl[C::KS][8];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const float4 *cp = reinterpret_cast<const float4 *>(cvec + (16 * w + lr) * N2 + 32 * ks + 8 * g);
    const float4 u = cp[0], v = cp[1];
    cl[ks][0] = u.x; cl[ks][1] = u.y; cl[ks][2] = u.z; cl[ks][3] = u.w;
    cl[ks][4] = v.x; cl[ks][5] = v.y; cl[ks][6] = v.z; cl[ks][7] = v.w;
  }
  if constexpr (C::MT % 2 == 1) {  // the absent last block's half of Z stays zero
    for (int i = tid; i < C::ZBYTES / 16; i += C::THREADS)
      reinterpret_cast<uint4 *>(s_z)[i] = make_uint4(0u, 0u, 0u, 0u);
  }

  for (int it = 0; tok < T; tok += gridDim.x, ++it) {
    const int par = it & 1;
    // this token's rows have landed: at least one store (the codes) was issued after the
    // last DMA, so waiting for all but one vector-memory operation covers the DMA
    wait_and_fence<wait_vm_imm(1)>();
    uint4 raw[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      raw[ks] = *reinterpret_cast<const uint4 *>(rows + lr * C::RB + (((4 * ks + g) ^ ((lr / 2) % 8)) * 16));
    wait_and_fence<kWaitLgkm0>();  // the rows are read: the next token's may come in
    if (tok + gridDim.x < T) dma_rows(tok + gridDim.x);

    // ---- stage 1 on the wave's rows: Z' = x^ P2' ----
    uint32_t xm = 0;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) xm = absmax_bf16(raw[ks], xm);
    const float xmw = wave_max_uniform(__uint_as_float(xm << 16));
    if (lane == 0) s_xm[par][w] = xmw;
    lds_barrier();  // (0) every block's |x| maximum is published
    float xmax = 0.f;
#pragma unroll
    for (int v = 0; v < C::MT; ++v) xmax = max_nn(xmax, s_xm[par][v]);
    const int sx = __builtin_amdgcn_readfirstlane(f16_scale_exp(__fmul_rn(xmax, cmax)));
    f16x8 av[C::KS];
    if (sx == 0) {
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) av[ks] = scale_round_f16<false>(raw[ks], cl[ks], 0);
    } else {
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) av[ks] = scale_round_f16<true>(raw[ks], cl[ks], sx);
    }
    f32x4 zacc[C::NT];
#pragma unroll
    for (int a = 0; a < C::NT; ++a) {
      zacc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) zacc[a] = mfma_f16(av[ks], p2w[ks][a], zacc[a]);
    }
    const float zm = wave_max_uniform(absmax_acc(zacc, 0.f));
    if (lane == 0) s_zm[par][w] = zm;
    lds_barrier();  // (1) every block's |Z'| maximum is published
    float zmax = 0.f;
#pragma unroll
    for (int v = 0; v < C::MT; ++v) zmax = max_nn(zmax, s_zm[par][v]);
    const int zs = __builtin_amdgcn_readfirstlane(f16_scale_exp(zmax));
#pragma unroll
    for (int a = 0; a < C::NT; ++a) {
      _Float16 h[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) h[r] = (_Float16)(zs == 0 ? zacc[a][r] : __builtin_ldexpf(zacc[a][r], zs));
      *reinterpret_cast<u32x2_t *>(s_z + ((a * C::KK + w / 2) * 64 + lane) * 16 + (w % 2) * 8) =
          __builtin_bit_cast(u32x2_t, h);
    }
    lds_barrier();  // (2) Z is complete in LDS

    // ---- stage 2: Y'^T[:, rows of block w] = Z^T P1'[:, rows of block w] ----
    f32x4 yacc[C::NT];
#pragma unroll
    for (int a = 0; a < C::NT; ++a) yacc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk)
#pragma unroll
      for (int a = 0; a < C::NT; ++a) {
        const f16x8 za = *reinterpret_cast<const f16x8 *>(s_z + ((a * C::KK + kk) * 64 + lane) * 16);
        yacc[a] = mfma_f16(za, p1w[kk], yacc[a]);
      }
    const int ty = f_exp - sx - zs;  // Y = Y' 2^(f1 + f2 - sx - sz), exact
    const float ym = wave_max_uniform(absmax_acc(yacc, 0.f));
    if (lane == 0) s_ym[par][w] = ym;
    lds_barrier();  // (3) every block's |Y'| maximum is published
    float amax_y = 0.f;
#pragma unroll
    for (int v = 0; v < C::MT; ++v) amax_y = max_nn(amax_y, s_ym[par][v]);
    const float amax = __builtin_ldexpf(amax_y, ty);
    const TokenScale sc = token_scale(amax, clip, scale_fp16);
    float inv_y;
    int ty_dbg = ty;
    if (!__builtin_amdgcn_readfirstlane(fold_scale(sc.inv, ty, amax, inv_y) ? 1 : 0)) {
#pragma unroll
      for (int a = 0; a < C::NT; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) yacc[a][r] = __builtin_ldexpf(yacc[a][r], ty);
      inv_y = sc.inv;
      ty_dbg = 0;
    }
    // lane holds Y[16 w + lr][16 g + 4 a + r]: 16 consecutive codes of its row, 8 bytes
    const float y0[8] = {yacc[0][0], yacc[0][1], yacc[0][2], yacc[0][3],
                         yacc[1][0], yacc[1][1], yacc[1][2], yacc[1][3]};
    const float y1[8] = {yacc[2][0], yacc[2][1], yacc[2][2], yacc[2][3],
                         yacc[3][0], yacc[3][1], yacc[3][2], yacc[3][3]};
    u32x2_t cw;
    if (__builtin_amdgcn_readfirstlane(clamp_needed(clip_allows_no_clamp, sc.s32) ? 1 : 0)) {
      cw = u32x2_t{quant8<true>(y0, inv_y), quant8<true>(y1, inv_y)};
    } else {
      cw = u32x2_t{quant8<false>(y0, inv_y), quant8<false>(y1, inv_y)};
    }
    const int row = 16 * w + lr;
    __builtin_nontemporal_store(
        cw, reinterpret_cast<u32x2_t *>(codes + tok * (int64_t)(n / 2) + row * (N2 / 2) + g * 8));
    if (w == 0 && lane == 0) store_scale(scales, tok, sc, scale_fp16);
    if constexpr (YDBG) {
      float4 *yp = reinterpret_cast<float4 *>(ydbg + tok * (int64_t)n + row * N2 + 16 * g);
#pragma unroll
      for (int a = 0; a < C::NT; ++a)
        yp[a] = make_float4(__builtin_ldexpf(yacc[a][0], ty_dbg), __builtin_ldexpf(yacc[a][1], ty_dbg),
                            __builtin_ldexpf(yacc[a][2], ty_dbg), __builtin_ldexpf(yacc[a][3], ty_dbg));
    }
  }
}

// ------------------------------------------------------------------------------------
// pair kernel: a workgroup of two waves per token, each wave one half of the columns
// ------------------------------------------------------------------------------------
// A column half of Y needs only the same column half of Z (stage 2 mixes rows, not
// columns), so wave h computes Z[:, half h] = V P2[:, half h] and Y[:, half h] = P1^T of
// it with both operand sets resident in registers: P2's half (its stage-1 B operands)
// and P1 (stage-2 B operands). Only V comes from LDS, read by both waves. The token tile
// is double-buffered: each wave DMAs one half of a tile (whole 128-byte row pieces, in
// the A-operand lane order) two tokens ahead. Two barriers per token, between the two
// waves of the pair only: "tile landed" and "tile read + absmax half exchanged"; the
// buffer is refilled right after the second one. Four pairs share a CU, one wave of two
// pairs per SIMD, so the MFMA work of one pair overlaps the waits of another.
template <int N1, int N2>
struct PairCfg {
  static_assert(N1 % 16 == 0 && N1 >= 16 && N1 <= 64, "pair kernel: n1 in {16, 32, 48, 64}");
  static_assert(N2 == 64 || N2 == 128, "pair kernel: n2 in {64, 128}");
  static constexpr int THREADS = 128;
  static constexpr int MT = N1 / 16;            // row tiles of V / Z
  static constexpr int CB = N2 / 2;             // output columns per wave
  static constexpr int NH = CB / 16;            // column tiles per wave
  static constexpr int KS = N2 / 32;            // stage-1 reduction steps
  static constexpr int KK = (N1 + 31) / 32;     // stage-2 reduction steps
  static constexpr bool KHALF = (N1 % 32) != 0;
  static constexpr int LPL = CB / 4;            // consecutive output columns per lane and row
  static constexpr int TILE = N1 * N2 * 2;      // bytes of one token
  static constexpr int CHUNKS = MT * KS;        // 1 KiB DMA chunks per tile
  static constexpr int HALF_LOADS = CHUNKS / 2; // DMA instructions per wave and tile
  static_assert(CHUNKS % 2 == 0 && HALF_LOADS < 64, "vmcnt range");
  static constexpr int kWaitHalf = 0x0F70 | (HALF_LOADS & 15) | ((HALF_LOADS >> 4) << 14);
};

// lane's LPL consecutive codes of each of its rows: LPL / 2 bytes (INT4) or LPL bytes (INT8)
template <int N1, int N2, int BITS = 4>
__device__ __forceinline__ void store_codes_half(uint8_t *codes, int64_t tok, int wave,
                                                 const uint32_t (*w)[BITS == 4 ? N2 / 64 : N2 / 32],
                                                 int lr, int g) {
  using C = PairCfg<N1, N2>;
  if constexpr (BITS == 8) {
    uint8_t *crow = codes + tok * (int64_t)(N1 * N2) + wave * C::CB + g * C::LPL;
#pragma unroll
    for (int nt = 0; nt < C::MT; ++nt) {
      uint8_t *dst = crow + (nt * 16 + lr) * N2;
      if constexpr (N2 == 128) {
        const u32x4_t v = {w[nt][0], w[nt][1], w[nt][2], w[nt][3]};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(dst));
      } else {
        const u32x2_t v = {w[nt][0], w[nt][1]};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t *>(dst));
      }
    }
    return;
  }
  uint8_t *crow = codes + tok * (int64_t)(N1 * N2 / 2) + wave * (C::CB / 2) + g * (C::LPL / 2);
#pragma unroll
  for (int nt = 0; nt < C::MT; ++nt) {
    uint8_t *dst = crow + (nt * 16 + lr) * (N2 / 2);
    if constexpr (N2 == 128) {
      const u32x2_t v = {w[nt][0], w[nt][1]};
      __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t *>(dst));
    } else {
      __builtin_nontemporal_store(w[nt][0], reinterpret_cast<uint32_t *>(dst));
    }
  }
}

template <int N1, int N2, bool YDBG, int BITS = 4>
__global__ __launch_bounds__(128, 2) void kq_pair_kernel(
    const __bf16 *__restrict__ X, int64_t T, int64_t ldx,
    const bf16x8 *__restrict__ p2op, const bf16x8 *__restrict__ p1op,
    float clip, int scale_fp16, int clip_allows_no_clamp,
    uint8_t *__restrict__ codes, void *__restrict__ scales, float *__restrict__ ydbg) {
  using C = PairCfg<N1, N2>;
  constexpr int n = N1 * N2;
  __shared__ __align__(16) unsigned char s_tile[2][C::TILE];
  __shared__ float s_max[2];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // column half
  const int g = lane >> 4;
  const int lr = lane & 15;


  // this wave's half of token tok's tile into buffer b: chunk c = mt KS + ks (lane L's 16
  // bytes of it at buffer + (c 64 + L) 16), for c in [wave HALF_LOADS, (wave+1) HALF_LOADS)
  const uint32_t lane_off = (uint32_t)(lr * N2 + g * 8);  // elements, fixed per lane
  auto dma_half = [&](int64_t tok, int b) {
    const __bf16 *xt = X + tok * ldx;  // wave-uniform base
#pragma unroll
    for (int i = 0; i < C::HALF_LOADS; ++i) {
      const int c = wave * C::HALF_LOADS + i;
      const int mt = c / C::KS, ks = c % C::KS;
      dma16_nt(xt + (mt * 16 * N2 + ks * 32), lane_off * 2, lds_addr(s_tile[b] + c * 1024));
    }
  };

  const int64_t G = gridDim.x;
  int64_t tok = blockIdx.x;
  if (tok < T) dma_half(tok, 0);  // first, so that it overlaps the operand loads below

  bf16x8 p2r[C::KS][C::NH];  // stage-1 B operands of this wave's column half
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
    for (int a = 0; a < C::NH; ++a) p2r[ks][a] = p2op[((wave * C::KS + ks) * C::NH + a) * 64 + lane];
  bf16x8 p1r[C::KK][C::MT];  // stage-2 B operands
#pragma unroll
  for (int kk = 0; kk < C::KK; ++kk)
#pragma unroll
    for (int nt = 0; nt < C::MT; ++nt) p1r[kk][nt] = p1op[(kk * C::MT + nt) * 64 + lane];
  // operands resident (and the first tile landed) before any later DMA is counted: the
  // compiler's own waits for these loads know nothing of the DMAs
  wait_and_fence<kWaitVm0>();
  if (tok + G < T) dma_half(tok + G, 1);

  // codes of the previous token, stored one step late (8 or 4 values per dword)
  uint32_t pend[C::MT][BITS == 4 ? C::NH / 2 : C::NH];
  TokenScale pend_s{0.f, (_Float16)0.f, 0.f};
  int64_t pend_tok = -1;

  for (int it = 0; tok < T; tok += G, ++it) {
    const int b = it & 1;
    // this wave's half of the tile has landed once at most the next tile's loads are in
    // flight (loads complete in issue order); the barrier adds the partner's half
    if (tok + G < T) wait_and_fence<C::kWaitHalf>();
    else wait_and_fence<kWaitVm0>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    if (pend_tok >= 0) {
      store_codes_half<N1, N2, BITS>(codes, pend_tok, wave, pend, lr, g);
      if (wave == 0 && lane == 0) store_scale(scales, pend_tok, pend_s, scale_fp16);
    }
    const unsigned char *tile = s_tile[b];

    // ---- stage 1: Z[:, half] = V P2[:, half] ----
    f32x4 zacc[C::MT][C::NH];
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
      for (int a = 0; a < C::NH; ++a) zacc[mt][a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      bf16x8 av[C::MT];
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
        av[mt] = *reinterpret_cast<const bf16x8 *>(tile + ((mt * C::KS + ks) * 64 + lane) * 16);
#pragma unroll
      for (int a = 0; a < C::NH; ++a)
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt) zacc[mt][a] = mfma(av[mt], p2r[ks][a], zacc[mt][a]);
    }
    // ---- stage 2: Y[:, half]^T = Z[:, half]^T P1 (Z rounded to bf16 as the A operand) ----
    bf16x8 za[C::KK][C::NH];
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      const bool pad = C::KHALF && kk == C::KK - 1;
#pragma unroll
      for (int m2 = 0; m2 < C::NH; ++m2)
        za[kk][m2] = pack8(zacc[2 * kk][m2], pad ? zero : zacc[(2 * kk + 1) % C::MT][m2]);
    }
    f32x4 yacc[C::NH][C::MT];
    float pm[C::NH];
#pragma unroll
    for (int m2 = 0; m2 < C::NH; ++m2) {
#pragma unroll
      for (int nt = 0; nt < C::MT; ++nt) yacc[m2][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk)
#pragma unroll
        for (int nt = 0; nt < C::MT; ++nt) yacc[m2][nt] = mfma(za[kk][m2], p1r[kk][nt], yacc[m2][nt]);
      pm[m2] = 0.f;
#pragma unroll
      for (int nt = 0; nt < C::MT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) pm[m2] = fmaxf(pm[m2], fabsf(yacc[m2][nt][r]));
    }

    // ---- absmax over both halves; lane holds Y[16 nt + lr][CB wave + LPL g + 4 m2 + r] ----
#pragma unroll
    for (int w = C::NH / 2; w >= 1; w /= 2)
#pragma unroll
      for (int i = 0; i < w; ++i) pm[i] = fmaxf(pm[i], pm[i + w]);
    const float m = wave_max_uniform(pm[0]);
    if (lane == 0) s_max[wave] = m;
    wait_and_fence<kWaitLgkm0>();  // tile reads returned, own maximum written
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    const float amax = fmaxf(m, s_max[wave ^ 1]);
    if (tok + 2 * G < T) dma_half(tok + 2 * G, b);  // both waves are done with buffer b

    const TokenScale ts = token_scale(amax, clip, scale_fp16, BITS == 4 ? 7.0f : 127.0f);
    if constexpr (BITS == 8) {
      quant_tile8<C::MT, C::NH>(yacc, ts.inv, pend);
    } else if (__builtin_amdgcn_readfirstlane(clamp_needed(clip_allows_no_clamp, ts.s32) ? 1 : 0)) {
      quant_tile<true, C::MT, C::NH>(yacc, ts.inv, pend);
    } else {
      quant_tile<false, C::MT, C::NH>(yacc, ts.inv, pend);
    }
    pend_s = ts;
    pend_tok = tok;
    if constexpr (YDBG) {
#pragma unroll
      for (int nt = 0; nt < C::MT; ++nt) {
        float4 *yp = reinterpret_cast<float4 *>(ydbg + tok * (int64_t)n + (nt * 16 + lr) * N2 +
                                                wave * C::CB + g * C::LPL);
#pragma unroll
        for (int m2 = 0; m2 < C::NH; ++m2)
          yp[m2] = make_float4(yacc[m2][nt][0], yacc[m2][nt][1], yacc[m2][nt][2], yacc[m2][nt][3]);
      }
    }
  }
  if (pend_tok >= 0) {
    store_codes_half<N1, N2, BITS>(codes, pend_tok, wave, pend, lr, g);
    if (wave == 0 && lane == 0) store_scale(scales, pend_tok, pend_s, scale_fp16);
  }
}

// ------------------------------------------------------------------------------------
// rows kernel: identity left factor, one step per row of V (per-head transform)
// ------------------------------------------------------------------------------------
// With P1 = I the rows of V never mix: row r (token t = r / n1, head i = r % n1) is
// y = x P2 on its own and gets its own INT4 step ("FlatQuant" page, Symbol Map and
// Transformer integration: the per-head transforms of keys and values ahead of the
// quantized KV cache). Rows are streamed in tiles of 16 MT, whatever n1 is; 8 waves per
// CU, each with a ring of SLOTS LDS tiles and all of P2's B operands in registers. A wave
// works on the MT 16-row groups of a tile at once: the groups' MFMA chains, row maxima,
// steps and quantizers are independent, which hides their latencies with only two waves
// per SIMD. P2's columns are permuted in the plan so that after the single MFMA stage a
// lane holds NT consecutive columns of each of its 4 rows per group: one code word per
// row, and the row's absmax is a 16-lane DPP reduction.
template <int N2>
struct RowsCfg {
  static_assert(N2 == 64 || N2 == 128, "rows kernel: n2 in {64, 128}");
  static constexpr int WAVES = 8;
  static constexpr int MT = 1;                  // 16-row groups per tile
  static constexpr int SLOTS = 4;               // ring of tiles per wave
  static constexpr int THREADS = WAVES * 64;
  static constexpr int ROWS = 16 * MT;          // rows per tile
  static constexpr int NT = N2 / 16;            // column tiles = consecutive columns per lane
  static constexpr int KS = N2 / 32;            // reduction steps
  static constexpr int RB = N2 * 2;             // bytes per row
  static constexpr int PPR = RB / 16;           // 16-byte pieces per row
  static constexpr int RPB = 256 / RB;          // rows per 256-byte bank row
  static constexpr int RPI = 1024 / RB;         // rows per DMA instruction
  static constexpr int TILE = ROWS * RB;        // bytes per tile
  static constexpr int LOADS = TILE / 1024;     // DMA instructions per tile
  static_assert(WAVES * SLOTS * TILE <= 160 * 1024, "LDS budget");
  __device__ static constexpr int swz(int R) { return (R / RPB) % PPR; }
  // vmcnt(k LOADS): at most k later tiles' loads still in flight
  template <int K>
  static constexpr int wait_imm = 0x0F70 | ((K * LOADS) & 15) | (((K * LOADS) >> 4) << 14);
  static_assert((SLOTS - 1) * LOADS < 64, "vmcnt field");
  // wait for the tile that has `later` of this wave's tiles after it (at most K in flight)
  template <int K>
  __device__ static void wait_tile(int later) {
    if constexpr (K == 0) {
      wait_and_fence<kWaitVm0>();
    } else {
      if (later >= K) wait_and_fence<wait_imm<K>>();
      else wait_tile<K - 1>(later);
    }
  }
};

// 4 consecutive values -> 2 code bytes (value e in bits 4e..4e+3), clamped to [-8, 7]
// (CLAMP = false only where the clamp is a no-op, as for quant8)
template <bool CLAMP = true>
__device__ __forceinline__ uint32_t quant4(const float (&y)[4], float inv) {
  constexpr float kMagic = 12582920.0f;   // 1.5 * 2^23 + 8 (see quant8)
  constexpr int kLo = 0x4B400000, kHi = 0x4B40000F;
  uint32_t u[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float t = __fadd_rn(__fmul_rn(y[e], inv), kMagic);
    u[e] = (CLAMP ? (uint32_t)min(max(__float_as_int(t), kLo), kHi) : __float_as_uint(t)) & 0xFu;
  }
  return ((u[0] | (u[1] << 4) | (u[2] << 8) | (u[3] << 12)) ^ 0x8888u);
}

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

// Scale of row (lr & 3) of each lane's quad; the other rows' steps arrive by quad
// broadcasts, so each lane computes one step instead of four.
template <int R>
__device__ __forceinline__ float quad_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), R | (R << 2) | (R << 4) | (R << 6),
                                                 0xF, 0xF, false));
}

template <int N2, bool YDBG, int BITS = 4>
__global__ __launch_bounds__(512) void kq_rows_kernel(
    const __bf16 *__restrict__ X, int64_t T, int n1, int64_t ldx,
    const bf16x8 *__restrict__ p2op, float clip, int scale_fp16, int clip_allows_no_clamp,
    uint8_t *__restrict__ codes, void *__restrict__ scales, float *__restrict__ ydbg) {
  using C = RowsCfg<N2>;
  constexpr int MT = C::MT;
  __shared__ __align__(16) unsigned char s_tile[C::WAVES][C::SLOTS][C::TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, lr = lane & 15;
  // rows: R = T n1 < 2^31 (checked on the host), so row and tile indices are 32-bit
  const uint32_t uT = (uint32_t)T, un1 = (uint32_t)n1;
  const uint32_t R = uT * un1;
  const uint32_t ntiles = (R + (C::ROWS - 1)) / (uint32_t)C::ROWS;
  const uint32_t stride = gridDim.x * C::WAVES;
  const uint32_t first = blockIdx.x * C::WAVES + wave;
  const int ntl = first < ntiles ? (int)((ntiles - 1u - first) / stride) + 1 : 0;  // my tiles
  const bool contiguous = ldx == (int64_t)un1 * N2;  // rows one after another in memory

  // DMA cursor: first row of the next tile to load and its (token, head), wave-uniform;
  // it moves on by stride * ROWS rows per tile without a division. Instruction j fills
  // tile rows RPI j .. RPI j + RPI - 1; lane i lands at row RPI j + i / PPR, position
  // i % PPR (piece (i % PPR) ^ swz(row)).
  //  - a whole tile of contiguous rows is one block of memory: the lanes' offsets in it
  //    are fixed (voff) and the base is uniform;
  //  - otherwise a lane's head offset x = h0 + row < n1 + ROWS is split into
  //    (x / n1, x % n1) in floating point: with rn1 = fp32(1 / n1), fp32(fp32(x + 1/2) rn1)
  //    lies within 2^-23 relative of (x + 1/2) / n1, which is at least 1/(2 n1) away from
  //    any integer, so truncation gives x / n1 exactly for x < 2^22 (n1 <= 2^20 is checked
  //    on the host). Rows past the end (token >= T) read the last row; their results are
  //    not stored.
  const uint32_t adv = stride * (uint32_t)C::ROWS;
  const uint32_t adv_t = adv / un1, adv_h = adv - adv_t * un1;
  const float rn1 = __fdiv_rn(1.0f, (float)un1);
  uint32_t crow = first * (uint32_t)C::ROWS;
  uint32_t ct = crow / un1, ch = crow - ct * un1;
  uint32_t voff[C::LOADS];
#pragma unroll
  for (int j = 0; j < C::LOADS; ++j) {
    const int Rl = j * C::RPI + lane / C::PPR;
    voff[j] = (uint32_t)(Rl * C::RB + (((lane % C::PPR) ^ C::swz(Rl)) * 16));
  }
  auto dma_next = [&](int b) {
    if (contiguous && crow + (uint32_t)C::ROWS <= R) {
      const __bf16 *base = X + (uint64_t)crow * N2;
#pragma unroll
      for (int j = 0; j < C::LOADS; ++j)
        dma16<true>(base, voff[j], lds_addr(s_tile[wave][b] + j * 1024));
    } else {
#pragma unroll
      for (int j = 0; j < C::LOADS; ++j) {
        const int Rl = j * C::RPI + lane / C::PPR;
        const uint32_t x = ch + (uint32_t)Rl;
        const uint32_t q = (uint32_t)__fmul_rn(__fadd_rn((float)x, 0.5f), rn1);
        const uint32_t t0 = ct + q, h0 = x - q * un1;
        const bool past = t0 >= uT;
        const uint32_t t = past ? uT - 1u : t0, hd = past ? un1 - 1u : h0;
        const int piece = (lane % C::PPR) ^ C::swz(Rl);
        dma16_addr<true>(X + (uint64_t)t * (uint64_t)ldx + (hd * N2 + piece * 8),
                         lds_addr(s_tile[wave][b] + j * 1024));
      }
    }
    crow += adv;
    ch += adv_h;
    const uint32_t wrap = ch >= un1 ? 1u : 0u;
    ch -= wrap * un1;
    ct += adv_t + wrap;
  };
#pragma unroll
  for (int k = 0; k < C::SLOTS; ++k)
    if (k < ntl) dma_next(k);

  bf16x8 p2r[C::KS][C::NT];  // all of P2's B operands, resident in registers
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) p2r[ks][nt] = p2op[(ks * C::NT + nt) * 64 + lane];
  // operands resident (and the first tiles landed) before the loop counts DMAs: the
  // compiler's own waits for these loads know nothing of the DMAs
  wait_and_fence<kWaitVm0>();

  // the previous tile's results: this lane's code words of each of its rows (row
  // pend_trow + 16 mt + 4 g + r: one dword of NT nibbles, or NT / 4 dwords of bytes), and
  // the step of row pend_trow + 16 mt + 4 g + (lr & 3)
  constexpr int CW = BITS == 4 ? 1 : C::NT / 4;  // code dwords per lane and row
  constexpr int ROWB = N2 * BITS / 8;            // code bytes per row
  uint32_t pend[MT][4][CW];
  TokenScale pend_s[MT];
  uint32_t pend_trow = 0;  // first row of that tile (wave-uniform)
  const int esz = scale_fp16 ? 2 : 4;

  auto store_pend = [&](bool tail) {
    uint8_t *cbase = codes + (uint64_t)pend_trow * ROWB;
    unsigned char *sbase = static_cast<unsigned char *>(scales) + (uint64_t)pend_trow * esz;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t rl = (uint32_t)(16 * mt + 4 * g + r);
        if (!tail || pend_trow + rl < R) {
          uint8_t *dst = cbase + rl * ROWB + lr * (C::NT * BITS / 8);
          if constexpr (BITS == 8 && CW == 2) {
            typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
            __builtin_nontemporal_store(u32x2_t{pend[mt][r][0], pend[mt][r][1]},
                                        reinterpret_cast<u32x2_t *>(dst));
          } else if constexpr (BITS == 8 || N2 == 128) {
            __builtin_nontemporal_store(pend[mt][r][0], reinterpret_cast<uint32_t *>(dst));
          } else {
            __builtin_nontemporal_store((uint16_t)pend[mt][r][0], reinterpret_cast<uint16_t *>(dst));
          }
        }
      }
      const uint32_t srl = (uint32_t)(16 * mt + 4 * g + (lr & 3));
      if (lr < 4 && (!tail || pend_trow + srl < R)) {
        if (scale_fp16) *reinterpret_cast<_Float16 *>(sbase + srl * 2) = pend_s[mt].s16;
        else *reinterpret_cast<float *>(sbase + srl * 4) = pend_s[mt].s32;
      }
    }
  };

  for (int it = 0; it < ntl; ++it) {
    const int b = it % C::SLOTS;
    // this tile has landed once at most the later tiles' loads (up to SLOTS - 1 tiles) are
    // in flight: loads complete in issue order, and stores are not counted on
    const int later = ntl - 1 - it;
    C::template wait_tile<C::SLOTS - 1>(later);
    const unsigned char *tile = s_tile[wave][b];
    bf16x8 av[MT][C::KS];  // A operands: row 16 mt + lr, piece 4 ks + g
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
        av[mt][ks] = *reinterpret_cast<const bf16x8 *>(
            tile + (16 * mt + lr) * C::RB + (((ks * 4 + g) ^ C::swz(16 * mt + lr)) * 16));
    wait_and_fence<kWaitLgkm0>();  // slot b is free again
    // tiles stored inside the loop are never a wave's last tile, hence never ragged
    if (it > 0) store_pend(false);
    if (later >= C::SLOTS) dma_next(b);

    f32x4 zacc[MT][C::NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) zacc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          zacc[mt][nt] = mfma(av[mt][ks], p2r[ks][nt], zacc[mt][nt]);

    // lane holds Y[row trow + 16 mt + 4 g + r][lr NT + nt]
    const uint32_t trow = (first + (uint32_t)it * stride) * (uint32_t)C::ROWS;
    const bool b0 = (lr & 1) != 0, b1 = (lr & 2) != 0;
    bool need_clamp = false;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float m[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = 0.f;
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) v = fmaxf(v, fabsf(zacc[mt][nt][r]));
        m[r] = v;
      }
      // transposing butterfly over the 16 lanes of g: after the two quad steps a lane
      // holds the quad's max of row 4 g + (lr & 3) (rows b0 and 2 + b0 after the first),
      // and two row rotations by 4 and 8 lanes combine the four quads
      const float k0 = max_nn(b0 ? m[1] : m[0], dpp_read<0xB1>(b0 ? m[0] : m[1]));
      const float k1 = max_nn(b0 ? m[3] : m[2], dpp_read<0xB1>(b0 ? m[2] : m[3]));
      float k = max_nn(b1 ? k1 : k0, dpp_read<0x4E>(b1 ? k0 : k1));
      k = dpp_step<0x124>(k);  // row_ror:4
      k = dpp_step<0x128>(k);  // row_ror:8
      pend_s[mt] = token_scale(k, clip, scale_fp16, BITS == 4 ? 7.0f : 127.0f);
      need_clamp |= BITS == 8 || clamp_needed(clip_allows_no_clamp, pend_s[mt].s32);
    }
    // the clamp is skipped only when no row of the wave can need it (one branch for all
    // rows of the tile)
    auto quantize = [&](auto clamp_tag) {
      constexpr bool CL = decltype(clamp_tag)::value;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const float inv[4] = {quad_bcast<0>(pend_s[mt].inv), quad_bcast<1>(pend_s[mt].inv),
                              quad_bcast<2>(pend_s[mt].inv), quad_bcast<3>(pend_s[mt].inv)};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (BITS == 8) {  // INT8 codes always clamp (quant4x8)
#pragma unroll
            for (int q = 0; q < CW; ++q)
              pend[mt][r][q] = quant4x8(zacc[mt][4 * q][r], zacc[mt][4 * q + 1][r],
                                        zacc[mt][4 * q + 2][r], zacc[mt][4 * q + 3][r], inv[r]);
          } else if constexpr (N2 == 128) {
            const float yv[8] = {zacc[mt][0][r], zacc[mt][1][r], zacc[mt][2][r], zacc[mt][3][r],
                                 zacc[mt][4][r], zacc[mt][5][r], zacc[mt][6][r], zacc[mt][7][r]};
            pend[mt][r][0] = quant8<CL>(yv, inv[r]);
          } else {
            const float yv[4] = {zacc[mt][0][r], zacc[mt][1][r], zacc[mt][2][r], zacc[mt][3][r]};
            pend[mt][r][0] = quant4<CL>(yv, inv[r]);
          }
        }
      }
    };
    if (__builtin_amdgcn_ballot_w64(need_clamp) != 0) quantize(BoolTag<true>{});
    else quantize(BoolTag<false>{});
    if constexpr (YDBG) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t row = trow + (uint32_t)(16 * mt + 4 * g + r);
          if (row < R) {
            float *yp = ydbg + (uint64_t)row * N2 + lr * C::NT;
#pragma unroll
            for (int q = 0; q < C::NT / 4; ++q)
              reinterpret_cast<float4 *>(yp)[q] =
                  make_float4(zacc[mt][4 * q][r], zacc[mt][4 * q + 1][r], zacc[mt][4 * q + 2][r],
                              zacc[mt][4 * q + 3][r]);
          }
        }
    }
    pend_trow = trow;
  }
  if (ntl > 0) store_pend(true);
}

// ------------------------------------------------------------------------------------
// column kernel: W = n2p/32 waves per token (n2p: n2 rounded up to a multiple of 32)
// ------------------------------------------------------------------------------------
// Waves per workgroup of the column kernel: one per 32 output columns of a token (n2p is
// n2 rounded up to a multiple of 32); where that is fewer than four, as many whole tokens
// as fill four waves share a workgroup.
constexpr int cols_waves(int n2p) {
  return n2p / 32 >= kWaves ? n2p / 32 : (n2p / 32) * (kWaves / (n2p / 32));
}
constexpr int cols_n2p(int n2) { return (n2 + 31) / 32 * 32; }

// Two workgroups per CU for n2 = 128 and n1 >= 80 (see ColsCfg::TWO), otherwise one.
constexpr bool cols_two(int n1, int n2) { return n2 == 128 && (n1 + 15) / 16 * 16 >= 80; }
constexpr int cols_min_blocks(int n1, int n2) { return cols_two(n1, n2) ? 2 : 1; }

template <int N1, int N2, bool HAS_C>
struct ColsCfg {
  static_assert(N1 >= 16 && N1 <= 128, "n1 in [16, 128]");
  static_assert(N2 % 8 == 0 && N2 >= 32 && N2 <= 256, "n2 must be a multiple of 8 in [32, 256]");
  // n2 that is not a multiple of 32 is padded with zero columns to N2P: P2's padded rows
  // and columns are zero (in the plan's operand copy), so the padded columns of V add
  // nothing to Z and the padded columns of Y are zero; they are not stored
  static constexpr int N2P = cols_n2p(N2);
  static constexpr bool PADC = N2P != N2;
  static constexpr int W = N2P / 32;                // waves per token
  static constexpr int WAVES = cols_waves(N2P);     // waves per workgroup
  static constexpr int THREADS = WAVES * 64;
  static constexpr int TPI = WAVES / W;             // tokens per workgroup iteration
  // n1 that is not a multiple of 16 is padded to whole row tiles: the padded rows of V
  // stay zero in LDS, P1's operands are zero beyond n1, so the padded rows of Y are zero
  // (no effect on the absmax) and are not stored
  static constexpr bool PADDED = (N1 % 16) != 0;
  static constexpr int MT = (N1 + 15) / 16;         // 16-row tiles of V / Z
  static constexpr int N1P = MT * 16;
  static constexpr int KS = N2P / 32;               // stage-1 reduction steps
  static constexpr int KK = (N1P + 31) / 32;        // stage-2 reduction steps of 32
  static constexpr bool KHALF = (N1P % 32) != 0;    // last step holds 16 rows + 16 zeros
  static constexpr int CH = N2 / 8;                 // 16-byte chunks per row of X
  static constexpr int CHP = N2P / 8;               // chunks per row of the tile in LDS
  static constexpr int VPLANES = HAS_C ? 2 : 1;     // hi (+ lo) bf16 planes of x*c
  static constexpr int P1_BYTES = KK * MT * 1024;   // n1 x n1 bf16, zero-padded to 32-steps
  // Two workgroups per CU (n2 = 128, n1 >= 80): with P2, P1 and the tile in LDS a single
  // workgroup of 4 waves fills the CU and runs its phases (loads, tile store, stage 1,
  // stage 2, quantizer, barriers) one after the other. Here each wave keeps its 32-column
  // block of P2 in registers and c is re-read from L2 for every tile instead of living in
  // registers; where the tile's planes and P1 would still exceed half of the LDS, the tile
  // passes through LDS in KH = 2 column halves (stage 1 reduces over each half in turn).
  // Two workgroups then share the CU and overlap each other's phases.
  static constexpr bool TWO = cols_two(N1, N2);
  static constexpr int KH = TWO && N1P * CH * 16 * VPLANES + P1_BYTES + 64 > 80 * 1024 ? 2 : 1;
  static_assert(KH == 1 || !PADC, "column parts of a padded row");
  static constexpr int CHK = CH / KH;               // chunks per row of one column part
  static constexpr int CHL = CHP / KH;              // the same in LDS (with padded columns)
  static constexpr int KSH = KS / KH;               // stage-1 steps per column part
  // row layout in LDS: vchunk_off's (an XOR swizzle for power-of-two rows, an XOR inside
  // 8- or 4-chunk groups for rows of 24, or 20 and 28, chunks, else rows padded by one chunk)
  static constexpr bool POW2 = (CHL & (CHL - 1)) == 0;
  static constexpr bool SWZ4 = vrow_swz4<CHL>();
  static constexpr int ROW_CHUNKS = vrow_chunks<CHL>();
  // byte offset of chunk cc of row r in one plane of the tile
  __device__ static int voff(int r, int cc) { return vchunk_off<CHL>(r, cc); }
  static constexpr int TOK_CHUNKS = N1 * CHK;       // chunks of one column part of a token
  static constexpr int CPT = (TPI * TOK_CHUNKS + THREADS - 1) / THREADS;  // chunks per thread
  static constexpr bool EVEN = CPT * THREADS == TPI * TOK_CHUNKS;        // no idle slots
  static constexpr int V_BYTES = N1P * ROW_CHUNKS * 16;
  static constexpr int VBUF = TPI * V_BYTES * VPLANES;
  static_assert(!TWO || VBUF + P1_BYTES + 64 <= 80 * 1024, "two workgroups per CU");
  static_assert(KS % KH == 0, "column parts");
  // P2 operands: shared in LDS while they fit, else read from the plan's copy in global
  // memory, which stays in the L2 caches
  static constexpr bool P2_LDS = N2P <= 128 && !TWO;
  static constexpr int P2_BYTES = P2_LDS ? N2P * N2P * 2 : 16;
  static_assert(!HAS_C || N2 <= 128, "column kernel with c: n2 <= 128");
  // Large n2 (P2 outside LDS): each wave keeps its 32-column block of P2 in registers and
  // the next token's tile arrives by DMA in a second LDS buffer, when two tiles and P1 fit
  static constexpr bool DMA = N2P > 128 && 2 * VBUF + P1_BYTES + 64 <= 160 * 1024;
  static constexpr bool P2REG = DMA || TWO;          // P2 block of the wave in registers
  static constexpr int VBUFS = DMA ? 2 : 1;
  static constexpr int SLOTS = N1 * ROW_CHUNKS;      // 16-byte LDS slots of one tile
  static constexpr int DMA_INSTR = (SLOTS + 63) / 64;
  static_assert(!DMA || (TPI == 1 && SLOTS % 64 == 0 && KH == 1), "tile DMA: whole instructions");
  static_assert(!PADDED || N2 <= 128, "padded n1: n2 <= 128");
};


// BITS = 4: INT4 codes (8 per dword); BITS = 8: INT8 codes (one byte per value)
template <int N1, int N2, bool HAS_C, bool YDBG = false, int BITS = 4>
__global__ __launch_bounds__(cols_waves(cols_n2p(N2)) * 64, cols_min_blocks(N1, N2)) void kq_cols_kernel(
    const __bf16 *__restrict__ X, int64_t T, int64_t ldx,
    const bf16x8 *__restrict__ p2op, const bf16x8 *__restrict__ p1op,
    const float *__restrict__ cvec, float clip, int scale_fp16, int clip_allows_no_clamp,
    uint8_t *__restrict__ codes, void *__restrict__ scales, float *__restrict__ ydbg) {
  using C = ColsCfg<N1, N2, HAS_C>;
  constexpr int n = N1 * N2;
  __shared__ __align__(16) unsigned char s_p2[C::P2_BYTES];
  __shared__ __align__(16) unsigned char s_p1[C::P1_BYTES];
  __shared__ __align__(16) unsigned char s_v[C::VBUF * C::VBUFS];
  __shared__ float s_red[C::WAVES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g = lane >> 4;
  const int lr = lane & 15;
  const int ts = wave / C::W;  // token slot within the iteration
  const int wt = wave % C::W;  // column block of this wave
  const int64_t ngroups = (T + C::TPI - 1) / C::TPI;

  if constexpr (C::P2_LDS) copy_to_lds(s_p2, p2op, C::P2_BYTES, tid, C::THREADS);
  copy_to_lds(s_p1, p1op, C::P1_BYTES, tid, C::THREADS);
  if constexpr (C::PADDED) {  // rows n1 .. n1P of every tile plane stay zero
    constexpr int PAD_UNITS = (C::N1P - N1) * C::ROW_CHUNKS;  // 16-byte units per plane
    for (int q = tid; q < C::TPI * C::VPLANES * PAD_UNITS; q += C::THREADS)
      *reinterpret_cast<uint4 *>(s_v + (q / PAD_UNITS) * C::V_BYTES + N1 * C::ROW_CHUNKS * 16 +
                                 (q % PAD_UNITS) * 16) = make_uint4(0u, 0u, 0u, 0u);
  }
  if constexpr (C::PADC && !C::DMA) {  // chunks CH .. CHP of every row stay zero
    constexpr int PC = C::CHP - C::CH, PER_PLANE = N1 * PC;
    for (int q = tid; q < C::TPI * C::VPLANES * PER_PLANE; q += C::THREADS) {
      const int pl = q / PER_PLANE, r = (q % PER_PLANE) / PC, cc = C::CH + q % PC;
      *reinterpret_cast<uint4 *>(s_v + pl * C::V_BYTES + C::voff(r, cc)) =
          make_uint4(0u, 0u, 0u, 0u);
    }
  }
  // (with the tile DMA, the padded chunks of a row receive a copy of its first chunk:
  // finite values that meet P2's zero rows)

  // per-thread chunk coordinates (fixed for the whole kernel)
  int c_ts[C::CPT], c_row[C::CPT], c_cc[C::CPT];
  bool c_ok[C::CPT];  // chunk q exists (threads can outnumber a padded tile's chunks)
#pragma unroll
  for (int i = 0; i < C::CPT; ++i) {
    const int q0 = tid + C::THREADS * i;
    c_ok[i] = C::EVEN || q0 < C::TPI * C::TOK_CHUNKS;
    const int q = c_ok[i] ? q0 : 0;
    c_ts[i] = q / C::TOK_CHUNKS;
    const int qq = q % C::TOK_CHUNKS;
    c_row[i] = qq / C::CHK;
    c_cc[i] = qq % C::CHK;
  }
  // per-channel scale of this thread's chunks, kept in registers (re-read from L2 for each
  // tile in the two-workgroup mode)
  float creg[HAS_C && !C::TWO ? C::CPT : 1][8];
  if constexpr (HAS_C && !C::TWO) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const float4 *cp = reinterpret_cast<const float4 *>(cvec + c_row[i] * N2 + c_cc[i] * 8);
      const float4 a = cp[0], b = cp[1];
      creg[i][0] = a.x; creg[i][1] = a.y; creg[i][2] = a.z; creg[i][3] = a.w;
      creg[i][4] = b.x; creg[i][5] = b.y; creg[i][6] = b.z; creg[i][7] = b.w;
    }
  }

  // loads of column part h (chunks h CHK .. h CHK + CHK - 1 of every row) of group grp,
  // into that part's own registers
  uint4 pre[C::KH][C::CPT];
  auto issue_loads = [&](int64_t grp, int h) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int64_t t = grp * C::TPI + c_ts[i];
      if (c_ok[i] && t < T) {
        pre[h][i] = *reinterpret_cast<const uint4 *>(X + t * ldx + c_row[i] * N2 + (h * C::CHK + c_cc[i]) * 8);
      } else {
        pre[h][i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };
  auto store_lds = [&](int h) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      if (!c_ok[i]) continue;
      const int off = c_ts[i] * C::V_BYTES + C::voff(c_row[i], c_cc[i]);
      if constexpr (HAS_C) {
        uint4 hi, lo;
        if constexpr (C::TWO) {
          const float4 *cp =
              reinterpret_cast<const float4 *>(cvec + c_row[i] * N2 + (h * C::CHK + c_cc[i]) * 8);
          const float4 a = cp[0], b = cp[1];
          const float cl[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
          split_scaled(pre[h][i], cl, hi, lo);
        } else {
          split_scaled(pre[h][i], creg[i], hi, lo);
        }
        *reinterpret_cast<uint4 *>(s_v + off) = hi;
        *reinterpret_cast<uint4 *>(s_v + C::TPI * C::V_BYTES + off) = lo;
      } else {
        *reinterpret_cast<uint4 *>(s_v + off) = pre[h][i];
      }
    }
  };

  // Large n2: P2 does not fit in LDS next to the tile and P1, but one wave only ever uses
  // its own 32-column block of P2 (n2 x 32 values, KS x 2 operands), which it keeps in
  // registers for the whole kernel. The workgroup loads the next token's tile by DMA into
  // the other LDS buffer: LDS slot q of the tile (row q / ROW_CHUNKS, position q %
  // ROW_CHUNKS, which holds the chunk that voff puts there; a padding chunk re-reads chunk
  // 0) is written by lane q % 64 of instruction q / 64.
  // No other global load sits inside the token loop, so one wait before the end-of-token
  // barrier covers the DMA.
  auto dma_tile = [&](int64_t t, int b) {
    const __bf16 *base = X + t * ldx;
    for (int j = wave; j < C::DMA_INSTR; j += C::WAVES) {
      const int q = j * 64 + lane;
      const int r = q / C::ROW_CHUNKS;
      const int cc = C::SWZ4 ? (q % C::ROW_CHUNKS) ^ ((r >> 1) & vrow_xmask<C::CHL>()) : q % C::ROW_CHUNKS;
      const uint32_t voff = (uint32_t)((r * N2 + (cc < C::CH ? cc : 0) * 8) * 2);
      dma16<true>(base, voff, __builtin_amdgcn_readfirstlane(lds_addr(s_v + b * C::VBUF + j * 1024)));
    }
  };
  bf16x8 p2w[C::P2REG ? C::KS : 1][2];
  if constexpr (C::P2REG) {
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      p2w[ks][0] = p2op[((wt * C::KS + ks) * 2 + 0) * 64 + lane];
      p2w[ks][1] = p2op[((wt * C::KS + ks) * 2 + 1) * 64 + lane];
    }
  }

  int64_t grp = blockIdx.x;
  if constexpr (C::DMA) {
    if (grp < ngroups) dma_tile(grp, 0);
    wait_and_fence<kWaitVm0>();  // the first tile and P2's registers have landed
  } else {
    if (grp < ngroups)
#pragma unroll
      for (int h = 0; h < C::KH; ++h) issue_loads(grp, h);
  }
  lds_barrier();  // factors (and the first DMA tile) visible

  const bf16x8 *sp2 = reinterpret_cast<const bf16x8 *>(s_p2);
  const bf16x8 *sp1 = reinterpret_cast<const bf16x8 *>(s_p1);

  for (int it = 0; grp < ngroups; grp += gridDim.x, ++it) {
    const int64_t nxt = grp + gridDim.x;
    const int64_t tok = grp * C::TPI + ts;

    // ---- stage 1: Z[:, block] = V P2[:, block]  (M = n1 rows, K = n2, N = 32) ----
    f32x4 zacc[C::MT][2];
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) zacc[mt][0] = zacc[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < C::KH; ++h) {  // column parts of the tile
      const unsigned char *vt;
      if constexpr (C::DMA) {
        // the other buffer was last read in the previous iteration, before its final barrier
        if (nxt < ngroups) dma_tile(nxt, (it + 1) & 1);
        vt = s_v + (it & 1) * C::VBUF;
      } else {
        store_lds(h);
        lds_barrier();
        // this part's registers are free: the next group's same part is in flight for a
        // whole group's computation
        if (nxt < ngroups) issue_loads(nxt, h);
        vt = s_v + ts * C::V_BYTES;
      }
      // (n2 = 256: a rolled loop, so that only one step's operands are in registers)
      constexpr int KS_UNROLL = C::P2_LDS || C::P2REG ? C::KSH : 1;
#pragma unroll KS_UNROLL
      for (int ks = h * C::KSH; ks < (h + 1) * C::KSH; ++ks) {
        bf16x8 b0, b1;
        if constexpr (C::P2_LDS) {
          b0 = sp2[((wt * C::KS + ks) * 2 + 0) * 64 + lane];
          b1 = sp2[((wt * C::KS + ks) * 2 + 1) * 64 + lane];
        } else if constexpr (C::P2REG) {
          b0 = p2w[ks][0];
          b1 = p2w[ks][1];
        } else {  // from the plan's copy in global memory (L2-resident, shared by all CUs)
          b0 = p2op[((wt * C::KS + ks) * 2 + 0) * 64 + lane];
          b1 = p2op[((wt * C::KS + ks) * 2 + 1) * 64 + lane];
        }
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt) {
          const int off = C::voff(mt * 16 + lr, (ks - h * C::KSH) * 4 + g);
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(vt + off);
          zacc[mt][0] = mfma(a, b0, zacc[mt][0]);
          zacc[mt][1] = mfma(a, b1, zacc[mt][1]);
          if constexpr (HAS_C) {
            const bf16x8 al = *reinterpret_cast<const bf16x8 *>(vt + C::TPI * C::V_BYTES + off);
            zacc[mt][0] = mfma(al, b0, zacc[mt][0]);
            zacc[mt][1] = mfma(al, b1, zacc[mt][1]);
          }
        }
      }
      if (h + 1 < C::KH) lds_barrier();  // every wave is done with this part's planes
    }

    // ---- stage 2: Y^T[block, :] = Z[:, block]^T P1  (M = 32, K = n1, N = n1) ----
    // The stage-1 accumulators of row tiles (2kk, 2kk+1) form the A operand of step kk;
    // an odd number of row tiles pads the last step with zeros (and P1 with zero rows),
    // so that every accumulator chain uses the same MFMA opcode.
    // (Z is packed to bf16 first, so that its fp32 accumulators are dead before Y's are live)
    bf16x8 za[C::KK][2];
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      const bool pad = C::KHALF && kk == C::KK - 1;
      za[kk][0] = pack8(zacc[2 * kk][0], pad ? zero : zacc[(2 * kk + 1) % C::MT][0]);
      za[kk][1] = pack8(zacc[2 * kk][1], pad ? zero : zacc[(2 * kk + 1) % C::MT][1]);
    }
    f32x4 yacc[2][C::MT];
#pragma unroll
    for (int nt = 0; nt < C::MT; ++nt) yacc[0][nt] = yacc[1][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      const bf16x8 za0 = za[kk][0], za1 = za[kk][1];
#pragma unroll
      for (int nt = 0; nt < C::MT; ++nt) {
        const bf16x8 b = sp1[(kk * C::MT + nt) * 64 + lane];
        yacc[0][nt] = mfma(za0, b, yacc[0][nt]);
        yacc[1][nt] = mfma(za1, b, yacc[1][nt]);
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
    m = wave_max_uniform(m);
    if (lane == 0) s_red[wave] = m;
    lds_barrier();
    float amax = 0.f;
#pragma unroll
    for (int w = 0; w < C::W; ++w) amax = fmaxf(amax, s_red[ts * C::W + w]);
    const TokenScale sc = token_scale(amax, clip, scale_fp16, BITS == 4 ? 7.0f : 127.0f);

    if (tok < T) {
      // lane holds Y[j = nt*16 + lr][wt*32 + 8g + 4h + r]: 8 consecutive codes -> 1 dword
      // (INT4) or 2 dwords (INT8); a uniform row base plus a 32-bit lane offset (nothing
      // 64-bit per lane to keep)
      constexpr int RB = N2 * BITS / 8;  // code bytes per row of Y
      uint8_t *crow = codes + tok * (int64_t)(n * BITS / 8);
      const uint32_t loff = (uint32_t)(lr * RB + (wt * 32 + g * 8) * BITS / 8);
      // one scalar branch on the clamp (INT4: skipped where the clip ratio rules it out)
      auto emit = [&](auto clamp_tag) {
#pragma unroll
        for (int nt = 0; nt < C::MT; ++nt) {
          const int j = nt * 16 + lr;
          if (C::PADDED && j >= N1) continue;  // padded rows of Y are not stored
          if (C::PADC && wt * 32 + g * 8 >= N2) continue;  // nor its padded columns
          uint8_t *dst = crow + (loff + (uint32_t)(nt * 16 * RB));
          if constexpr (BITS == 8) {
            const u32x2_t w = {quant4x8(yacc[0][nt][0], yacc[0][nt][1], yacc[0][nt][2], yacc[0][nt][3], sc.inv),
                               quant4x8(yacc[1][nt][0], yacc[1][nt][1], yacc[1][nt][2], yacc[1][nt][3], sc.inv)};
            *reinterpret_cast<u32x2_t *>(dst) = w;
          } else {
            const float yv[8] = {yacc[0][nt][0], yacc[0][nt][1], yacc[0][nt][2], yacc[0][nt][3],
                                 yacc[1][nt][0], yacc[1][nt][1], yacc[1][nt][2], yacc[1][nt][3]};
            *reinterpret_cast<uint32_t *>(dst) = quant8<decltype(clamp_tag)::value>(yv, sc.inv);
          }
          if constexpr (YDBG) {
            float4 *yp = reinterpret_cast<float4 *>(ydbg + tok * (int64_t)n + j * N2 + wt * 32 + g * 8);
            yp[0] = make_float4(yacc[0][nt][0], yacc[0][nt][1], yacc[0][nt][2], yacc[0][nt][3]);
            yp[1] = make_float4(yacc[1][nt][0], yacc[1][nt][1], yacc[1][nt][2], yacc[1][nt][3]);
          }
        }
      };
      if (BITS == 8 || __builtin_amdgcn_readfirstlane(clamp_needed(clip_allows_no_clamp, sc.s32) ? 1 : 0))
        emit(std::true_type{});
      else
        emit(std::false_type{});
      if (wt == 0 && lane == 0) store_scale(scales, tok, sc, scale_fp16);
    }
    if constexpr (C::DMA) wait_and_fence<kWaitVm0>();  // the next tile has landed
    lds_barrier();  // V tile and s_red are reused by the next iteration
  }
}

// ------------------------------------------------------------------------------------
// column kernel with a per-channel scale: fp16 operands, two barriers per token
// ------------------------------------------------------------------------------------
// The same work split as the column kernel (W = n2p / 32 waves per token, each owning 32
// output columns; whole tokens fill four waves when W < 4), with both contractions on
// fp16 operands:
//  * x^ = fp16(fp32(x c) 2^sx), where the token's bound max|x| max|c| picks the
//    power-of-two sx (f16_scale_exp: 0 for ordinary tokens), stored as the token's plane in
//    LDS; P2 comes from the plan as fp16 operands (P2 2^-f2), kept per wave in registers;
//  * stage 1 accumulates Z' = x^ P2' in fp32; the token's largest |Z'| meets in LDS and
//    picks sz for Z's conversion to fp16; P1 comes from the plan as fp16 (P1 2^-f1);
//  * stage 2 accumulates Y' in fp32 and Y = Y' 2^(f1 + f2 - sx - sz) exactly.
// One LDS tile per token slot. Per token two barriers: (A) after stage 1, when every wave
// has read the tile and published its |Z'| maximum and the next token's |x| maximum (its
// chunks were loaded into registers a whole token earlier), the next token's tile is
// stored over this one; (B) after stage 2, when the next tile is complete and every wave
// has published its |Y| maximum. c stays in registers as fp16 where the plan allows it, else
// it is re-read from L2 for every tile. A token's codes are
// staged in LDS and written after the next barrier A.
template <int N1, int N2>
struct ColsCCfg {
  static_assert(N1 >= 16 && N1 <= 128, "n1 in [16, 128]");
  static_assert(N2 % 8 == 0 && N2 >= 32 && N2 <= 128, "n2 a multiple of 8 in [32, 128]");
  static constexpr int N2P = cols_n2p(N2);
  static constexpr bool PADC = N2P != N2;
  static constexpr int W = N2P / 32;                // waves per token
  static constexpr int WAVES = cols_waves(N2P);     // waves per workgroup
  static constexpr int THREADS = WAVES * 64;
  static constexpr int TPI = WAVES / W;             // tokens per workgroup iteration
  static constexpr bool PADDED = (N1 % 16) != 0;
  static constexpr int MT = (N1 + 15) / 16;
  static constexpr int N1P = MT * 16;
  static constexpr int KS = N2P / 32;
  static constexpr int KK = (N1P + 31) / 32;
  static constexpr bool KHALF = (N1P % 32) != 0;
  static constexpr int CH = N2 / 8;                 // 16-byte chunks per row of X
  static constexpr int CHP = N2P / 8;               // chunks per row in LDS
  static constexpr bool POW2 = (CHP & (CHP - 1)) == 0;
  static constexpr int ROW_CHUNKS = vrow_chunks<CHP>();
  static constexpr int TOK_CHUNKS = N1 * CH;
  static constexpr int CPT = (TPI * TOK_CHUNKS + THREADS - 1) / THREADS;
  static constexpr bool EVEN = CPT * THREADS == TPI * TOK_CHUNKS;
  static constexpr int V_BYTES = N1P * ROW_CHUNKS * 16;
  static constexpr int VBUF = TPI * V_BYTES;
  static constexpr int P1_BYTES = KK * MT * 1024;
  // two workgroups per CU when both fit in LDS
  static constexpr bool TWO = VBUF + P1_BYTES + 1024 <= 80 * 1024;
  // a thread's c values fit its registers next to the rest for tiles of up to 112 rows
  static constexpr bool CREG_OK = MT <= 7;
};

// workgroups per CU the launch bounds ask for
template <int N1, int N2>
constexpr int colsc_blocks = ColsCCfg<N1, N2>::TWO ? 2 : 1;

template <int N1, int N2, bool YDBG = false, int BITS = 4, bool CREG = false>
__global__ __launch_bounds__(cols_waves(cols_n2p(N2)) * 64, (colsc_blocks<N1, N2>)) void kq_colsc_kernel(
    const __bf16 *__restrict__ X, int64_t T, int64_t ldx,
    const f16x8 *__restrict__ p2op, const f16x8 *__restrict__ p1op,
    const float *__restrict__ cvec, int f_exp, float cmax, float clip, int scale_fp16,
    int clip_allows_no_clamp, uint8_t *__restrict__ codes, void *__restrict__ scales,
    float *__restrict__ ydbg) {
  using C = ColsCCfg<N1, N2>;
  constexpr int n = N1 * N2;
  // A lane holds 8 columns of a row (4 bytes of INT4 codes), so direct code stores would
  // scatter 16-byte pieces over 16 rows per instruction. Where LDS allows (the occupancy
  // unchanged), a token's codes are staged in LDS in their global layout and written
  // after the next barrier as whole 16-byte words per lane, consecutive across lanes.
  constexpr int TOK_CODE = n * BITS / 8;  // code bytes per token
  constexpr int STAGED_BYTES = C::TPI * TOK_CODE;
  constexpr int LDS_BASE = C::P1_BYTES + C::VBUF + 1024;
  // (not for 128-row tiles: the staging addresses would make the wave spill)
  constexpr bool STAGE = TOK_CODE % 16 == 0 && C::N1P < 128 &&
                         LDS_BASE + STAGED_BYTES <= (C::TWO ? 80 * 1024 : 160 * 1024);
  __shared__ __align__(16) unsigned char s_code[STAGE ? STAGED_BYTES : 16];
  __shared__ __align__(16) unsigned char s_p1[C::P1_BYTES];
  __shared__ __align__(16) unsigned char s_v[C::VBUF];
  __shared__ float s_zmax[2][C::WAVES];
  __shared__ float s_xmax[2][C::WAVES][C::TPI];
  __shared__ float s_red[2][C::WAVES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int lr = lane & 15;
  const int ts = wave / C::W;  // token slot within the iteration
  const int wt = wave % C::W;  // column block of this wave
  const int64_t ngroups = (T + C::TPI - 1) / C::TPI;

  copy_to_lds(s_p1, p1op, C::P1_BYTES, tid, C::THREADS);
  if constexpr (C::PADDED) {  // rows n1 .. n1p of every slot stay zero
    constexpr int PAD_UNITS = (C::N1P - N1) * C::ROW_CHUNKS;
    for (int q = tid; q < C::TPI * PAD_UNITS; q += C::THREADS)
      *reinterpret_cast<uint4 *>(s_v + (q / PAD_UNITS) * C::V_BYTES + N1 * C::ROW_CHUNKS * 16 +
                                 (q % PAD_UNITS) * 16) = make_uint4(0u, 0u, 0u, 0u);
  }
  if constexpr (C::PADC) {  // chunks ch .. chp of every row stay zero
    constexpr int PC = C::CHP - C::CH, PER_SLOT = N1 * PC;
    for (int q = tid; q < C::TPI * PER_SLOT; q += C::THREADS) {
      const int sl = q / PER_SLOT, r = (q % PER_SLOT) / PC, cc = C::CH + q % PC;
      *reinterpret_cast<uint4 *>(s_v + sl * C::V_BYTES + vchunk_off<C::CHP>(r, cc)) =
          make_uint4(0u, 0u, 0u, 0u);
    }
  }

  // per-thread chunk coordinates (fixed for the whole kernel), as expressions of tid: chunk
  // i of the thread is chunk q = tid + THREADS i of the group, i.e. chunk qq = q % TOK_CHUNKS
  // of token slot q / TOK_CHUNKS, whose 8 values start at element 8 qq of the token (rows of
  // X hold CH chunks)
  auto c_okf = [&](int i) { return C::EVEN || (unsigned)tid + C::THREADS * i < (unsigned)(C::TPI * C::TOK_CHUNKS); };
  auto c_q = [&](int i) { return c_okf(i) ? (unsigned)tid + C::THREADS * i : 0u; };
  auto c_tsf = [&](int i) { return C::TPI == 1 ? 0 : (int)(c_q(i) / C::TOK_CHUNKS); };
  auto c_qq = [&](int i) { return C::TPI == 1 ? c_q(i) : c_q(i) % C::TOK_CHUNKS; };
  auto c_rowf = [&](int i) { return (int)(c_qq(i) / C::CH); };
  auto c_ccf = [&](int i) { return (int)(c_qq(i) % C::CH); };
  uint4 pre[C::CPT];
  // The channels a thread converts are the same for every token. Where registers allow
  // (tiles of up to 112 rows) and the plan found every nonzero |c| in fp16's normal range
  // [2^-14, 2^15) (CREG), the thread's c values stay in registers rounded to fp16, and
  // x^ = fp16(fp32(x fp16(c)) 2^sx), where x fp16(c) is exact in fp32 (8 + 11 significant
  // bits). Otherwise c is re-read from L2 (fp32) for every tile and x^ = fp16(fp32(x c) 2^sx).
  constexpr bool USE_CREG = CREG && C::CREG_OK;
  f16x8 creg[USE_CREG ? C::CPT : 1];
  if constexpr (USE_CREG) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const float4 *cp = reinterpret_cast<const float4 *>(cvec + 8 * c_qq(i));
      const float4 a = cp[0], b = cp[1];
      creg[i] = f16x8{(_Float16)a.x, (_Float16)a.y, (_Float16)a.z, (_Float16)a.w,
                      (_Float16)b.x, (_Float16)b.y, (_Float16)b.z, (_Float16)b.w};
    }
  }
  auto issue_loads = [&](int64_t grp) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int64_t t = grp * C::TPI + c_tsf(i);
      if (c_okf(i) && t < T)
        pre[i] = *reinterpret_cast<const uint4 *>(X + t * ldx + 8 * c_qq(i));
      else
        pre[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  };
  // |x| maximum of the loaded chunks per token slot, wave-reduced, into s_xmax[b]
  auto publish_xmax = [&](int b) {
    uint32_t m[C::TPI];
#pragma unroll
    for (int sl = 0; sl < C::TPI; ++sl) m[sl] = 0;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const uint32_t a = absmax_bf16(pre[i], 0);
#pragma unroll
      for (int sl = 0; sl < C::TPI; ++sl)
        if (c_tsf(i) == sl) m[sl] = a > m[sl] ? a : m[sl];
    }
#pragma unroll
    for (int sl = 0; sl < C::TPI; ++sl) {
      const float v = wave_max_uniform(__uint_as_float(m[sl] << 16));
      if (lane == 0) s_xmax[b][wave][sl] = v;
    }
  };
  // the scale exponent of x^ for every token slot, from the published maxima
  auto x_scales = [&](int b, int (&sx)[C::TPI]) {
#pragma unroll
    for (int sl = 0; sl < C::TPI; ++sl) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < C::WAVES; ++w) v = fmaxf(v, s_xmax[b][w][sl]);
      sx[sl] = __builtin_amdgcn_readfirstlane(f16_scale_exp(__fmul_rn(v, cmax)));
    }
  };
  // x^ of the loaded chunks into the tile. The scales are wave-uniform, so tokens that
  // need none (the usual case) take the branch without the ldexp.
  auto store_lds = [&](const int (&sx)[C::TPI]) {
    auto store = [&](auto scale) {
#pragma unroll
      for (int i = 0; i < C::CPT; ++i) {
        if (!c_okf(i)) continue;
        int s = sx[0];
#pragma unroll
        for (int sl = 1; sl < C::TPI; ++sl) s = c_tsf(i) == sl ? sx[sl] : s;
        float cl[8];
        if constexpr (USE_CREG) {
#pragma unroll
          for (int e = 0; e < 8; ++e) cl[e] = (float)creg[i][e];
        } else {
          const float4 *cp = reinterpret_cast<const float4 *>(cvec + 8 * c_qq(i));
          const float4 a = cp[0], b = cp[1];
          cl[0] = a.x; cl[1] = a.y; cl[2] = a.z; cl[3] = a.w;
          cl[4] = b.x; cl[5] = b.y; cl[6] = b.z; cl[7] = b.w;
        }
        *reinterpret_cast<f16x8 *>(s_v + c_tsf(i) * C::V_BYTES + vchunk_off<C::CHP>(c_rowf(i), c_ccf(i))) =
            scale_round_f16<decltype(scale)::value>(pre[i], cl, s);
      }
    };
    int any = 0;
#pragma unroll
    for (int sl = 0; sl < C::TPI; ++sl) any |= sx[sl];
    if (any == 0) store(std::false_type{});
    else store(std::true_type{});
  };
  f16x8 p2w[C::KS][2];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    p2w[ks][0] = p2op[((wt * C::KS + ks) * 2 + 0) * 64 + lane];
    p2w[ks][1] = p2op[((wt * C::KS + ks) * 2 + 1) * 64 + lane];
  }

  int64_t grp = blockIdx.x;
  int sx[C::TPI];
  if (grp < ngroups) issue_loads(grp);
  publish_xmax(1);
  lds_barrier();  // P1, the zero padding and the first token's |x| maxima visible
  x_scales(1, sx);
  if (grp < ngroups) store_lds(sx);
  int sx_tok = sx[0];  // the scale of x^ of this wave's token
#pragma unroll
  for (int sl = 1; sl < C::TPI; ++sl) sx_tok = ts == sl ? sx[sl] : sx_tok;
  lds_barrier();  // the first tile visible
  if (grp + gridDim.x < ngroups) issue_loads(grp + gridDim.x);

  // the staged codes of group `gq` to global memory: its tokens are consecutive, so the
  // staged bytes (slot-major) are one contiguous run of codes; 16-byte words, consecutive
  // threads on consecutive words, the tokens at or beyond T left out
  // Staged INT4 rows of 128 codes (64 bytes, 4 words): the 16 rows a code store covers
  // would put 4 lanes on every bank, so word w of row R sits at w ^ ((R / 4) % 4) within
  // its row (then the 64 lanes' 4-byte pieces hit 64 different banks); code_unit maps a
  // word's place in the token's codes to its place in the staging buffer (an involution)
  constexpr bool SWZ_CODE = STAGE && BITS == 4 && N2 == 128;
  static_assert(!SWZ_CODE || C::TPI == 1 || (TOK_CODE / 16) % 16 == 0, "word swizzle per token");
  auto code_unit = [](int u) { return SWZ_CODE ? u ^ ((u >> 4) & 3) : u; };
  auto store_staged = [&](int64_t gq) {
    constexpr int WPT = TOK_CODE / 16;  // 16-byte words per token
    const int64_t t0 = gq * C::TPI;
    const int lim = (int)(T - t0 < C::TPI ? T - t0 : C::TPI) * WPT;
    uint8_t *dst = codes + t0 * (int64_t)TOK_CODE;
#pragma unroll
    for (int u = tid; u < C::TPI * WPT; u += C::THREADS) {
      if (u < lim)
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t *>(s_code + code_unit(u) * 16),
                                    reinterpret_cast<u32x4_t *>(dst + u * 16));
    }
  };
  int64_t staged_grp = -1;  // group whose codes wait in s_code

  const f16x8 *sp1 = reinterpret_cast<const f16x8 *>(s_p1);
  const unsigned char *vt = s_v + ts * C::V_BYTES;
  for (int it = 0; grp < ngroups; grp += gridDim.x, ++it) {
    const int64_t tok = grp * C::TPI + ts;
    const int64_t nxt = grp + gridDim.x;
    // ---- stage 1: Z'[:, block] = x^ P2'[:, block] ----
    f32x4 zacc[C::MT][2];
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) zacc[mt][0] = zacc[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) {
        const f16x8 a = *reinterpret_cast<const f16x8 *>(vt + vchunk_off<C::CHP>(mt * 16 + lr, ks * 4 + g));
        zacc[mt][0] = mfma_f16(a, p2w[ks][0], zacc[mt][0]);
        zacc[mt][1] = mfma_f16(a, p2w[ks][1], zacc[mt][1]);
      }
    float zm = 0.f;
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) zm = absmax_acc(zacc[mt], zm);
    zm = wave_max_uniform(zm);
    if (lane == 0) s_zmax[it & 1][wave] = zm;
    if (nxt < ngroups) publish_xmax(it & 1);  // the next token's chunks, loaded a token ago
    lds_barrier();  // (A) the tile is read; the |Z'| and next |x| maxima are published
    float zmax = 0.f;
#pragma unroll
    for (int w = 0; w < C::W; ++w) zmax = fmaxf(zmax, s_zmax[it & 1][ts * C::W + w]);
    const int zs = __builtin_amdgcn_readfirstlane(f16_scale_exp(zmax));
    const int ty = f_exp - sx_tok - zs;  // Y = Y' 2^(f1 + f2 - sx - sz), exact
    // Z' as stage 2's fp16 operands (packed before the next tile's conversion, so that the
    // stage-1 accumulators are dead while it runs)
    f16x8 za[C::KK][2];
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      const bool pad = C::KHALF && kk == C::KK - 1;
      za[kk][0] = pack8_f16(zacc[2 * kk][0], pad ? zero : zacc[(2 * kk + 1) % C::MT][0], zs);
      za[kk][1] = pack8_f16(zacc[2 * kk][1], pad ? zero : zacc[(2 * kk + 1) % C::MT][1], zs);
    }
    // the next group's tile replaces this one
    if (nxt < ngroups) {
      x_scales(it & 1, sx);
      store_lds(sx);
      if (nxt + gridDim.x < ngroups) issue_loads(nxt + gridDim.x);
    }
    // The previous group's codes are complete in s_code (written before barrier A); they
    // are read here, before barrier B, and s_code is rewritten only after it. Issued after
    // the tile store and the prefetch, so that no wait for those loads covers these stores.
    if constexpr (STAGE) {
      if (staged_grp >= 0) store_staged(staged_grp);
    }

    // ---- stage 2: Y'^T[block, :] = Z'[:, block]^T P1' on fp16 operands ----
    f32x4 yacc[2][C::MT];
#pragma unroll
    for (int nt = 0; nt < C::MT; ++nt) yacc[0][nt] = yacc[1][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk)
#pragma unroll
      for (int nt = 0; nt < C::MT; ++nt) {
        const f16x8 b = sp1[(kk * C::MT + nt) * 64 + lane];
        yacc[0][nt] = mfma_f16(za[kk][0], b, yacc[0][nt]);
        yacc[1][nt] = mfma_f16(za[kk][1], b, yacc[1][nt]);
      }
    if (nxt < ngroups) {  // the next token's scale, for the next iteration
      sx_tok = sx[0];
#pragma unroll
      for (int sl = 1; sl < C::TPI; ++sl) sx_tok = ts == sl ? sx[sl] : sx_tok;
    }

    // ---- epilogue: absmax over the token, then codes ----
    // The maxima are those of Y' (Y = Y' 2^ty); ldexp is monotone, so max|Y| is the
    // scaled maximum.
    float m = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h) m = absmax_acc(yacc[h], m);
    m = wave_max_uniform(m);
    if (lane == 0) s_red[it & 1][wave] = m;
    lds_barrier();  // (B) the next tile is stored; the |Y| maxima are published
    float amax_y = 0.f;
#pragma unroll
    for (int w = 0; w < C::W; ++w) amax_y = max_nn(amax_y, s_red[it & 1][ts * C::W + w]);
    const float amax = __builtin_ldexpf(amax_y, ty);
    const TokenScale sc = token_scale(amax, clip, scale_fp16, BITS == 4 ? 7.0f : 127.0f);
    // codes straight from Y' with the reciprocal scaled by 2^ty where that is exact, else
    // from Y = ldexp(Y', ty) (then ty_dbg = 0: yacc holds Y)
    float inv_y;
    int ty_dbg = ty;
    if (!__builtin_amdgcn_readfirstlane(fold_scale(sc.inv, ty, amax, inv_y) ? 1 : 0)) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int nt = 0; nt < C::MT; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r) yacc[h][nt][r] = __builtin_ldexpf(yacc[h][nt][r], ty);
      inv_y = sc.inv;
      ty_dbg = 0;
    }
    const bool clamp = BITS == 8 || __builtin_amdgcn_readfirstlane(
                                        clamp_needed(clip_allows_no_clamp, sc.s32) ? 1 : 0);

    if (tok < T) {
      // lane holds Y[j = nt*16 + lr][wt*32 + 8g + 4h + r]
      constexpr int RB = N2 * BITS / 8;
      uint8_t *crow = STAGE ? s_code + ts * TOK_CODE : codes + tok * (int64_t)TOK_CODE;
      // (rows 16 nt + lr share lr % 16, so one swizzle serves all of the lane's rows)
      const uint32_t loff = (uint32_t)(lr * RB + (SWZ_CODE ? ((wt ^ ((lr >> 2) & 3)) * 16 + g * 4)
                                                           : (wt * 32 + g * 8) * BITS / 8));
      // one scalar branch on the clamp for the whole tile
      auto emit = [&](auto clamp_tag) {
#pragma unroll
        for (int nt = 0; nt < C::MT; ++nt) {
          const int j = nt * 16 + lr;
          if (C::PADDED && j >= N1) continue;
          if (C::PADC && wt * 32 + g * 8 >= N2) continue;
          uint8_t *dst = crow + (loff + (uint32_t)(nt * 16 * RB));
          if constexpr (BITS == 8) {
            const u32x2_t w = {quant4x8(yacc[0][nt][0], yacc[0][nt][1], yacc[0][nt][2], yacc[0][nt][3], inv_y),
                               quant4x8(yacc[1][nt][0], yacc[1][nt][1], yacc[1][nt][2], yacc[1][nt][3], inv_y)};
            *reinterpret_cast<u32x2_t *>(dst) = w;
          } else {
            const float yv[8] = {yacc[0][nt][0], yacc[0][nt][1], yacc[0][nt][2], yacc[0][nt][3],
                                 yacc[1][nt][0], yacc[1][nt][1], yacc[1][nt][2], yacc[1][nt][3]};
            *reinterpret_cast<uint32_t *>(dst) = quant8<decltype(clamp_tag)::value>(yv, inv_y);
          }
          if constexpr (YDBG) {
            float yd[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) yd[e] = __builtin_ldexpf(yacc[e / 4][nt][e % 4], ty_dbg);
            float4 *yp = reinterpret_cast<float4 *>(ydbg + tok * (int64_t)n + j * N2 + wt * 32 + g * 8);
            yp[0] = make_float4(yd[0], yd[1], yd[2], yd[3]);
            yp[1] = make_float4(yd[4], yd[5], yd[6], yd[7]);
          }
        }
      };
      if (clamp) emit(std::true_type{});
      else emit(std::false_type{});
      if (wt == 0 && lane == 0) store_scale(scales, tok, sc, scale_fp16);
    }
    staged_grp = grp;
  }
  if constexpr (STAGE) {  // the last group's codes
    lds_barrier();
    if (staged_grp >= 0) store_staged(staged_grp);
  }
}

// ------------------------------------------------------------------------------------
// launchers and the variant table
// ------------------------------------------------------------------------------------
template <int N1, int N2, int WPT, bool HAS_C, bool DEEP>
hipError_t launch_reg(const kq_plan *p, const void *X, int64_t T, int64_t ldx, uint8_t *codes,
                      void *scales, float *y_debug, void *ws, hipStream_t stream) {
  using C = RegCfg<N1, N2, WPT, HAS_C, DEEP>;
  const int64_t ngroups = (T + C::TPI - 1) / C::TPI;
  const int grid = (int)(ngroups < (int64_t)p->grid_cap ? ngroups : (int64_t)p->grid_cap);
  hipLaunchKernelGGL((kq_reg_kernel<N1, N2, WPT, HAS_C, DEEP>), dim3(grid), dim3(kThreads), 0, stream,
                     static_cast<const __bf16 *>(X), T, ldx,
                     static_cast<const bf16x8 *>(p->p2op), static_cast<const bf16x8 *>(p->p1op),
                     p->c, p->clip, p->scale_dtype == KQ_FP16 ? 1 : 0, p->clip >= 0.935f ? 1 : 0,
                     codes, scales, y_debug);
  return hipGetLastError();
}

template <int N1, int N2, bool HAS_C, int BITS = 4>
hipError_t launch_cols(const kq_plan *p, const void *X, int64_t T, int64_t ldx, uint8_t *codes,
                       void *scales, float *y_debug, void *ws, hipStream_t stream) {
  using C = ColsCfg<N1, N2, HAS_C>;
  const int64_t ngroups = (T + C::TPI - 1) / C::TPI;
  const int grid = (int)(ngroups < (int64_t)p->grid_cap ? ngroups : (int64_t)p->grid_cap);
  // the debug output has its own instantiation, so that the timed kernel keeps its registers
  auto k = y_debug ? &kq_cols_kernel<N1, N2, HAS_C, true, BITS>
                   : &kq_cols_kernel<N1, N2, HAS_C, false, BITS>;
  hipLaunchKernelGGL(k, dim3(grid), dim3(C::THREADS), 0, stream,
                     static_cast<const __bf16 *>(X), T, ldx,
                     static_cast<const bf16x8 *>(p->p2op), static_cast<const bf16x8 *>(p->p1op),
                     p->c, p->clip, p->scale_dtype == KQ_FP16 ? 1 : 0, p->clip >= 0.935f ? 1 : 0,
                     codes, scales, y_debug);
  return hipGetLastError();
}

template <int N1, int N2, bool HAS_C, int BITS = 4, int N2R = N2>
hipError_t launch_stream(const kq_plan *p, const void *X, int64_t T, int64_t ldx, uint8_t *codes,
                         void *scales, float *y_debug, void *ws, hipStream_t stream) {
  using C = StreamCfg<N1, N2, HAS_C>;
  const int64_t ngroups = (T + C::WAVES - 1) / C::WAVES;
  const int grid = (int)(ngroups < (int64_t)p->grid_cap ? ngroups : (int64_t)p->grid_cap);
  // the debug output has its own instantiation so that the timed kernel keeps its
  // registers; both compute Y with the same per-accumulator MFMA order
  auto k = y_debug ? &kq_stream_kernel<N1, N2, HAS_C, true, BITS, N2R>
                   : &kq_stream_kernel<N1, N2, HAS_C, false, BITS, N2R>;
  hipLaunchKernelGGL(k, dim3(grid), dim3(C::THREADS), 0, stream,
                     static_cast<const __bf16 *>(X), T, ldx,
                     static_cast<const bf16x8 *>(p->p2op), static_cast<const bf16x8 *>(p->p1op),
                     p->c, p->p1_exp + p->p2_exp, p->c_absmax, p->clip,
                     p->scale_dtype == KQ_FP16 ? 1 : 0, p->clip >= 0.935f ? 1 : 0, codes, scales,
                     y_debug);
  return hipGetLastError();
}

template <int N1>
hipError_t launch_rsplit(const kq_plan *p, const void *X, int64_t T, int64_t ldx, uint8_t *codes,
                         void *scales, float *y_debug, void *, hipStream_t stream) {
  using C = RsplitCfg<N1>;
  const int grid = (int)(T < (int64_t)p->grid_cap ? T : (int64_t)p->grid_cap);
  auto k = y_debug ? &kq_rsplit_kernel<N1, true> : &kq_rsplit_kernel<N1, false>;
  hipLaunchKernelGGL(k, dim3(grid), dim3(C::THREADS), 0, stream, static_cast<const __bf16 *>(X), T,
                     ldx, static_cast<const f16x8 *>(p->p2op), static_cast<const f16x8 *>(p->p1op),
                     p->c, p->p1_exp + p->p2_exp, p->c_absmax, p->clip,
                     p->scale_dtype == KQ_FP16 ? 1 : 0, p->clip >= 0.935f ? 1 : 0, codes, scales,
                     y_debug);
  return hipGetLastError();
}

template <int N1, int N2, int BITS = 4>
hipError_t launch_colsc(const kq_plan *p, const void *X, int64_t T, int64_t ldx, uint8_t *codes,
                        void *scales, float *y_debug, void *, hipStream_t stream) {
  using C = ColsCCfg<N1, N2>;
  const int64_t ngroups = (T + C::TPI - 1) / C::TPI;
  const int grid = (int)(ngroups < (int64_t)p->grid_cap ? ngroups : (int64_t)p->grid_cap);
  auto k = y_debug ? &kq_colsc_kernel<N1, N2, true, BITS> : &kq_colsc_kernel<N1, N2, false, BITS>;
  if constexpr (C::CREG_OK) {
    if (p->c_f16)
      k = y_debug ? &kq_colsc_kernel<N1, N2, true, BITS, true> : &kq_colsc_kernel<N1, N2, false, BITS, true>;
  }
  hipLaunchKernelGGL(k, dim3(grid), dim3(C::THREADS), 0, stream, static_cast<const __bf16 *>(X), T,
                     ldx, static_cast<const f16x8 *>(p->p2op), static_cast<const f16x8 *>(p->p1op),
                     p->c, p->p1_exp + p->p2_exp, p->c_absmax, p->clip,
                     p->scale_dtype == KQ_FP16 ? 1 : 0, p->clip >= 0.935f ? 1 : 0, codes, scales,
                     y_debug);
  return hipGetLastError();
}

template <int N1, int N2, int BITS = 4>
hipError_t launch_pair(const kq_plan *p, const void *X, int64_t T, int64_t ldx, uint8_t *codes,
                       void *scales, float *y_debug, void *ws, hipStream_t stream) {
  using C = PairCfg<N1, N2>;
  const int grid = (int)(T < (int64_t)p->grid_cap ? T : (int64_t)p->grid_cap);
  auto k = y_debug ? &kq_pair_kernel<N1, N2, true, BITS> : &kq_pair_kernel<N1, N2, false, BITS>;
  hipLaunchKernelGGL(k, dim3(grid), dim3(C::THREADS), 0, stream,
                     static_cast<const __bf16 *>(X), T, ldx,
                     static_cast<const bf16x8 *>(p->p2op), static_cast<const bf16x8 *>(p->p1op),
                     p->clip, p->scale_dtype == KQ_FP16 ? 1 : 0, p->clip >= 0.935f ? 1 : 0, codes,
                     scales, y_debug);
  return hipGetLastError();
}

#define KQ_PAIR(A, B)                                                                  \
  kq_fused_variant{A, B, false, KQ_SPLIT_PAIR, 4, (B) / 2, PairCfg<A, B>::THREADS,          \
                   &launch_pair<A, B>,                                                 \
                   reinterpret_cast<const void *>(&kq_pair_kernel<A, B, false>),       \
                   "fused_mfma_bf16_pair_" #A "x" #B}
#define KQ_PAIR8(A, B)                                                                 \
  kq_fused_variant{A, B, false, KQ_SPLIT_PAIR, 8, (B) / 2, PairCfg<A, B>::THREADS,          \
                   &launch_pair<A, B, 8>,                                              \
                   reinterpret_cast<const void *>(&kq_pair_kernel<A, B, false, 8>),    \
                   "fused_mfma_bf16_pair_" #A "x" #B "_int8"}
template <int N2, int BITS = 4>
hipError_t launch_rows(const kq_plan *p, const void *X, int64_t T, int64_t ldx, uint8_t *codes,
                       void *scales, float *y_debug, void *ws, hipStream_t stream) {
  using C = RowsCfg<N2>;
  const int64_t ntiles = (T * p->n1 + C::ROWS - 1) / C::ROWS;
  const int64_t groups = (ntiles + C::WAVES - 1) / C::WAVES;
  const int grid = (int)(groups < (int64_t)p->grid_cap ? groups : (int64_t)p->grid_cap);
  auto k = y_debug ? &kq_rows_kernel<N2, true, BITS> : &kq_rows_kernel<N2, false, BITS>;
  hipLaunchKernelGGL(k, dim3(grid), dim3(C::THREADS), 0, stream, static_cast<const __bf16 *>(X),
                     T, p->n1, ldx, static_cast<const bf16x8 *>(p->p2op), p->clip,
                     p->scale_dtype == KQ_FP16 ? 1 : 0, p->clip >= 0.935f ? 1 : 0, codes,
                     scales, y_debug);
  return hipGetLastError();
}

#define KQ_STREAM(A, B)                                                                \
  kq_fused_variant{A, B, false, KQ_SPLIT_STREAM, 4, (B), StreamCfg<A, B>::THREADS,          \
                   &launch_stream<A, B, false>,                                        \
                   reinterpret_cast<const void *>(&kq_stream_kernel<A, B, false, false>), \
                   "fused_mfma_bf16_stream_" #A "x" #B}
#define KQ_STREAM8(A, B, HC, SUF)                                                      \
  kq_fused_variant{A, B, HC, KQ_SPLIT_STREAM, 8, (B), StreamCfg<A, B, HC>::THREADS,       \
                   &launch_stream<A, B, HC, 8>,                                        \
                   reinterpret_cast<const void *>(&kq_stream_kernel<A, B, HC, false, 8>), \
                   "fused_mfma_bf16_stream_" #A "x" #B SUF "_int8", nullptr, 0, 0, 0, (HC)}
// rows of 112 values in the 128-column layout (hidden 7168 = 64 x 112)
#define KQ_STREAM_P(A, B, BR)                                                          \
  kq_fused_variant{A, BR, false, KQ_SPLIT_STREAM, 4, (B), StreamCfg<A, B>::THREADS,         \
                   &launch_stream<A, B, false, 4, BR>,                                 \
                   reinterpret_cast<const void *>(&kq_stream_kernel<A, B, false, false, 4, BR>), \
                   "fused_mfma_bf16_stream_" #A "x" #BR}
#define KQ_STREAM_C(A, B)                                                              \
  kq_fused_variant{A, B, true, KQ_SPLIT_STREAM, 4, (B), StreamCfg<A, B, true>::THREADS,     \
                   &launch_stream<A, B, true>,                                         \
                   reinterpret_cast<const void *>(&kq_stream_kernel<A, B, true, false>), \
                   "fused_mfma_bf16_stream_" #A "x" #B "_c", nullptr, 0, 0, 0, true}
// the row split with a per-channel scale (n2 = 64): a token's 16-row blocks on their own waves
#define KQ_RSPLIT(A)                                                                   \
  kq_fused_variant{A, 64, true, KQ_SPLIT_RSPLIT, 4, 64, RsplitCfg<A>::THREADS, &launch_rsplit<A>, \
                   reinterpret_cast<const void *>(&kq_rsplit_kernel<A>),              \
                   "fused_mfma_bf16_rsplit_" #A "x64_c", nullptr, 0, 0, 0, true}
// the column split with a per-channel scale (x^ rounded once, Z in fp16)
#define KQ_COLSC(A, B)                                                                 \
  kq_fused_variant{A, B, true, KQ_SPLIT_COLS, 4, 32, ColsCCfg<A, B>::THREADS, &launch_colsc<A, B>, \
                   reinterpret_cast<const void *>(&kq_colsc_kernel<A, B>),            \
                   "fused_mfma_bf16_cols_" #A "x" #B "_c", nullptr, 0, 0, 0, true}
#define KQ_COLSC8(A, B)                                                                \
  kq_fused_variant{A, B, true, KQ_SPLIT_COLS, 8, 32, ColsCCfg<A, B>::THREADS, &launch_colsc<A, B, 8>, \
                   reinterpret_cast<const void *>(&kq_colsc_kernel<A, B, false, 8>),  \
                   "fused_mfma_bf16_cols_" #A "x" #B "_c_int8", nullptr, 0, 0, 0, true}
#define KQ_REG(A, B, WPT, HC, SUF)                                                     \
  kq_fused_variant{A, B, HC, WPT, 4, (B) / (WPT), kThreads, &launch_reg<A, B, WPT, HC, false>, \
                   reinterpret_cast<const void *>(&kq_reg_kernel<A, B, WPT, HC, false>), \
                   "fused_mfma_bf16_reg" #WPT "_" #A "x" #B SUF}
#define KQ_DEEP(A, B, HC, SUF)                                                         \
  kq_fused_variant{A, B, HC, KQ_SPLIT_DEEP, 4, (B), kThreads, &launch_reg<A, B, 1, HC, true>, \
                   reinterpret_cast<const void *>(&kq_reg_kernel<A, B, 1, HC, true>),   \
                   "fused_mfma_bf16_deep_" #A "x" #B SUF}
#define KQ_COLS(A, B, HC, SUF)                                                         \
  kq_fused_variant{A, B, HC, KQ_SPLIT_COLS, 4, 32, ColsCfg<A, B, HC>::THREADS, &launch_cols<A, B, HC>, \
                   reinterpret_cast<const void *>(&kq_cols_kernel<A, B, HC>),          \
                   "fused_mfma_bf16_cols_" #A "x" #B SUF}
#define KQ_COLS8(A, B, HC, SUF)                                                        \
  kq_fused_variant{A, B, HC, KQ_SPLIT_COLS, 8, 32, ColsCfg<A, B, HC>::THREADS, &launch_cols<A, B, HC, 8>, \
                   reinterpret_cast<const void *>(&kq_cols_kernel<A, B, HC, false, 8>), \
                   "fused_mfma_bf16_cols_" #A "x" #B SUF "_int8"}
#define KQ_ALL1(A, B)                                                                  \
  KQ_REG(A, B, 1, false, ""), KQ_REG(A, B, 1, true, "_c"), KQ_COLS(A, B, false, ""),    \
      KQ_COLSC(A, B)
#define KQ_ALL(A, B)                                                                   \
  KQ_ALL1(A, B), KQ_REG(A, B, 2, false, ""), KQ_REG(A, B, 2, true, "_c")

// Every work split that is built. The first match for a shape is its default, chosen by
// measurement on MI355X (T = 16384 and 65536, inputs rotated past the caches):
// - the stream kernel (one wave per token, next token in LDS by DMA) for n1 >= 32 with
//   n2 = 64 (with or without c) and for n2 = 128 without c: e.g. 64x64 31.8 us against
//   49.1 us for two waves per token with the token in registers, 32x64 with c 21.0 vs
//   44.8 us, 48x128 48.6 vs 74.6 us;
// - one wave per token with the token in registers for n1 = 16 with n2 = 64 (12.2 us at
//   16384 tokens, 33.3 us at 65536) and for 16..48 x 128 with c (16x128: 31.5 vs 44.5 us
//   for the column kernel);
// - the column kernel for 64 x 128 with c and everything larger.
// Stream plans switch to the pair kernel (or, where there is none, the column kernel) for
// small batches (kq_api.hip).
const kq_fused_variant kVariants[] = {
    // defaults
    KQ_REG(16, 32, 1, false, ""),  KQ_REG(16, 32, 1, true, "_c"),
    KQ_REG(32, 32, 1, false, ""),  KQ_REG(32, 32, 1, true, "_c"),
    KQ_REG(16, 64, 1, false, ""),  KQ_REG(16, 64, 1, true, "_c"),
    KQ_STREAM(32, 64),             KQ_STREAM_C(32, 64),
    KQ_STREAM(48, 64),             KQ_STREAM_C(48, 64),
    KQ_STREAM(64, 64),             KQ_STREAM_C(64, 64),
    KQ_STREAM(16, 128),            KQ_REG(16, 128, 1, true, "_c"),
    KQ_STREAM(32, 128),            KQ_REG(32, 128, 1, true, "_c"),
    KQ_STREAM(48, 128),            KQ_REG(48, 128, 1, true, "_c"),
    KQ_STREAM(64, 128),            KQ_COLSC(64, 128),
    KQ_COLS(80, 128, false, ""),   KQ_COLSC(80, 128),
    KQ_COLS(96, 128, false, ""),   KQ_COLSC(96, 128),
    KQ_COLS(112, 128, false, ""),  KQ_COLSC(112, 128),
    KQ_COLS(86, 128, false, ""),   KQ_COLSC(86, 128),   // 11008 (padded to 96)
    KQ_COLS(108, 128, false, ""),  KQ_COLSC(108, 128),  // 13824 (padded to 112)
    KQ_COLS(128, 128, false, ""),  KQ_COLSC(128, 128),
    // hidden sizes whose larger factor exceeds 128 (e.g. 28672 -> 128 x 224)
    KQ_COLS(128, 160, false, ""),  KQ_COLS(128, 192, false, ""),
    KQ_COLS(128, 224, false, ""),  KQ_COLS(128, 256, false, ""),
    // n2 not a multiple of 32, padded to one: the factors that minimise n1 + n2 for 1536
    // (32 x 48), 5120 (64 x 80), 7168 (64 x 112), 18432 (128 x 144), 6656 (64 x 104, n2 an
    // odd multiple of 8), and 3584 (56 x 64, n1 padded)
    KQ_COLS(32, 48, false, ""),    KQ_COLSC(32, 48),
    KQ_COLS(64, 80, false, ""),    KQ_COLSC(64, 80),
    KQ_STREAM_P(64, 128, 112),     KQ_COLS(64, 112, false, ""),   KQ_COLSC(64, 112),
    KQ_COLS(128, 144, false, ""),
    KQ_COLS(56, 64, false, ""),    KQ_COLSC(56, 64),
    KQ_COLS(64, 104, false, ""),   KQ_COLSC(64, 104),
    // 2560 (40 x 64, n1 padded to 48), 5632 (64 x 88, n2 padded to 96), 6144 (64 x 96) and
    // 8960 (80 x 112, n2 padded to 128)
    KQ_COLS(40, 64, false, ""),    KQ_COLSC(40, 64),
    KQ_COLS(64, 88, false, ""),    KQ_COLSC(64, 88),
    KQ_COLS(64, 96, false, ""),    KQ_COLSC(64, 96),
    KQ_COLS(80, 112, false, ""),   KQ_COLSC(80, 112),
    // the other splits, selectable with KQ_FLAG_SPLIT_*
    KQ_ALL1(16, 32), KQ_ALL1(32, 32), KQ_ALL(16, 64), KQ_ALL(32, 64), KQ_ALL(48, 64),
    KQ_ALL(64, 64), KQ_ALL(16, 128), KQ_ALL(32, 128), KQ_ALL(48, 128), KQ_ALL(64, 128),
    KQ_DEEP(64, 128, false, ""), KQ_DEEP(64, 64, false, ""), KQ_DEEP(64, 64, true, "_c"),
    KQ_STREAM(16, 64), KQ_STREAM(32, 64), KQ_STREAM(48, 64), KQ_STREAM(64, 64),
    KQ_STREAM_C(16, 64), KQ_STREAM_C(32, 64), KQ_STREAM_C(48, 64), KQ_STREAM_C(64, 64),
    KQ_RSPLIT(16), KQ_RSPLIT(32), KQ_RSPLIT(48), KQ_RSPLIT(64),
    // INT8 codes (stream kernel shapes)
    KQ_STREAM8(16, 64, false, ""), KQ_STREAM8(32, 64, false, ""), KQ_STREAM8(48, 64, false, ""),
    KQ_STREAM8(64, 64, false, ""), KQ_STREAM8(16, 128, false, ""), KQ_STREAM8(32, 128, false, ""),
    KQ_STREAM8(48, 128, false, ""), KQ_STREAM8(64, 128, false, ""),
    KQ_STREAM8(16, 64, true, "_c"), KQ_STREAM8(32, 64, true, "_c"), KQ_STREAM8(48, 64, true, "_c"),
    KQ_STREAM8(64, 64, true, "_c"),
    // INT8 codes on the column kernel: the shapes where it is the default (n1 > 64, or
    // 64 x 128 with c), e.g. FFN down-projection inputs kept at 8 bits
    KQ_COLSC8(64, 128),
    KQ_COLS8(80, 128, false, ""),  KQ_COLSC8(80, 128),
    KQ_COLS8(96, 128, false, ""),  KQ_COLSC8(96, 128),
    KQ_COLS8(112, 128, false, ""), KQ_COLSC8(112, 128),
    KQ_COLS8(86, 128, false, ""),  KQ_COLSC8(86, 128),
    KQ_COLS8(108, 128, false, ""), KQ_COLSC8(108, 128),
    KQ_COLS8(128, 128, false, ""), KQ_COLSC8(128, 128),
    KQ_COLS8(128, 160, false, ""), KQ_COLS8(128, 192, false, ""),
    KQ_COLS8(128, 224, false, ""), KQ_COLS8(128, 256, false, ""),
    KQ_COLS8(32, 48, false, ""),   KQ_COLSC8(32, 48),
    KQ_COLS8(64, 80, false, ""),   KQ_COLSC8(64, 80),
    KQ_COLS8(64, 112, false, ""),  KQ_COLSC8(64, 112),
    KQ_COLS8(128, 144, false, ""),
    KQ_COLS8(56, 64, false, ""),   KQ_COLSC8(56, 64),
    KQ_COLS8(64, 104, false, ""),  KQ_COLSC8(64, 104),
    KQ_COLS8(40, 64, false, ""),   KQ_COLSC8(40, 64),
    KQ_COLS8(64, 88, false, ""),   KQ_COLSC8(64, 88),
    KQ_COLS8(64, 96, false, ""),   KQ_COLSC8(64, 96),
    KQ_COLS8(80, 112, false, ""),  KQ_COLSC8(80, 112),
    KQ_STREAM(16, 128), KQ_STREAM(32, 128), KQ_STREAM(48, 128),
    KQ_PAIR(16, 64), KQ_PAIR(32, 64), KQ_PAIR(48, 64), KQ_PAIR(64, 64),
    KQ_PAIR(16, 128), KQ_PAIR(32, 128), KQ_PAIR(48, 128), KQ_PAIR(64, 128),
    KQ_PAIR8(16, 64), KQ_PAIR8(32, 64), KQ_PAIR8(48, 64), KQ_PAIR8(64, 64),
    KQ_PAIR8(16, 128), KQ_PAIR8(32, 128), KQ_PAIR8(48, 128), KQ_PAIR8(64, 128),
};

}  // namespace

const kq_fused_variant *kq_fused_lookup(int n1, int n2, bool has_c, int split, int bits) {
  for (const kq_fused_variant &e : kVariants)
    if (e.n1 == n1 && e.n2 == n2 && e.has_c == has_c && e.bits == bits &&
        (split == 0 || e.split == split))
      return &e;
  return nullptr;
}


namespace {
const kq_fused_variant kRowsVariants[] = {
#define KQ_ROWS(B, BITS, SUF)                                                          \
  kq_fused_variant{0, B, false, KQ_SPLIT_ROWS, BITS, 0, RowsCfg<B>::THREADS, &launch_rows<B, BITS>, \
                   reinterpret_cast<const void *>(&kq_rows_kernel<B, false, BITS>),       \
                   "fused_mfma_bf16_rows_" #B SUF}
    KQ_ROWS(64, 4, ""), KQ_ROWS(128, 4, ""), KQ_ROWS(64, 8, "_int8"), KQ_ROWS(128, 8, "_int8"),
};
}  // namespace

const kq_fused_variant *kq_fused_lookup_rows(int n2, int bits) {
  for (const kq_fused_variant &e : kRowsVariants)
    if (e.n2 == n2 && e.bits == bits) return &e;
  return nullptr;
}

// P2 as B operands of the rows kernel: [ks][tile a][lane L][slot v] =
//   P2[32 ks + 8 g + v][(L%16) NT + a],   g = L/16, NT = n2/16,
// so that after the MFMA lane L holds columns (L%16) NT + [0, NT) of its rows.
void kq_fused_arrange_p2_rows(const uint16_t *P2, int n2, uint16_t *out) {
  const int KS = n2 / 32, NT = n2 / 16;
  size_t o = 0;
  for (int ks = 0; ks < KS; ++ks)
    for (int a = 0; a < NT; ++a)
      for (int L = 0; L < 64; ++L)
        for (int v = 0; v < 8; ++v)
          out[o++] = P2[(size_t)(32 * ks + 8 * (L / 16) + v) * n2 + (L % 16) * NT + a];
}

size_t kq_fused_p1op_elems(int n1) {
  const int mt = (n1 + 15) / 16;  // n1 padded to whole 16-row tiles
  return (size_t)((mt * 16 + 31) / 32) * mt * 512;
}
// n2 that is not a multiple of 32 is padded with zero rows and columns to the next one
size_t kq_fused_p2op_elems(int n2) {
  const size_t n2p = (size_t)(n2 + 31) / 32 * 32;
  return n2p * n2p;
}

// P2 as stage-1 B operands, in blocks of `cb` output columns (one block per wave that
// shares a token): [block wb][step ks][tile a][lane L][slot v] =
//   P2[32 ks + 8 g + v][cb wb + (cb/4) b + 4 a + r],   g = L/16, b = (L%16)/4, r = L%4.
// Reduction slot (g, v) of step ks carries row 32 ks + 8 g + v. The 16 columns of tile a
// are spread so that, after stage 2, lane group g holds the cb/4 consecutive output
// columns cb wb + (cb/4) g + [0, cb/4) of a row of Y, i.e. cb/8 packed code bytes.
// Rows and columns from n2 up to the next multiple of 32 are zero.
void kq_fused_arrange_p2(const uint16_t *P2, int n2, int cb, uint16_t *out) {
  const int n2p = (n2 + 31) / 32 * 32;
  const int KS = n2p / 32, NB = n2p / cb, NT = cb / 16;
  size_t o = 0;
  for (int wb = 0; wb < NB; ++wb)
    for (int ks = 0; ks < KS; ++ks)
      for (int a = 0; a < NT; ++a)
        for (int L = 0; L < 64; ++L)
          for (int v = 0; v < 8; ++v) {
            const int g = L / 16, x = L % 16, b = x / 4, r = x % 4;
            const int i = 32 * ks + 8 * g + v, j = cb * wb + (cb / 4) * b + 4 * a + r;
            out[o++] = i < n2 && j < n2 ? P2[(size_t)i * n2 + j] : (uint16_t)0;
          }
}

// P1 as stage-2 B operands: [kk][tile t][lane L][slot v] =
//   P1[32 kk + 16 (v/4) + 4 g + (v%4)][16 t + L%16]   (zero where that row or column is
// >= n1: n1 is padded to whole 16-row tiles), i.e. the slot order of the stage-1
// accumulators of row tiles 2kk and 2kk+1.
void kq_fused_arrange_p1(const uint16_t *P1, int n1, uint16_t *out) {
  const int MT = (n1 + 15) / 16, KK = (MT * 16 + 31) / 32;
  size_t o = 0;
  for (int kk = 0; kk < KK; ++kk)
    for (int t = 0; t < MT; ++t)
      for (int L = 0; L < 64; ++L)
        for (int v = 0; v < 8; ++v) {
          const int g = L / 16;
          const int i = 32 * kk + 16 * (v / 4) + 4 * g + (v % 4), j = 16 * t + L % 16;
          out[o++] = i < n1 && j < n1 ? P1[(size_t)i * n1 + j] : (uint16_t)0;
        }
}
