// Kronecker transform + per-token quantization for factors too large for one CU's on-chip
// memory: the two designs of "FlatQuant: Fast Learnable Affine Quantization", Deep Dive:
// The fused kernel, Figure 8(b) and 8(c) (and Where It Breaks: on-chip memory overflow
// falls back to tiled or two-stage kernels with extra global-memory traffic).
//
// Both designs run two kernels that pass an intermediate through a device workspace the
// caller provides (kq_transform_quant_ws). They round like the fused kernels: V P2 on the
// matrix cores with fp32 accumulation, Z rounded once to bf16, P1^T Z on bf16 MFMA with
// fp32 accumulation, then the same quantizer. With a per-channel scale, Figure 8(c) feeds
// stage 1 with fp16 x c scaled by a power of two per 32-row item (and P2 as fp16), and
// Figure 8(b) with x c split into bf16 hi + lo planes.
//
//  * Figure 8(c), "two stages with a trip to global memory" (kq_z_kernel + kq_zq_kernel):
//    stage 1 computes Z = (x c) P2 for 32 rows of a token at a time and writes it to the
//    workspace as bf16, already in the operand order stage 2 reads (one contiguous 1 KiB
//    fragment per 16 x 32 block); stage 2 keeps P1 in LDS, streams a token's Z fragments
//    in, holds the token's whole Y in registers, and quantizes it in the same kernel.
//    Extra traffic: Z written and read once (2 x 2 bytes per padded value).
//  * Figure 8(b), "P1's non-reduction dimension tiled, quantization in a second kernel"
//    (kq_ptile_kernel + kq_yquant_kernel): one workgroup per token computes Z into
//    registers (each wave owns 32 columns of Z, exactly the columns of Y it produces, so Z
//    never leaves the wave), then applies P1 one tile of NTJ x 16 output rows (columns of
//    P1) at a time, each tile of P1 staged through LDS; every tile of Y is written to
//    global memory in fp32 while the token's absmax accumulates, and the step is stored.
//    The second kernel reads Y and the step and writes the codes. Extra traffic: Y in fp32
//    written and read once (8 bytes per value).
//
// Layouts are those of the column kernel: P2 as stage-1 B operands in blocks of 32 output
// columns (one block per wave), P1 as stage-2 B operands, so that after stage 2 a lane
// holds 8 consecutive output columns of a row of Y (one dword of INT4 codes).

#include "kq_internal.h"
#include "kq_device.h"
#include "kq_common.h"

namespace {

// workgroup size of the large-factor kernels: one wave per 32 (padded) columns of n2
constexpr int large_threads(int n2) { return 64 * ((n2 + 31) / 32); }

// HILO: x c staged as bf16 hi / lo planes (Figure 8(b) with c); without it, one plane (bf16 x,
// or fp16 x c for Figure 8(c) with c)
template <int N1, int N2, bool HAS_C, bool HILO = HAS_C>
struct LargeCfg {
  static_assert(N1 >= 16 && N1 <= 256, "n1 in [16, 256]");
  static_assert(N2 % 8 == 0 && N2 >= 32 && N2 <= 256, "n2 a multiple of 8 in [32, 256]");
  static constexpr int N2P = (N2 + 31) / 32 * 32;   // n2 padded with zero columns
  static constexpr int W = N2P / 32;                // waves per workgroup: 32 columns each
  static constexpr int THREADS = 64 * W;
  static constexpr int MT = (N1 + 15) / 16;         // 16-row tiles of V, Z and Y
  static constexpr int KK = (MT + 1) / 2;           // 32-row steps (stage-2 reduction)
  static constexpr int KS = N2P / 32;               // stage-1 reduction steps
  static constexpr int CH = N2 / 8;                 // 16-byte chunks per row of X
  static constexpr int CHP = N2P / 8;               // chunks per row in LDS
  static constexpr int ROW_CHUNKS = vrow_chunks<CHP>();
  static constexpr int VPLANES = HILO ? 2 : 1;      // hi (+ lo) bf16 planes of x*c
  static constexpr int PLANE = 32 * ROW_CHUNKS * 16;  // bytes of a 32-row plane in LDS
  static constexpr int STAGE = PLANE * VPLANES;       // one 32-row staging buffer
  static constexpr int STEP_CHUNKS = 32 * CH;         // 16-byte chunks of X per 32-row step
  static constexpr int CPT = (STEP_CHUNKS + THREADS - 1) / THREADS;
  static constexpr bool EVEN = CPT * THREADS == STEP_CHUNKS;
  static constexpr int ZT = N2P / 16;               // column tiles of Z
  static constexpr int P1_BYTES = KK * MT * 1024;   // P1 operands, n1 zero-padded
};

// One 32-row step (rows 32 kk .. 32 kk + 31 of token t) of X: each thread loads CPT chunks
// of 16 bytes into registers, then stores them (split into hi / lo planes with c) into an
// LDS staging buffer laid out like the column kernel's tile (vchunk_off: XOR-swizzled rows,
// or rows padded by one chunk). Rows at or beyond n1, and tokens at or beyond T, load zeros.
template <class C, int N1, int N2, bool HAS_C>
struct StepLoader {
  int row[C::CPT], cc[C::CPT];
  bool ok[C::CPT];
  uint4 pre[C::CPT];

  __device__ void init(int tid) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int q0 = tid + C::THREADS * i;
      ok[i] = C::EVEN || q0 < C::STEP_CHUNKS;
      const int q = ok[i] ? q0 : 0;
      row[i] = q / C::CH;
      cc[i] = q % C::CH;
    }
  }
  __device__ void load(const __bf16 *X, int64_t T, int64_t ldx, int64_t t, int kk) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int r = kk * 32 + row[i];
      if (ok[i] && t < T && r < N1)
        pre[i] = *reinterpret_cast<const uint4 *>(X + t * ldx + r * N2 + cc[i] * 8);
      else
        pre[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  // largest |x| of the loaded chunks (bf16 bit pattern of a non-negative value)
  __device__ uint32_t absmax() const {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) m = absmax_bf16(pre[i], m);
    return m;
  }
  // x c as fp16 scaled by 2^sx (one plane; rows beyond n1 hold zeros), SCALE = (sx != 0)
  template <bool SCALE>
  __device__ void store_f16(unsigned char *stage, const float *cvec, int kk, int sx) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      if (!ok[i]) continue;
      const int r = min(kk * 32 + row[i], N1 - 1);
      const float4 *cp = reinterpret_cast<const float4 *>(cvec + r * N2 + cc[i] * 8);
      const float4 a = cp[0], b = cp[1];
      const float cl[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      *reinterpret_cast<f16x8 *>(stage + vchunk_off<C::CHP>(row[i], cc[i])) =
          scale_round_f16<SCALE>(pre[i], cl, sx);
    }
  }
  __device__ void store(unsigned char *stage, const float *cvec, int kk) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      if (!ok[i]) continue;
      const int off = vchunk_off<C::CHP>(row[i], cc[i]);
      if constexpr (HAS_C) {
        // rows beyond n1 hold zeros; their c is read from a valid row and has no effect
        const int r = min(kk * 32 + row[i], N1 - 1);
        const float4 *cp = reinterpret_cast<const float4 *>(cvec + r * N2 + cc[i] * 8);
        const float4 a = cp[0], b = cp[1];
        const float cl[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        uint4 hi, lo;
        split_scaled(pre[i], cl, hi, lo);
        *reinterpret_cast<uint4 *>(stage + off) = hi;
        *reinterpret_cast<uint4 *>(stage + C::PLANE + off) = lo;
      } else {
        *reinterpret_cast<uint4 *>(stage + off) = pre[i];
      }
    }
  }
};

// Zero the padding chunks (n2 .. n2p) of every row of `nbuf` staging buffers: the loader
// never writes them, and they meet P2's zero rows (zero, not stale LDS contents, so that
// no NaN pattern can reach the MFMA).
template <class C, int N2>
__device__ __forceinline__ void zero_stage_padding(unsigned char *stage, int nbuf, int tid) {
  constexpr int PC = C::CHP - C::CH;
  if constexpr (PC > 0) {
    constexpr int PER_PLANE = 32 * PC;
    for (int q = tid; q < nbuf * C::VPLANES * PER_PLANE; q += C::THREADS) {
      const int pl = q / PER_PLANE, r = (q % PER_PLANE) / PC, c = C::CH + q % PC;
      *reinterpret_cast<uint4 *>(stage + pl * C::PLANE + vchunk_off<C::CHP>(r, c)) =
          make_uint4(0u, 0u, 0u, 0u);
    }
  }
}

// Stage 1 of one 32-row step for the wave's 32-column block: z[h] = the bf16 stage-2 A
// operand of column tile h (rows 32 kk + 16 (v / 4) + 4 g + v % 4 in its 8 slots).
// TIGHT: keep each reduction step's operand reads next to its MFMAs (a scheduling barrier
// per step), for kernels whose other live registers leave no room to read ahead.
template <class C, bool HAS_C, bool TIGHT = false>
__device__ __forceinline__ void stage1_step(const unsigned char *stage, const bf16x8 (&p2w)[C::KS][2],
                                            int lane, bf16x8 (&z)[2]) {
  const int g = lane >> 4, lr = lane & 15;
  f32x4 acc[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) acc[mt][0] = acc[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int off = vchunk_off<C::CHP>(mt * 16 + lr, ks * 4 + g);
      const bf16x8 a = *reinterpret_cast<const bf16x8 *>(stage + off);
      acc[mt][0] = mfma(a, p2w[ks][0], acc[mt][0]);
      acc[mt][1] = mfma(a, p2w[ks][1], acc[mt][1]);
      if constexpr (HAS_C) {
        const bf16x8 al = *reinterpret_cast<const bf16x8 *>(stage + C::PLANE + off);
        acc[mt][0] = mfma(al, p2w[ks][0], acc[mt][0]);
        acc[mt][1] = mfma(al, p2w[ks][1], acc[mt][1]);
      }
    }
    if constexpr (TIGHT) __builtin_amdgcn_sched_barrier(0);
  }
  z[0] = pack8(acc[0][0], acc[1][0]);
  z[1] = pack8(acc[0][1], acc[1][1]);
}

// Stage 1 of one 32-row step on fp16 operands (Figure 8(c) with a per-channel scale): the
// staged x^ = fp16(x c 2^sx) times P2's fp16 operands (P2 2^-f2), accumulated in fp32, then
// Z = Z' 2^e with e = f2 - sx (exact for normal results; e is wave-uniform, so the usual
// e = 0 skips it), rounded once to bf16 for the workspace.
template <class C>
__device__ __forceinline__ void stage1_step_f16(const unsigned char *stage, const bf16x8 (&p2w)[C::KS][2],
                                                int lane, int e, bf16x8 (&z)[2]) {
  const int g = lane >> 4, lr = lane & 15;
  f32x4 acc[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) acc[mt][0] = acc[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const f16x8 b0 = __builtin_bit_cast(f16x8, p2w[ks][0]), b1 = __builtin_bit_cast(f16x8, p2w[ks][1]);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const f16x8 a = *reinterpret_cast<const f16x8 *>(stage + vchunk_off<C::CHP>(mt * 16 + lr, ks * 4 + g));
      acc[mt][0] = mfma_f16(a, b0, acc[mt][0]);
      acc[mt][1] = mfma_f16(a, b1, acc[mt][1]);
    }
  }
  if (e != 0) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mt][h][r] = __builtin_ldexpf(acc[mt][h][r], e);
  }
  z[0] = pack8(acc[0][0], acc[1][0]);
  z[1] = pack8(acc[0][1], acc[1][1]);
}

template <class C>
__device__ __forceinline__ void load_p2_block(const bf16x8 *p2op, int wave, int lane,
                                              bf16x8 (&p2w)[C::KS][2]) {
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    p2w[ks][0] = p2op[((wave * C::KS + ks) * 2 + 0) * 64 + lane];
    p2w[ks][1] = p2op[((wave * C::KS + ks) * 2 + 1) * 64 + lane];
  }
}

// ------------------------------------------------------------------------------------
// Figure 8(c), stage 1: Z = (x c) P2 into the workspace (bf16 operand fragments)
// ------------------------------------------------------------------------------------
// Work items are (token, 32-row step) pairs over a persistent grid. The step's rows are
// loaded into registers one item ahead and stored into one of two LDS staging buffers, so
// one barrier per item orders the buffers. Each wave keeps its 32-column block of P2 in
// registers for the whole kernel. The workspace holds, per token, KK x ZT fragments of
// 1 KiB: fragment (kk, m2) at ((t KK + kk) ZT + m2) KiB, lane L's 16 bytes at L * 16.
// With a per-channel scale, stage 1 runs on fp16 operands: an item's x c is scaled by the
// power of two sx that its bound max|x| max|c| picks (f16_scale_exp: 0 for ordinary
// items). The rows of Z do not depend on each other, so the scale may differ between the
// items of a token; it is undone exactly on Z. The waves publish the next item's |x|
// maximum once its loads have landed, and a second barrier per item makes it visible.
template <int N1, int N2, bool HAS_C>
__global__ __launch_bounds__(large_threads(N2), HAS_C && N2 <= 224 ? 4 : 1) void kq_z_kernel(
    const __bf16 *__restrict__ X, int64_t T, int64_t ldx, const bf16x8 *__restrict__ p2op,
    const float *__restrict__ cvec, int p2_exp, float cmax, bf16x8 *__restrict__ zws) {
  using C = LargeCfg<N1, N2, HAS_C, false>;
  __shared__ __align__(16) unsigned char s_stage[2 * C::STAGE];
  __shared__ float s_xmax[2][C::W];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  zero_stage_padding<C, N2>(s_stage, 2, tid);
  bf16x8 p2w[C::KS][2];
  load_p2_block<C>(p2op, wave, lane, p2w);
  StepLoader<C, N1, N2, HAS_C> ld;
  ld.init(tid);

  const int64_t items = T * C::KK;
  int64_t it = blockIdx.x;
  if (it < items) ld.load(X, T, ldx, it / C::KK, (int)(it % C::KK));
  // publish the loaded item's |x| maximum into s_xmax[b] (with c)
  auto publish_xmax = [&](int b) {
    const float v = wave_max_uniform(__uint_as_float(ld.absmax() << 16));
    if (lane == 0) s_xmax[b][wave] = v;
  };
  if constexpr (HAS_C) {
    if (it < items) publish_xmax(0);
    lds_barrier();  // the first item's maxima visible
  }
  for (int b = 0; it < items; it += gridDim.x, b ^= 1) {
    const int64_t t = it / C::KK;
    const int kk = (int)(it % C::KK);
    unsigned char *stage = s_stage + b * C::STAGE;
    int sx = 0;
    if constexpr (HAS_C) {
      float xm = 0.f;
#pragma unroll
      for (int w = 0; w < C::W; ++w) xm = fmaxf(xm, s_xmax[b][w]);
      sx = __builtin_amdgcn_readfirstlane(f16_scale_exp(__fmul_rn(xm, cmax)));
      if (sx == 0) ld.template store_f16<false>(stage, cvec, kk, 0);
      else ld.template store_f16<true>(stage, cvec, kk, sx);
    } else {
      ld.store(stage, cvec, kk);
    }
    lds_barrier();  // this buffer is complete; the other one is free (read an item ago)
    const int64_t nxt = it + gridDim.x;
    if (nxt < items) ld.load(X, T, ldx, nxt / C::KK, (int)(nxt % C::KK));
    bf16x8 z[2];
    if constexpr (HAS_C) stage1_step_f16<C>(stage, p2w, lane, p2_exp - sx, z);
    else stage1_step<C, false>(stage, p2w, lane, z);
    bf16x8 *zt = zws + ((t * C::KK + kk) * C::ZT + 2 * wave) * 64 + lane;
    zt[0] = z[0];
    zt[64] = z[1];
    if constexpr (HAS_C) {
      if (nxt < items) publish_xmax(b ^ 1);  // the next item's loads have landed
      lds_barrier();  // its maxima visible (s_xmax[b ^ 1] was last read an item ago)
    }
  }
}

// ------------------------------------------------------------------------------------
// Figure 8(c), stage 2 + quantizer: Y = P1^T Z from the workspace, absmax, codes
// ------------------------------------------------------------------------------------
// One token per workgroup iteration (persistent grid). P1's operands stay in LDS. Wave w
// owns column tiles 2w, 2w+1 of Y: it reads its KK x 2 Z fragments (one 16-byte load per
// fragment and lane), accumulates Y^T for those 32 columns and all rows in registers, and
// loads the next token's fragments as soon as the MFMAs have consumed the current ones,
// so that they arrive during the epilogue. The absmax of the token's W waves meets in LDS
// (two slots, alternating per token: one barrier per token).
template <int N1, int N2, bool YDBG, int BITS>
__global__ __launch_bounds__(large_threads(N2)) void kq_zq_kernel(
    const bf16x8 *__restrict__ zws, int64_t T, const bf16x8 *__restrict__ p1op, float clip,
    int scale_fp16, int clip_allows_no_clamp, uint8_t *__restrict__ codes,
    void *__restrict__ scales, float *__restrict__ ydbg) {
  using C = LargeCfg<N1, N2, false>;
  constexpr int n = N1 * N2;
  __shared__ __align__(16) unsigned char s_p1[C::P1_BYTES];
  __shared__ float s_red[2][C::W];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, lr = lane & 15;
  {
    const uint4 *s = reinterpret_cast<const uint4 *>(p1op);
    uint4 *d = reinterpret_cast<uint4 *>(s_p1);
    for (int i = tid; i < C::P1_BYTES / 16; i += C::THREADS) d[i] = s[i];
  }
  lds_barrier();
  const bf16x8 *sp1 = reinterpret_cast<const bf16x8 *>(s_p1);

  bf16x8 zf[C::KK][2];
  auto load_z_range = [&](int64_t t, int k0, int k1) {
    const bf16x8 *zt = zws + (t * C::KK * C::ZT + 2 * wave) * 64 + lane;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      if (kk < k0 || kk >= k1) continue;
      zf[kk][0] = zt[(kk * C::ZT) * 64];
      zf[kk][1] = zt[(kk * C::ZT + 1) * 64];
    }
  };
  int64_t tok = blockIdx.x;
  if (tok < T) load_z_range(tok, 0, C::KK);
  for (int it = 0; tok < T; tok += gridDim.x, ++it) {
    f32x4 yacc[2][C::MT];
#pragma unroll
    for (int nt = 0; nt < C::MT; ++nt) yacc[0][nt] = yacc[1][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
#pragma unroll
      for (int nt = 0; nt < C::MT; ++nt) {
        const bf16x8 b = sp1[(kk * C::MT + nt) * 64 + lane];
        yacc[0][nt] = mfma(zf[kk][0], b, yacc[0][nt]);
        yacc[1][nt] = mfma(zf[kk][1], b, yacc[1][nt]);
        // with the whole Y tile and Z in registers (n1 > 224), read P1 at most 4
        // operands ahead
        if constexpr (C::MT > 14) {
          if (nt % 4 == 3) __builtin_amdgcn_sched_barrier(0);
        }
      }
      // (n1 > 192: no step's P1 read ahead of the previous step)
      if constexpr (C::MT > 12) __builtin_amdgcn_sched_barrier(0);
    }
    // The next token's fragments go out now and land during the epilogue; where Y's
    // accumulators and all of Z do not fit next to the epilogue's registers, the second
    // half of the steps (n1 > 192), or all of them (n1 > 224), are loaded after the codes
    // are written.
    constexpr int KPRE = C::MT > 14 ? 0 : C::MT > 12 ? C::KK / 2 : C::KK;
    const int64_t nxt = tok + gridDim.x;
    if (nxt < T) load_z_range(nxt, 0, KPRE);

    // lane holds Y[16 nt + lr][32 wave + 8 g + 4 h + r]
    float m = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int nt = 0; nt < C::MT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(yacc[h][nt][r]));
    m = wave_max_uniform(m);
    if (lane == 0) s_red[it & 1][wave] = m;
    lds_barrier();
    float amax = 0.f;
#pragma unroll
    for (int w = 0; w < C::W; ++w) amax = fmaxf(amax, s_red[it & 1][w]);
    const TokenScale sc = token_scale(amax, clip, scale_fp16, BITS == 4 ? 7.0f : 127.0f);

    constexpr int RB = N2 * BITS / 8;  // code bytes per row of Y
    const int col0 = wave * 32 + g * 8;
    if (col0 < N2) {  // padded columns are not stored
      uint8_t *crow = codes + tok * (int64_t)(n * BITS / 8) + col0 * BITS / 8;
      // one scalar branch on the clamp (INT4: skipped where the clip ratio rules it out)
      auto emit = [&](auto clamp_tag) {
#pragma unroll
        for (int nt = 0; nt < C::MT; ++nt) {
          const int j = nt * 16 + lr;
          if (j >= N1) continue;  // nor padded rows
          uint8_t *dst = crow + j * RB;
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
            float4 *yp = reinterpret_cast<float4 *>(ydbg + tok * (int64_t)n + j * N2 + col0);
            yp[0] = make_float4(yacc[0][nt][0], yacc[0][nt][1], yacc[0][nt][2], yacc[0][nt][3]);
            yp[1] = make_float4(yacc[1][nt][0], yacc[1][nt][1], yacc[1][nt][2], yacc[1][nt][3]);
          }
        }
      };
      if (BITS == 8 || __builtin_amdgcn_readfirstlane(clamp_needed(clip_allows_no_clamp, sc.s32) ? 1 : 0))
        emit(std::true_type{});
      else
        emit(std::false_type{});
    }
    if (wave == 0 && lane == 0) store_scale(scales, tok, sc, scale_fp16);
    if (KPRE < C::KK && nxt < T) load_z_range(nxt, KPRE, C::KK);
  }
}

// ------------------------------------------------------------------------------------
// Figure 8(b): Z in registers, P1 applied one tile of its output dimension at a time
// ------------------------------------------------------------------------------------
// One token per workgroup iteration. Stage 1 runs the token's 32-row steps through one
// LDS staging buffer (two barriers per step) and keeps each step's Z fragments for the
// wave's 32 columns in registers (KK x 2 operands). Stage 2 walks P1's output dimension
// in tiles of NTJ x 16 columns of P1 (rows of Y): the workgroup copies the tile's
// operands (KK x NTJ fragments) into one of two LDS buffers, and each wave computes its
// 32 columns of those rows of Y, writes them to `yout` in fp32 (row-major, row stride n)
// and folds them into its absmax. The token's step is stored at the end; the codes come
// from the second kernel.
template <int N1, int NTJ>
struct PtileCfg {
  static constexpr int MT = (N1 + 15) / 16;
  static constexpr int KK = (MT + 1) / 2;
  static constexpr int JT = (MT + NTJ - 1) / NTJ;       // tiles of P1's output dimension
  static constexpr int TILE_BYTES = KK * NTJ * 1024;    // one tile's operands
};

template <int N1, int N2, bool HAS_C, int NTJ>
__global__ __launch_bounds__(large_threads(N2)) void kq_ptile_kernel(
    const __bf16 *__restrict__ X, int64_t T, int64_t ldx, const bf16x8 *__restrict__ p2op,
    const bf16x8 *__restrict__ p1op, const float *__restrict__ cvec, float clip, int scale_fp16,
    float *__restrict__ yout, void *__restrict__ scales) {
  using C = LargeCfg<N1, N2, HAS_C>;
  using PC = PtileCfg<N1, NTJ>;
  constexpr int n = N1 * N2;
  __shared__ __align__(16) unsigned char s_stage[C::STAGE];
  __shared__ __align__(16) unsigned char s_p1[2][PC::TILE_BYTES];
  __shared__ float s_red[C::W];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, lr = lane & 15;

  zero_stage_padding<C, N2>(s_stage, 1, tid);
  bf16x8 p2w[C::KS][2];
  load_p2_block<C>(p2op, wave, lane, p2w);
  StepLoader<C, N1, N2, HAS_C> ld;
  ld.init(tid);

  // operands of P1 tile jt (fragments (kk, nt) for nt in [NTJ jt, NTJ jt + NTJ), zero
  // beyond MT) into LDS buffer b: fragment (kk, q) at (kk NTJ + q) KiB
  auto copy_tile = [&](int jt, int b) {
    uint4 *d = reinterpret_cast<uint4 *>(s_p1[b]);
    const uint4 *s = reinterpret_cast<const uint4 *>(p1op);
    for (int i = tid; i < PC::TILE_BYTES / 16; i += C::THREADS) {
      const int f = i / 64, u = i % 64, kk = f / NTJ, q = f % NTJ, nt = jt * NTJ + q;
      d[i] = nt < C::MT ? s[(kk * C::MT + nt) * 64 + u] : make_uint4(0u, 0u, 0u, 0u);
    }
  };

  int64_t tok = blockIdx.x;
  if (tok < T) ld.load(X, T, ldx, tok, 0);
  for (; tok < T; tok += gridDim.x) {
    // ---- stage 1: Z for the wave's 32 columns, all rows, as bf16 operands ----
    bf16x8 zf[C::KK][2];
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      ld.store(s_stage, cvec, kk);
      if (kk == 0) copy_tile(0, 0);
      lds_barrier();
      if (kk + 1 < C::KK) ld.load(X, T, ldx, tok, kk + 1);
      else if (tok + gridDim.x < T) ld.load(X, T, ldx, tok + gridDim.x, 0);
      stage1_step<C, HAS_C, (HAS_C && C::KK * 8 + C::KS * 8 > 96)>(s_stage, p2w, lane, zf[kk]);
      lds_barrier();  // staging buffer free again (and, after the last step, P1 tile 0 visible)
    }
    // ---- stage 2, tile by tile of P1's output dimension ----
    float m = 0.f;
    const int col0 = wave * 32 + g * 8;
#pragma unroll 1
    for (int jt = 0; jt < PC::JT; ++jt) {
      if (jt + 1 < PC::JT) copy_tile(jt + 1, (jt + 1) & 1);
      const bf16x8 *sp1 = reinterpret_cast<const bf16x8 *>(s_p1[jt & 1]);
      f32x4 yacc[2][NTJ];
#pragma unroll
      for (int q = 0; q < NTJ; ++q) yacc[0][q] = yacc[1][q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk)
#pragma unroll
        for (int q = 0; q < NTJ; ++q) {
          const bf16x8 b = sp1[(kk * NTJ + q) * 64 + lane];
          yacc[0][q] = mfma(zf[kk][0], b, yacc[0][q]);
          yacc[1][q] = mfma(zf[kk][1], b, yacc[1][q]);
        }
      // lane holds Y[16 (NTJ jt + q) + lr][col0 + 4 h + r]; padded rows and columns are 0
#pragma unroll
      for (int q = 0; q < NTJ; ++q) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(yacc[h][q][r]));
        const int j = (jt * NTJ + q) * 16 + lr;
        if (j < N1 && col0 < N2) {
          float4 *yp = reinterpret_cast<float4 *>(yout + tok * (int64_t)n + j * N2 + col0);
          yp[0] = make_float4(yacc[0][q][0], yacc[0][q][1], yacc[0][q][2], yacc[0][q][3]);
          yp[1] = make_float4(yacc[1][q][0], yacc[1][q][1], yacc[1][q][2], yacc[1][q][3]);
        }
      }
      lds_barrier();  // tile jt + 1 copied; every wave is done with tile jt's buffer
    }
    m = wave_max_uniform(m);
    if (lane == 0) s_red[wave] = m;
    lds_barrier();
    float amax = 0.f;
#pragma unroll
    for (int w = 0; w < C::W; ++w) amax = fmaxf(amax, s_red[w]);
    if (tid == 0) store_scale(scales, tok, token_scale(amax, clip, scale_fp16), scale_fp16);
    // s_red is written again only after the next token's stage-1 barriers
  }
}

// The second kernel of Figure 8(b): codes from Y (fp32, row stride n) and the stored step.
// inv = fp32(1 / s) of the stored step, exactly as the step's own kernel would have formed
// it (a step stored as 0 gives inv = 0 and zero codes). Each thread quantizes 8 values of
// a token into one dword of INT4 codes (or two of INT8); grid-stride over all of them.
template <int BITS>
__global__ __launch_bounds__(256) void kq_yquant_kernel(const float *__restrict__ Y, int64_t T,
                                                        int n, const void *__restrict__ scales,
                                                        int scale_fp16, int clip_allows_no_clamp,
                                                        uint8_t *__restrict__ codes) {
  const int64_t per_tok = n / 8;
  const int64_t total = T * per_tok;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = e / per_tok;
    const float s = scale_fp16 ? (float)reinterpret_cast<const _Float16 *>(scales)[t]
                               : reinterpret_cast<const float *>(scales)[t];
    const float inv = (s == 0.f) ? 0.f : __fdiv_rn(1.0f, s);
    const float4 a = reinterpret_cast<const float4 *>(Y)[2 * e];
    const float4 b = reinterpret_cast<const float4 *>(Y)[2 * e + 1];
    if constexpr (BITS == 8) {
      const u32x2_t w = {quant4x8(a.x, a.y, a.z, a.w, inv), quant4x8(b.x, b.y, b.z, b.w, inv)};
      reinterpret_cast<u32x2_t *>(codes)[e] = w;
    } else {
      const float yv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      // the clamp bound holds for the stored step as for s32 (normal fp16 or exact fp32)
      reinterpret_cast<uint32_t *>(codes)[e] =
          clamp_needed(clip_allows_no_clamp, s) ? quant8<true>(yv, inv) : quant8<false>(yv, inv);
    }
  }
}

// ------------------------------------------------------------------------------------
// launchers and the variant table
// ------------------------------------------------------------------------------------
template <int N1, int N2, bool HAS_C, int BITS>
hipError_t launch_twostage(const kq_plan *p, const void *X, int64_t T, int64_t ldx, uint8_t *codes,
                           void *scales, float *y_debug, void *ws, hipStream_t stream) {
  using C = LargeCfg<N1, N2, HAS_C>;
  bf16x8 *z = static_cast<bf16x8 *>(ws);
  const int64_t items = T * C::KK;
  const int g1 = (int)(items < (int64_t)p->grid_cap ? items : (int64_t)p->grid_cap);
  hipLaunchKernelGGL((kq_z_kernel<N1, N2, HAS_C>), dim3(g1), dim3(C::THREADS), 0, stream,
                     static_cast<const __bf16 *>(X), T, ldx, static_cast<const bf16x8 *>(p->p2op),
                     p->c, p->p2_exp, p->c_absmax, z);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int g2 = (int)(T < (int64_t)p->grid_cap2 ? T : (int64_t)p->grid_cap2);
  auto k = y_debug ? &kq_zq_kernel<N1, N2, true, BITS> : &kq_zq_kernel<N1, N2, false, BITS>;
  hipLaunchKernelGGL(k, dim3(g2), dim3(C::THREADS), 0, stream, static_cast<const bf16x8 *>(z), T,
                     static_cast<const bf16x8 *>(p->p1op), p->clip, p->scale_dtype == KQ_FP16 ? 1 : 0,
                     p->clip >= 0.935f ? 1 : 0, codes, scales, y_debug);
  return hipGetLastError();
}

// rows of Y (in 16-row tiles) per tile of P1: 4, or 2 with a per-channel scale (the hi /
// lo planes of stage 1 leave fewer registers for Y's accumulators)
constexpr int ptile_ntj(int n1, bool has_c) {
  return (n1 + 15) / 16 < (has_c ? 2 : 4) ? (n1 + 15) / 16 : (has_c ? 2 : 4);
}

template <int N1, int N2, bool HAS_C, int BITS>
hipError_t launch_ptile(const kq_plan *p, const void *X, int64_t T, int64_t ldx, uint8_t *codes,
                        void *scales, float *y_debug, void *ws, hipStream_t stream) {
  using C = LargeCfg<N1, N2, HAS_C>;
  // Y goes to the caller's debug buffer when there is one, else to the workspace
  float *y = y_debug ? y_debug : static_cast<float *>(ws);
  const int g1 = (int)(T < (int64_t)p->grid_cap ? T : (int64_t)p->grid_cap);
  hipLaunchKernelGGL((kq_ptile_kernel<N1, N2, HAS_C, ptile_ntj(N1, HAS_C)>), dim3(g1), dim3(C::THREADS), 0,
                     stream, static_cast<const __bf16 *>(X), T, ldx,
                     static_cast<const bf16x8 *>(p->p2op), static_cast<const bf16x8 *>(p->p1op), p->c,
                     p->clip, p->scale_dtype == KQ_FP16 ? 1 : 0, y, scales);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t units = T * (int64_t)(N1 * N2 / 8);
  const int64_t blocks = (units + 255) / 256;
  const int g2 = (int)(blocks < (int64_t)p->grid_cap2 ? blocks : (int64_t)p->grid_cap2);
  hipLaunchKernelGGL((kq_yquant_kernel<BITS>), dim3(g2), dim3(256), 0, stream,
                     static_cast<const float *>(y), T, N1 * N2, static_cast<const void *>(scales),
                     p->scale_dtype == KQ_FP16 ? 1 : 0, p->clip >= 0.935f ? 1 : 0, codes);
  return hipGetLastError();
}

// Z bytes per token of the two-stage design (KK x ZT fragments of 1 KiB)
constexpr size_t z_bytes(int n1, int n2) {
  return (size_t)(((n1 + 15) / 16 + 1) / 2) * (size_t)((n2 + 31) / 32 * 2) * 1024;
}

#define KQ_TWOSTAGE(A, B, HC, SUF)                                                        \
  kq_fused_variant{A, B, HC, KQ_SPLIT_TWOSTAGE, 4, 32, LargeCfg<A, B, HC>::THREADS,           \
                   &launch_twostage<A, B, HC, 4>,                                          \
                   reinterpret_cast<const void *>(&kq_z_kernel<A, B, HC>),                 \
                   "twostage_mfma_bf16_" #A "x" #B SUF,                                    \
                   reinterpret_cast<const void *>(&kq_zq_kernel<A, B, false, 4>),          \
                   LargeCfg<A, B, HC>::THREADS, z_bytes(A, B), 0, false, HC}
#define KQ_PTILE(A, B, HC, SUF)                                                           \
  kq_fused_variant{A, B, HC, KQ_SPLIT_PTILE, 4, 32, LargeCfg<A, B, HC>::THREADS,              \
                   &launch_ptile<A, B, HC, 4>,                                             \
                   reinterpret_cast<const void *>(&kq_ptile_kernel<A, B, HC, ptile_ntj(A, HC)>), \
                   "ptile_mfma_bf16_" #A "x" #B SUF,                                       \
                   reinterpret_cast<const void *>(&kq_yquant_kernel<4>), 256,              \
                   (size_t)(A) * (B) * 4, 0}
#define KQ_LARGE(A, B, HC, SUF) KQ_TWOSTAGE(A, B, HC, SUF), KQ_PTILE(A, B, HC, SUF)

// The first match for a shape (with the split left to the plan) is its default. Figure
// 8(b) with a per-channel scale stops at n2p * 32 + n1 <= 8384 (168 x 176): beyond that, a
// wave's P2 block, the token's Z and the hi / lo planes of x*c exceed its 256 registers,
// and Figure 8(c) covers the shape. Shapes:
// the factors kq_choose_factors gives for hidden sizes whose smaller factor exceeds 128
// (25600 = 160 x 160, 27648 = 144 x 192, 29568 = 168 x 176, 53248 = 208 x 256,
// 65536 = 256 x 256), and n1 = 128 with n2 in 160 .. 256 with a per-channel scale (the
// column kernel has them only without one).
const kq_fused_variant kLargeVariants[] = {
    KQ_LARGE(160, 160, false, ""), KQ_LARGE(160, 160, true, "_c"),
    KQ_LARGE(144, 192, false, ""), KQ_LARGE(144, 192, true, "_c"),
    KQ_LARGE(168, 176, false, ""), KQ_LARGE(168, 176, true, "_c"),
    KQ_LARGE(208, 256, false, ""), KQ_TWOSTAGE(208, 256, true, "_c"),
    KQ_LARGE(256, 256, false, ""), KQ_TWOSTAGE(256, 256, true, "_c"),
    KQ_LARGE(128, 160, true, "_c"), KQ_LARGE(128, 192, true, "_c"),
    KQ_LARGE(128, 224, true, "_c"), KQ_LARGE(128, 256, true, "_c"),
    // also without c, next to the column kernel's single-kernel design (selectable)
    KQ_LARGE(128, 224, false, ""),
};

}  // namespace

const kq_fused_variant *kq_large_lookup(int n1, int n2, bool has_c, int split, int bits) {
  if (bits != 4) return nullptr;
  for (const kq_fused_variant &e : kLargeVariants)
    if (e.n1 == n1 && e.n2 == n2 && e.has_c == has_c && (split == 0 || e.split == split))
      return &e;
  return nullptr;
}
