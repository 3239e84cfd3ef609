// Device helpers shared by the MFMA kernels of libkq (gfx950): operand types, the
// LDS-only barrier, wave reductions of the absmax, bf16 packing, the hi/lo split of x*c,
// the per-token step and the INT4 / INT8 code packers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) unsigned short u16x2_t;

namespace {


// Workgroup barrier that orders LDS only. __syncthreads() also fences global memory,
// which makes every wave wait for its in-flight prefetch loads at each barrier; these
// kernels only exchange data through LDS, so the release/acquire is restricted to it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Max over the wave of a non-negative value, returned wave-uniform: within each row of 16
// lanes with DPP (quad swaps, half-row and row mirrors), then the four row maxima read
// into scalars. No LDS round trips.
// Maxima of absolute values (x >= 0, never NaN: the in-lane maxima start from 0 and
// fmaxf drops NaN operands). For such x the float order is the order of the bit patterns
// as unsigned integers, so the cross-lane steps use the integer max, which takes its DPP
// operand directly (every DPP pattern used here reads a valid lane: no "old" value).
__device__ __forceinline__ float max_nn(float a, float b) {
  const uint32_t x = __float_as_uint(a), y = __float_as_uint(b);
  return __uint_as_float(x > y ? x : y);
}
template <int CTRL>
__device__ __forceinline__ float dpp_read(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ float dpp_step(float v) {
  return max_nn(v, dpp_read<CTRL>(v));
}
__device__ __forceinline__ float wave_max_uniform(float v) {
  v = dpp_step<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_step<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_step<0x141>(v);  // row_half_mirror
  v = dpp_step<0x140>(v);  // row_mirror: every lane of a row holds the row max
  const int i = __float_as_int(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(i, 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(i, 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(i, 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(i, 48));
  return max_nn(max_nn(r0, r1), max_nn(r2, r3));
}

__device__ __forceinline__ bf16x8 pack8(const f32x4 &a, const f32x4 &b) {
  bf16x8 r;
  r[0] = (__bf16)a[0]; r[1] = (__bf16)a[1]; r[2] = (__bf16)a[2]; r[3] = (__bf16)a[3];
  r[4] = (__bf16)b[0]; r[5] = (__bf16)b[1]; r[6] = (__bf16)b[2]; r[7] = (__bf16)b[3];
  return r;
}

// x (8 bf16) * c (8 fp32) in fp32, split into hi = bf16(x*c) and lo = bf16(x*c - hi):
// hi + lo carries ~16 significant bits, so one extra MFMA pass over lo keeps the
// per-channel scale from adding a second bf16 rounding to the transform.
// Per pair of values: 2 unpacks, 2 multiplies, one paired RNE conversion for hi, 2 unpacks
// of hi, 2 subtractions, one paired conversion for lo (5 VALU per value).
__device__ __forceinline__ void split_scaled(const uint4 &raw, const float *c, uint4 &hi,
                                             uint4 &lo) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float s0 = __fmul_rn(__uint_as_float(w[e] << 16), c[2 * e]);
    const float s1 = __fmul_rn(__uint_as_float(w[e] & 0xFFFF0000u), c[2 * e + 1]);
    const bf16x2_t hv = {(__bf16)s0, (__bf16)s1};  // v_cvt_pk_bf16_f32
    h[e] = __builtin_bit_cast(uint32_t, hv);
    // opaque to the optimizer, so that hi's fp32 values are unpacked from this word
    // instead of converting s0 a second time
    asm("" : "+v"(h[e]));
    const float r0 = __fsub_rn(s0, __uint_as_float(h[e] << 16));
    const float r1 = __fsub_rn(s1, __uint_as_float(h[e] & 0xFFFF0000u));
    const bf16x2_t lv = {(__bf16)r0, (__bf16)r1};
    l[e] = __builtin_bit_cast(uint32_t, lv);
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// Per-token step: s32 = fp32(fp32(clip * a) / 7), stored as fp16 (RNE) or fp32; the
// codes use the stored step, inv = fp32(1 / s) (0 when s == 0, giving all-zero codes). An
// fp32 step of at most 2^-128 has no finite reciprocal: it is treated as an underflow, so
// it is stored as 0 and the codes are 0 (an fp16 step is either 0 or at least 2^-24).
struct TokenScale {
  float s32;
  _Float16 s16;
  float inv;
};

// qmax = 2^(b-1) - 1: 7 for INT4 codes, 127 for INT8 codes
__device__ __forceinline__ TokenScale token_scale(float amax, float clip, int scale_fp16,
                                                  float qmax = 7.0f) {
  TokenScale t;
  t.s32 = __fdiv_rn(__fmul_rn(clip, amax), qmax);
  t.s16 = (_Float16)t.s32;
  const float sf = scale_fp16 ? (float)t.s16 : t.s32;
  t.inv = (sf == 0.f) ? 0.f : __fdiv_rn(1.0f, sf);
  if (__builtin_isinf(t.inv)) {
    t.s32 = 0.f;
    t.inv = 0.f;
  }
  return t;
}

__device__ __forceinline__ void store_scale(void *scales, int64_t tok, const TokenScale &t,
                                            int scale_fp16) {
  if (scale_fp16) reinterpret_cast<_Float16 *>(scales)[tok] = t.s16;
  else reinterpret_cast<float *>(scales)[tok] = t.s32;
}

// Quantize 8 consecutive values into one dword of 4-bit two's-complement codes (value e
// in bits 4e..4e+3). Per value: v = fp32(y * inv); adding 1.5*2^23 + 8 in fp32 rounds v
// to the nearest integer with ties to even (the sum's unit in the last place is 1 and
// 1.5*2^23 + 8 is even) and leaves q + 8 in the low mantissa bits, for |v| < 2^22; the
// integer clamp of the bit pattern is the clamp of q to [-8, 7]. The two steps are
// separate roundings on purpose (no fused multiply-add). Codes are assembled as q + 8
// and turned into two's complement with one xor per dword. CLAMP = false is only used
// when every |v| < 7.5 is guaranteed (see clamp_needed), where the clamp is a no-op.
template <bool CLAMP = true>
__device__ __forceinline__ uint32_t quant8(const float (&y)[8], float inv) {
  constexpr float kMagic = 12582920.0f;   // 1.5 * 2^23 + 8, bit pattern 0x4B400008
  constexpr int kLo = 0x4B400000, kHi = 0x4B40000F;
  uint32_t u[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float t = __fadd_rn(__fmul_rn(y[e], inv), kMagic);
    u[e] = CLAMP ? (uint32_t)min(max(__float_as_int(t), kLo), kHi) : __float_as_uint(t);
  }
  // byte k of the result = u[2k] | u[2k+1] << 4 (bits above the low byte are ignored)
  const uint32_t p0 = (u[1] << 4) | u[0], p1 = (u[3] << 4) | u[2];
  const uint32_t p2 = (u[5] << 4) | u[4], p3 = (u[7] << 4) | u[6];
  const uint32_t lo = __builtin_amdgcn_perm(p1, p0, 0x0C0C0400u);  // [p0.b0, p1.b0, 0, 0]
  const uint32_t hi = __builtin_amdgcn_perm(p3, p2, 0x04000C0Cu);  // [0, 0, p2.b0, p3.b0]
  return (lo | hi) ^ 0x88888888u;
}

// Whether the clamp to [-8, 7] can change a code. With |y| <= a, inv = fp32(1/s) and
// s the stored step of s32 = fp32(fp32(clip a)/7): for an fp16 step in the normal
// range (relative rounding error <= 2^-11; an fp32 step is exact) every
// |fp32(y inv)| <= (7/clip)(1 + 2^-10) < 7.5 once clip >= 0.935 (checked on the host),
// so rint gives |q| <= 7. A zero or overflowed step gives inv = 0 and q = 0.
__device__ __forceinline__ bool clamp_needed(int clip_allows_no_clamp, float s32) {
  return !(clip_allows_no_clamp && (s32 >= 6.103515625e-05f || s32 == 0.f));
}

__device__ __forceinline__ f32x4 mfma_f16(const f16x8 &a, const f16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Largest |x| of 8 bf16 values (bit patterns in raw), as the bit pattern of a
// non-negative bf16 in the low 16 bits (integer order = magnitude order for |x|)
__device__ __forceinline__ uint32_t absmax_bf16(const uint4 &raw, uint32_t m) {
  u16x2_t v = __builtin_bit_cast(u16x2_t, raw.x & 0x7FFF7FFFu);
  v = __builtin_elementwise_max(v, __builtin_bit_cast(u16x2_t, raw.y & 0x7FFF7FFFu));
  v = __builtin_elementwise_max(v, __builtin_bit_cast(u16x2_t, raw.z & 0x7FFF7FFFu));
  v = __builtin_elementwise_max(v, __builtin_bit_cast(u16x2_t, raw.w & 0x7FFF7FFFu));
  const uint32_t a = v[0] > v[1] ? v[0] : v[1];
  return a > m ? a : m;
}

// x (8 bf16) * c (8 fp32) in fp32, scaled by 2^s (exact for normal results), rounded once
// to fp16 (round to nearest even): the stage-1 operand of the kernels that run both
// contractions on fp16 operands. SCALE = false is the s = 0 case (no ldexp); callers pick
// it with a wave-uniform branch, since ordinary tokens need no scaling.
template <bool SCALE = true>
__device__ __forceinline__ f16x8 scale_round_f16(const uint4 &raw, const float *c, int s) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  f16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float s0 = __fmul_rn(__uint_as_float(w[e] << 16), c[2 * e]);
    float s1 = __fmul_rn(__uint_as_float(w[e] & 0xFFFF0000u), c[2 * e + 1]);
    if constexpr (SCALE) {
      s0 = __builtin_ldexpf(s0, s);
      s1 = __builtin_ldexpf(s1, s);
    }
    r[2 * e] = (_Float16)s0;
    r[2 * e + 1] = (_Float16)s1;
  }
  return r;
}

// largest |v| over a run of accumulators (and m). Written as one running chain
// m = max(m, |v|): the compiler then pairs the steps into v_max3_f32 with absolute-value
// modifiers (two values per instruction). Nested as max(m, max(|a|, |b|)) it first
// canonicalizes every MFMA result with an extra v_max_f32.
template <int K>
__device__ __forceinline__ float absmax_acc(const f32x4 (&v)[K], float m) {
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(v[k][r]));
  return m;
}

// The quantizer's reciprocal for Y = Y' 2^ty, applied to Y' directly. With t = 2^ty,
// fp32(Y' * fp32(inv t)) equals fp32(fp32(Y' t) * inv) whenever both scalings are exact,
// since both then round the same real product: inv t must be normal (checked by scaling
// back) or inv = 0, and every nonzero Y' t must be a normal, finite fp32. The latter holds
// when amax = max|Y'| t is finite and ty >= -78: each nonzero |Y'| is at least 2^-48 (a
// sum of products of fp16 values, all multiples of 2^-24, accumulated in fp32). Returns
// false when the kernel has to scale Y itself.
__device__ __forceinline__ bool fold_scale(float inv, int ty, float amax, float &inv_y) {
  inv_y = __builtin_ldexpf(inv, ty);
  if (ty < -78 || !__builtin_isfinite(amax)) return false;
  if (inv == 0.f) return true;
  return __builtin_isfinite(inv_y) && inv_y >= 1.17549435e-38f &&
         __builtin_ldexpf(inv_y, -ty) == inv;
}

// Power-of-two exponent s that brings a token's values into fp16's range before the
// conversion, from a bound zmax on their magnitudes: 0 when zmax lies in [2^-8, 2^15) (the
// values convert as they are), else 14 - floor(log2 zmax), which puts zmax * 2^s in
// [2^14, 2^15) (clamped to [-126, 127]). A function of zmax alone, so every kernel that
// sees the same values picks the same s.
__device__ __forceinline__ int f16_scale_exp(float zmax) {
  const int eb = (int)((__float_as_uint(zmax) >> 23) & 0xFFu);  // biased exponent
  if (eb >= 127 - 8 && eb < 127 + 15) return 0;
  const int s = 14 - (eb - 127);
  return s < -126 ? -126 : (s > 127 ? 127 : s);
}

// 8 fp32 values (two accumulators) -> fp16 operand, each scaled by 2^s first (exact for
// normal results) and rounded to nearest even
__device__ __forceinline__ f16x8 pack8_f16(const f32x4 &a, const f32x4 &b, int s) {
  f16x8 r;
  if (s == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[e] = (_Float16)a[e];
      r[4 + e] = (_Float16)b[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[e] = (_Float16)__builtin_ldexpf(a[e], s);
      r[4 + e] = (_Float16)__builtin_ldexpf(b[e], s);
    }
  }
  return r;
}

__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}


// INT8: 4 consecutive values -> one dword of two's-complement bytes (value e in byte e).
// Adding 1.5*2^23 in fp32 rounds v = fp32(y * inv) to the nearest integer, ties to even,
// and leaves q in the low mantissa bits (|v| < 2^22); clamping the bit pattern clamps q to
// [-128, 127], and its low byte is then q as a two's-complement byte.
__device__ __forceinline__ uint32_t quant4x8(float y0, float y1, float y2, float y3, float inv) {
  constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23, bit pattern 0x4B400000
  constexpr int kLo = 0x4B400000 - 128, kHi = 0x4B400000 + 127;
  const float y[4] = {y0, y1, y2, y3};
  uint32_t u[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    u[e] = (uint32_t)min(max(__float_as_int(__fadd_rn(__fmul_rn(y[e], inv), kMagic)), kLo), kHi);
  const uint32_t lo = __builtin_amdgcn_perm(u[1], u[0], 0x0C0C0400u);  // [u0.b0, u1.b0, 0, 0]
  const uint32_t hi = __builtin_amdgcn_perm(u[3], u[2], 0x04000C0Cu);  // [0, 0, u2.b0, u3.b0]
  return lo | hi;
}


// Row layout of a token tile in LDS with CH 16-byte chunks per row: an XOR swizzle of the
// chunks when CH is a power of two; for rows of 20, 24 or 28 chunks, an XOR of (R / 2) % 8
// within each aligned group of 8 chunks (24) or of (R / 2) % 4 within each aligned group of
// 4 chunks (20, 28) (rows padded by one chunk read at half speed on MI355X: an LDS access
// probe measured 8 cycles per 16-byte wave read against 4, and (R / 2) % 4 on 24-chunk rows
// also conflicts); else rows padded by one chunk.
template <int CH>
constexpr bool vrow_swz4() { return (CH & (CH - 1)) != 0 && CH % 4 == 0 && CH >= 20; }
template <int CH>
constexpr int vrow_xmask() { return CH % 8 == 0 ? 7 : 3; }
template <int CH>
constexpr int vrow_chunks() { return (CH & (CH - 1)) == 0 || vrow_swz4<CH>() ? CH : CH + 1; }

// byte offset of 16-byte chunk `cc` of row `r` of a token tile in LDS
template <int CH>
__device__ __forceinline__ int vchunk_off(int r, int cc) {
  if constexpr ((CH & (CH - 1)) == 0) return (r * CH + (cc ^ (r & (CH - 1)))) * 16;
  else if constexpr (vrow_swz4<CH>()) return (r * CH + (cc ^ ((r >> 1) & vrow_xmask<CH>()))) * 16;
  else return (r * (CH + 1) + cc) * 16;
}

// Quantize a wave's whole Y tile (lane holds yacc[m2][nt] = 4 consecutive columns of row
// 16 nt + lr) into packed code words w[nt][q] (8 consecutive columns each).
template <bool CLAMP, int MT, int NT>
__device__ __forceinline__ void quant_tile(const f32x4 (&yacc)[NT][MT], float inv,
                                           uint32_t (&w)[MT][NT / 2]) {
#pragma unroll
  for (int nt = 0; nt < MT; ++nt)
#pragma unroll
    for (int q = 0; q < NT / 2; ++q) {
      const float yv[8] = {yacc[2 * q][nt][0],     yacc[2 * q][nt][1],     yacc[2 * q][nt][2],
                           yacc[2 * q][nt][3],     yacc[2 * q + 1][nt][0], yacc[2 * q + 1][nt][1],
                           yacc[2 * q + 1][nt][2], yacc[2 * q + 1][nt][3]};
      w[nt][q] = quant8<CLAMP>(yv, inv);
    }
}

// N2R: the real row length when the tile is laid out for N2 = 128 and rows hold only
// N2R = 112 values (lane group 3 then holds 16 real and 16 padding columns). Rows of codes
// are then 56 bytes, and the 16 rows of block nt are 896 contiguous bytes: 56 words of 16
// bytes, seven whole 128-byte lines. Lane k < 56 gathers word k across the wave and writes
// it, so one store instruction writes each line whole. Dword d of word k is byte b = 16k + 4d
// of the block, i.e. byte cb = b % 56 of row r = b / 56, held by lane r + 16 (cb / 16) as
// its dword (cb % 16) / 4 = (d + 2r) % 4. A lane of an odd row swaps its two 8-byte halves
// first, so that each lane's dword d is the one its reader asks for in slot d.
// The whole wave must be active (cross-lane reads).
template <int N1, int N2, int N2R = N2>
__device__ __forceinline__ void store_codes(uint8_t *codes, int64_t tok, const uint32_t (*w)[N2 / 32],
                                            int lr, int g) {
  static_assert(N2R == N2 || (N2 == 128 && N2R == 112), "padded stream rows: 112 of 128");
  uint8_t *crow = codes + tok * (int64_t)(N1 * N2R / 2);
  if constexpr (N2R != N2) {
    constexpr int kBlk = 16 * N2R / 2;  // bytes of codes per 16-row block
    const int lane = lr + 16 * g;
    const bool odd = (lr & 1) != 0;
    int src[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int b = 16 * lane + 4 * d, r = b / (N2R / 2), cb = b - r * (N2R / 2);
      src[d] = 4 * (lane < kBlk / 16 ? r + 16 * (cb >> 4) : lane);
    }
#pragma unroll
    for (int nt = 0; nt < N1 / 16; ++nt) {
      const uint32_t s[4] = {odd ? w[nt][2] : w[nt][0], odd ? w[nt][3] : w[nt][1],
                             odd ? w[nt][0] : w[nt][2], odd ? w[nt][1] : w[nt][3]};
      u32x4_t v;
#pragma unroll
      for (int d = 0; d < 4; ++d) v[d] = (uint32_t)__builtin_amdgcn_ds_bpermute(src[d], (int)s[d]);
      if (lane < kBlk / 16)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(crow + nt * kBlk + 16 * lane));
    }
    return;
  }
#pragma unroll
  for (int nt = 0; nt < N1 / 16; ++nt) {
    uint8_t *dst = crow + (nt * 16 + lr) * (N2R / 2) + g * (N2 / 8);
    if constexpr (N2 == 128) {
      const u32x4_t v = {w[nt][0], w[nt][1], w[nt][2], w[nt][3]};
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(dst));
    } else {
      const u32x2_t v = {w[nt][0], w[nt][1]};
      __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t *>(dst));
    }
  }
}

}  // namespace
