// Host side of libkq: argument checks, plan construction (factor re-layout, clip ratio),
// kernel selection and launch. See include/kq.h for the contract of each entry point.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "kq_internal.h"

namespace {

bool is_aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elem_size(kq_dtype d) {
  switch (d) {
    case KQ_BF16: return 2;
    case KQ_FP16: return 2;
    case KQ_FP32: return 4;
  }
  return 0;
}

// clip = sigmoid(alpha) in double with the host libm, rounded once to fp32
// ("FlatQuant: Fast Learnable Affine Quantization", Symbol Map: alpha_a is mapped into
// (0, 1) by a sigmoid). The two branches avoid overflow of exp for large |alpha|.
float clip_from_alpha(float alpha) {
  const double a = (double)alpha;
  if (isinf(a)) return a > 0 ? 1.0f : 0.0f;
  double v;
  if (a >= 0) {
    v = 1.0 / (1.0 + exp(-a));
  } else {
    const double e = exp(a);
    v = e / (1.0 + e);
  }
  return (float)v;
}

// fp32 -> bf16 bit pattern, round to nearest even (finite values)
uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

// bf16 patterns -> fp16 patterns of P * 2^-f (round to nearest even) in place; returns f,
// the smallest exponent >= 0 that keeps max |P| 2^-f below 2^15
int to_scaled_f16(std::vector<uint16_t> &v) {
  float mx = 0.f;
  for (uint16_t b : v) mx = fmaxf(mx, fabsf(bf16_to_f32(b)));
  int f = 0;
  while (ldexpf(mx, -f) >= 32768.0f) ++f;
  for (uint16_t &b : v) {
    const _Float16 h = (_Float16)ldexpf(bf16_to_f32(b), -f);
    memcpy(&b, &h, 2);
  }
  return f;
}

void free_plan_buffers(kq_plan *p) {
  if (!p) return;
  if (p->p1op) (void)hipFree(p->p1op);
  if (p->p2op) (void)hipFree(p->p2op);
  if (p->p1f) (void)hipFree(p->p1f);
  if (p->p2f) (void)hipFree(p->p2f);
  if (p->c) (void)hipFree(p->c);
  if (p->small_p2op) (void)hipFree(p->small_p2op);
}

kq_status upload(void **dst, const void *src, size_t bytes, hipStream_t s) {
  if (hipMalloc(dst, bytes) != hipSuccess) {
    *dst = nullptr;
    return KQ_ERR_OUT_OF_MEMORY;
  }
  if (hipMemcpyAsync(*dst, src, bytes, hipMemcpyHostToDevice, s) != hipSuccess) return KQ_ERR_HIP;
  return KQ_OK;
}

// Scratch memory of kq_transform_quant_noalloc: the workspace of the two-kernel designs
// for callers that cannot allocate. One copy per GPU, held from the library's load until
// the process ends; every such call on a GPU shares it, so calls that overlap on one GPU
// (different streams, or host threads without ordering) race on it. Nothing in it needs
// to start at zero: both designs write every byte of the intermediate they read back.
constexpr size_t kScratchBytes = KQ_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of each device's copy of `scratch`, looked up once per device with that
// device current. In host code the name `scratch` is only a host-side stand-in symbol:
// every use of the memory from the host goes through these addresses.
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mutex;

kq_status scratch_address(int dev, void **out) {
  if (dev < 0 || dev >= kMaxDevices) return KQ_ERR_UNSUPPORTED;
  void *a = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!a) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    a = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!a) {
      if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return KQ_ERR_HIP;
      g_scratch_addr[dev].store(a, std::memory_order_release);
    }
  }
  *out = a;
  return KQ_OK;
}

const char *dtype_name(kq_dtype d) {
  return d == KQ_BF16 ? "bf16" : d == KQ_FP32 ? "fp32" : d == KQ_FP16 ? "fp16" : "?";
}

}  // namespace

bool kq_log_on() {
  static const bool on = [] {
    const char *e = getenv("KQ_LOG");
    return e && *e && strcmp(e, "0") != 0;
  }();
  return on;
}

void kq_logf(const char *fmt, ...) {
  char line[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(line, sizeof line, fmt, ap);
  va_end(ap);
  fprintf(stderr, "[kq] %s\n", line);
}

extern "C" {

int kq_version(void) { return 10200; }

const char *kq_status_string(kq_status s) {
  switch (s) {
    case KQ_OK: return "ok";
    case KQ_ERR_INVALID_ARG: return "invalid argument";
    case KQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case KQ_ERR_ALIGNMENT: return "misaligned pointer or leading dimension";
    case KQ_ERR_OUT_OF_MEMORY: return "out of memory";
    case KQ_ERR_HIP: return "HIP runtime error";
    case KQ_ERR_WORKSPACE: return "the call needs a larger device workspace";
  }
  return "unknown status";
}

kq_status kq_choose_factors(int64_t n, int *n1, int *n2) {
  if (n < 1 || !n1 || !n2 || n > (int64_t)1 << 40) return KQ_ERR_INVALID_ARG;
  int64_t d = (int64_t)sqrt((double)n);
  while (d * d > n) --d;
  while ((d + 1) * (d + 1) <= n) ++d;
  for (; d >= 1; --d) {
    if (n % d == 0) {
      if (n / d > 0x7fffffff) return KQ_ERR_INVALID_ARG;
      *n1 = (int)d;
      *n2 = (int)(n / d);
      return KQ_OK;
    }
  }
  return KQ_ERR_INVALID_ARG;
}

// A plan of the rows kernel: identity left factor (P1 == NULL), one step per row of V.
kq_status create_rows_plan(kq_plan **out, int n1, int n2, kq_dtype scale_dtype, const void *P2,
                           float alpha, int bits, hipStream_t s) {
  const kq_fused_variant *fv = kq_fused_lookup_rows(n2, bits);
  if (!fv || n1 > (1 << 20)) return KQ_ERR_UNSUPPORTED;  // rows kernel: n1 <= 2^20
  kq_plan *p = static_cast<kq_plan *>(calloc(1, sizeof(kq_plan)));
  if (!p) return KQ_ERR_OUT_OF_MEMORY;
  p->n1 = n1;
  p->n2 = n2;
  p->n = n1 * n2;
  p->x_dtype = KQ_BF16;
  p->scale_dtype = scale_dtype;
  p->clip = clip_from_alpha(alpha);
  p->kind = KQ_KIND_FUSED_MFMA;
  p->kname = fv->name;
  p->launch = fv->launch;
  p->per_row = 1;
  p->bits = bits;
  kq_status st = KQ_OK;
  std::vector<uint16_t> h2((size_t)n2 * n2), a2((size_t)n2 * n2);
  int dev = 0, ncu = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipMemcpyAsync(h2.data(), P2, h2.size() * 2, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess) {
    st = KQ_ERR_HIP;
    goto fail;
  }
  p->device = dev;
  kq_fused_arrange_p2_rows(h2.data(), n2, a2.data());
  if ((st = upload(&p->p2op, a2.data(), a2.size() * 2, s)) != KQ_OK) goto fail;
  if (hipStreamSynchronize(s) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fv->kernel_symbol, fv->threads, 0) !=
          hipSuccess) {
    st = KQ_ERR_HIP;
    goto fail;
  }
  if (per_cu < 1) { st = KQ_ERR_UNSUPPORTED; goto fail; }
  p->grid_cap = ncu * per_cu;
  *out = p;
  return KQ_OK;
fail:
  (void)hipStreamSynchronize(s);  // no copy still in flight into a buffer freed below
  free_plan_buffers(p);
  free(p);
  return st;
}

static kq_status create_ex_impl(kq_plan **out, int n1, int n2, kq_dtype x_dtype,
                                kq_dtype scale_dtype, const void *P1, const void *P2,
                                const float *c, float alpha, void *stream, unsigned flags) {
  if (!out) return KQ_ERR_INVALID_ARG;
  *out = nullptr;
  if (n1 < 1 || n2 < 1 || (int64_t)n1 * n2 > (1 << 24)) return KQ_ERR_INVALID_ARG;
  const int n = n1 * n2;
  if (n % 2) return KQ_ERR_INVALID_ARG;
  if (x_dtype != KQ_BF16 && x_dtype != KQ_FP32) return KQ_ERR_INVALID_ARG;
  if (scale_dtype != KQ_FP16 && scale_dtype != KQ_FP32) return KQ_ERR_INVALID_ARG;
  if (isnan(alpha)) return KQ_ERR_INVALID_ARG;
  if (flags & KQ_FLAG_PER_ROW) {
    // identity left factor only; bf16; no per-channel scale; no other flag but INT8
    if (P1 || !P2 || c || x_dtype != KQ_BF16 || (flags & ~(KQ_FLAG_PER_ROW | KQ_FLAG_INT8)))
      return KQ_ERR_INVALID_ARG;
    return create_rows_plan(out, n1, n2, scale_dtype, P2, alpha, (flags & KQ_FLAG_INT8) ? 8 : 4,
                            static_cast<hipStream_t>(stream));
  }
  if (!P1 || !P2) return KQ_ERR_INVALID_ARG;
  const int bits = (flags & KQ_FLAG_INT8) ? 8 : 4;
  // INT8 codes: bf16 MFMA kernels only (no generic fallback)
  if (bits == 8 && (x_dtype != KQ_BF16 || (flags & KQ_FLAG_FORCE_GENERIC))) return KQ_ERR_INVALID_ARG;
  flags &= ~KQ_FLAG_INT8;
  const unsigned split_flags =
      flags & (KQ_FLAG_SPLIT_REG1 | KQ_FLAG_SPLIT_REG2 | KQ_FLAG_SPLIT_COLS | KQ_FLAG_SPLIT_DEEP |
               KQ_FLAG_SPLIT_STREAM | KQ_FLAG_SPLIT_PAIR | KQ_FLAG_SPLIT_TWOSTAGE |
               KQ_FLAG_SPLIT_PTILE | KQ_FLAG_SPLIT_RSPLIT);
  if (flags & ~(KQ_FLAG_FORCE_GENERIC | split_flags)) return KQ_ERR_INVALID_ARG;
  if ((split_flags & (split_flags - 1)) != 0) return KQ_ERR_INVALID_ARG;  // at most one
  if (split_flags && ((flags & KQ_FLAG_FORCE_GENERIC) || x_dtype != KQ_BF16))
    return KQ_ERR_INVALID_ARG;
  const int split = split_flags == KQ_FLAG_SPLIT_REG1   ? KQ_SPLIT_REG1
                    : split_flags == KQ_FLAG_SPLIT_REG2 ? KQ_SPLIT_REG2
                    : split_flags == KQ_FLAG_SPLIT_COLS ? KQ_SPLIT_COLS
                    : split_flags == KQ_FLAG_SPLIT_DEEP ? KQ_SPLIT_DEEP
                    : split_flags == KQ_FLAG_SPLIT_STREAM ? KQ_SPLIT_STREAM
                    : split_flags == KQ_FLAG_SPLIT_PAIR ? KQ_SPLIT_PAIR
                    : split_flags == KQ_FLAG_SPLIT_TWOSTAGE ? KQ_SPLIT_TWOSTAGE
                    : split_flags == KQ_FLAG_SPLIT_PTILE ? KQ_SPLIT_PTILE
                    : split_flags == KQ_FLAG_SPLIT_RSPLIT ? KQ_SPLIT_RSPLIT
                                                        : 0;
  const bool large_split = split == KQ_SPLIT_TWOSTAGE || split == KQ_SPLIT_PTILE;

  // kernel choice (pure host logic, before any HIP call)
  const char *kname = nullptr;
  const void *ksym = nullptr;
  kq_launch_fn fn = nullptr;
  int kind = -1;
  const kq_fused_variant *fv = nullptr;
  if (x_dtype == KQ_BF16 && !(flags & KQ_FLAG_FORCE_GENERIC)) {
    // single-kernel designs first; factors beyond them (or a forced two-kernel split) go
    // to the designs of kq_large.hip
    fv = large_split ? nullptr : kq_fused_lookup(n1, n2, c != nullptr, split, bits);
    if (!fv && (split == 0 || large_split)) fv = kq_large_lookup(n1, n2, c != nullptr, split, bits);
    if (fv) {
      fn = fv->launch;
      kname = fv->name;
      ksym = fv->kernel_symbol;
      kind = KQ_KIND_FUSED_MFMA;
    }
  }
  if (!fn && x_dtype == KQ_FP32 && !(flags & KQ_FLAG_FORCE_GENERIC) && bits == 4) {
    fv = kq_f32_lookup(n1, n2, c != nullptr);
    if (fv) {
      fn = fv->launch;
      kname = fv->name;
      ksym = fv->kernel_symbol;
      kind = KQ_KIND_FUSED_F32;
    }
  }
  if (!fn) {
    if (split || bits == 8 || n > kq_generic_max_n()) return KQ_ERR_UNSUPPORTED;
    fn = kq_generic_launcher(&kname, &ksym);
    kind = KQ_KIND_GENERIC;
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  kq_plan *p = static_cast<kq_plan *>(calloc(1, sizeof(kq_plan)));
  if (!p) return KQ_ERR_OUT_OF_MEMORY;
  p->n1 = n1;
  p->n2 = n2;
  p->n = n;
  p->x_dtype = x_dtype;
  p->scale_dtype = scale_dtype;
  p->clip = clip_from_alpha(alpha);
  p->kind = kind;
  p->kname = kname;
  p->launch = fn;
  p->bits = bits;

  kq_status st = KQ_OK;
  const size_t es = elem_size(x_dtype);
  std::vector<unsigned char> h1((size_t)n1 * n1 * es), h2((size_t)n2 * n2 * es);
  std::vector<float> hc;
  int dev = 0, ncu = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) { st = KQ_ERR_HIP; goto fail; }
  p->device = dev;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    st = KQ_ERR_HIP;
    goto fail;
  }
  if (hipMemcpyAsync(h1.data(), P1, h1.size(), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipMemcpyAsync(h2.data(), P2, h2.size(), hipMemcpyDeviceToHost, s) != hipSuccess) {
    st = KQ_ERR_HIP;
    goto fail;
  }
  if (c) {
    hc.resize(n);
    if (hipMemcpyAsync(hc.data(), c, (size_t)n * 4, hipMemcpyDeviceToHost, s) != hipSuccess) {
      st = KQ_ERR_HIP;
      goto fail;
    }
  }
  if (hipStreamSynchronize(s) != hipSuccess) { st = KQ_ERR_HIP; goto fail; }

  if (kind == KQ_KIND_FUSED_MFMA) {
    std::vector<uint16_t> a1(kq_fused_p1op_elems(n1)), a2(kq_fused_p2op_elems(n2));
    // The factors' element patterns the kernels take: bf16 as given, or, for the variants
    // that run both contractions on fp16 operands, P * 2^-f as fp16 (round to nearest
    // even) with f >= 0 the smallest exponent that keeps max |P| 2^-f below 2^15 (fp16
    // holds up to 65504); f is undone on Y.
    std::vector<uint16_t> e1((const uint16_t *)h1.data(), (const uint16_t *)h1.data() + (size_t)n1 * n1);
    std::vector<uint16_t> e2((const uint16_t *)h2.data(), (const uint16_t *)h2.data() + (size_t)n2 * n2);
    if (fv->f16_ops || fv->f16_p2) {
      if (fv->f16_ops) p->p1_exp = to_scaled_f16(e1);
      p->p2_exp = to_scaled_f16(e2);
      float cm = 0.f;
      int f16ok = 1;
      for (size_t i = 0; i < hc.size(); ++i) {
        const float a = fabsf(hc[i]);
        cm = fmaxf(cm, a);
        if (a != 0.f && !(a >= 0x1p-14f && a < 0x1p15f)) f16ok = 0;
      }
      p->c_absmax = cm;
      p->c_f16 = c ? f16ok : 0;
    }
    kq_fused_arrange_p1(e1.data(), n1, a1.data());
    kq_fused_arrange_p2(e2.data(), n2, fv->p2_block, a2.data());
    if ((st = upload(&p->p1op, a1.data(), a1.size() * 2, s)) != KQ_OK) goto fail;
    if ((st = upload(&p->p2op, a2.data(), a2.size() * 2, s)) != KQ_OK) goto fail;
    if (c && (st = upload(reinterpret_cast<void **>(&p->c), hc.data(), hc.size() * 4, s)) != KQ_OK)
      goto fail;
    if (hipStreamSynchronize(s) != hipSuccess) { st = KQ_ERR_HIP; goto fail; }
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ksym, fv->threads, 0) !=
        hipSuccess) {
      st = KQ_ERR_HIP;
      goto fail;
    }
    if (fv->kernel_symbol2) {  // two-kernel design: the second kernel's grid and the workspace
      int per_cu2 = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu2, fv->kernel_symbol2, fv->threads2,
                                                       0) != hipSuccess) {
        st = KQ_ERR_HIP;
        goto fail;
      }
      if (per_cu2 < 1) { st = KQ_ERR_UNSUPPORTED; goto fail; }
      p->grid_cap2 = ncu * per_cu2;
      p->ws_a_per_token = fv->ws_a_per_token;
      p->ws_b_per_token = fv->ws_b_per_token;
    }
    // The stream kernel runs one wave per token and one workgroup of eight per CU: below
    // about four tokens per CU it leaves most CUs idle, and the pair kernel (two waves
    // per token, 2-wave workgroups) finishes a small batch sooner (measured on MI355X:
    // 64 tokens of 64x128 in 5.4 us vs 9.0 us; break-even near 1024 tokens).
    // Plans with c use the row split (a token's 16-row blocks on their own waves, the
    // stream kernel's arithmetic bit for bit): measured on MI355X under a HIP graph, 64x64
    // with c, 64 / 256 / 512 / 1024 tokens: 4.17 / 4.44 / 5.74 / 7.52 us against 5.39 /
    // 5.61 / 6.37 / 8.23 us for the column split and 6.31 / 6.63 / 6.84 / 7.20 us for the
    // stream split itself. Plans with neither (rows padded to the stream layout) use the
    // column kernel, which also spreads a token over several waves (64x112, 64 tokens:
    // 4.3 us vs 7.4 us).
    if (split == 0 && fv->split == KQ_SPLIT_STREAM) {
      const kq_fused_variant *sv = kq_fused_lookup(n1, n2, c != nullptr, KQ_SPLIT_PAIR, bits);
      if (!sv) sv = kq_fused_lookup(n1, n2, c != nullptr, KQ_SPLIT_RSPLIT, bits);
      if (!sv) sv = kq_fused_lookup(n1, n2, c != nullptr, KQ_SPLIT_COLS, bits);
      int small_per_cu = 0;
      if (sv) {
        std::vector<uint16_t> b2(kq_fused_p2op_elems(n2));
        if (sv->f16_ops != fv->f16_ops) { st = KQ_ERR_UNSUPPORTED; goto fail; }
        kq_fused_arrange_p2(e2.data(), n2, sv->p2_block, b2.data());
        if ((st = upload(&p->small_p2op, b2.data(), b2.size() * 2, s)) != KQ_OK) goto fail;
        if (hipStreamSynchronize(s) != hipSuccess) { st = KQ_ERR_HIP; goto fail; }
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&small_per_cu, sv->kernel_symbol,
                                                         sv->threads, 0) != hipSuccess) {
          st = KQ_ERR_HIP;
          goto fail;
        }
        if (small_per_cu >= 1) {
          p->small_launch = sv->launch;
          p->small_kname = sv->name;
          p->small_grid_cap = ncu * small_per_cu;
          p->small_max_T = (int64_t)4 * ncu;
        }
      }
    }
  } else if (kind == KQ_KIND_FUSED_F32) {
    // each factor as bf16 hi = bf16(p) and lo = bf16(p - hi), both in the fused kernels'
    // operand order, hi then lo in one buffer
    const float *f1 = reinterpret_cast<const float *>(h1.data());
    const float *f2 = reinterpret_cast<const float *>(h2.data());
    std::vector<uint16_t> s1h(h1.size() / 4), s1l(h1.size() / 4), s2h(h2.size() / 4), s2l(h2.size() / 4);
    for (size_t i = 0; i < s1h.size(); ++i) {
      s1h[i] = f32_to_bf16_rne(f1[i]);
      s1l[i] = f32_to_bf16_rne(f1[i] - bf16_to_f32(s1h[i]));
    }
    for (size_t i = 0; i < s2h.size(); ++i) {
      s2h[i] = f32_to_bf16_rne(f2[i]);
      s2l[i] = f32_to_bf16_rne(f2[i] - bf16_to_f32(s2h[i]));
    }
    const size_t e1 = kq_fused_p1op_elems(n1), e2 = kq_fused_p2op_elems(n2);
    std::vector<uint16_t> a1(2 * e1), a2(2 * e2);
    kq_fused_arrange_p1(s1h.data(), n1, a1.data());
    kq_fused_arrange_p1(s1l.data(), n1, a1.data() + e1);
    kq_fused_arrange_p2(s2h.data(), n2, fv->p2_block, a2.data());
    kq_fused_arrange_p2(s2l.data(), n2, fv->p2_block, a2.data() + e2);
    if ((st = upload(&p->p1op, a1.data(), a1.size() * 2, s)) != KQ_OK) goto fail;
    if ((st = upload(&p->p2op, a2.data(), a2.size() * 2, s)) != KQ_OK) goto fail;
    if (hipStreamSynchronize(s) != hipSuccess) { st = KQ_ERR_HIP; goto fail; }
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ksym, fv->threads, 0) != hipSuccess) {
      st = KQ_ERR_HIP;
      goto fail;
    }
  } else {
    std::vector<float> f1((size_t)n1 * n1), f2((size_t)n2 * n2);
    for (size_t i = 0; i < f1.size(); ++i)
      f1[i] = es == 2 ? bf16_to_f32(reinterpret_cast<const uint16_t *>(h1.data())[i])
                      : reinterpret_cast<const float *>(h1.data())[i];
    for (size_t i = 0; i < f2.size(); ++i)
      f2[i] = es == 2 ? bf16_to_f32(reinterpret_cast<const uint16_t *>(h2.data())[i])
                      : reinterpret_cast<const float *>(h2.data())[i];
    if ((st = upload(reinterpret_cast<void **>(&p->p1f), f1.data(), f1.size() * 4, s)) != KQ_OK)
      goto fail;
    if ((st = upload(reinterpret_cast<void **>(&p->p2f), f2.data(), f2.size() * 4, s)) != KQ_OK)
      goto fail;
    if (c && (st = upload(reinterpret_cast<void **>(&p->c), hc.data(), hc.size() * 4, s)) != KQ_OK)
      goto fail;
    if (hipStreamSynchronize(s) != hipSuccess) { st = KQ_ERR_HIP; goto fail; }
    const size_t lds = kq_generic_lds_bytes(n);
    if (lds > 64 * 1024 &&
        hipFuncSetAttribute(ksym, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) !=
            hipSuccess) {
      st = KQ_ERR_HIP;
      goto fail;
    }
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ksym, kq_generic_threads(), lds) !=
        hipSuccess) {
      st = KQ_ERR_HIP;
      goto fail;
    }
  }
  if (per_cu < 1) { st = KQ_ERR_UNSUPPORTED; goto fail; }
  p->grid_cap = ncu * per_cu;
  *out = p;
  return KQ_OK;

fail:
  (void)hipStreamSynchronize(s);  // no copy still in flight into a buffer freed below
  free_plan_buffers(p);
  free(p);
  return st;
}

kq_status kq_create_ex(kq_plan **out, int n1, int n2, kq_dtype x_dtype, kq_dtype scale_dtype,
                       const void *P1, const void *P2, const float *c, float alpha, void *stream,
                       unsigned flags) {
  const kq_status st =
      create_ex_impl(out, n1, n2, x_dtype, scale_dtype, P1, P2, c, alpha, stream, flags);
  if (kq_log_on()) {
    if (st == KQ_OK) {
      const kq_plan *p = *out;
      kq_logf("create %dx%d x=%s steps=%s c=%s alpha=%g flags=0x%x: kernel %s, grid cap %d, "
              "small batches (T < %lld) %s, workspace %zu + %zu B per token",
              n1, n2, dtype_name(x_dtype), dtype_name(scale_dtype), c ? "yes" : "no",
              (double)alpha, flags, p->kname, p->grid_cap, (long long)p->small_max_T,
              p->small_launch ? p->small_kname : "-", p->ws_a_per_token, p->ws_b_per_token);
    } else {
      kq_logf("create %dx%d x=%s steps=%s c=%s flags=0x%x: %s", n1, n2, dtype_name(x_dtype),
              dtype_name(scale_dtype), c ? "yes" : "no", flags, kq_status_string(st));
    }
  }
  return st;
}

kq_status kq_create(kq_plan **out, int n1, int n2, kq_dtype x_dtype, kq_dtype scale_dtype,
                    const void *P1, const void *P2, const float *c, float alpha, void *stream) {
  return kq_create_ex(out, n1, n2, x_dtype, scale_dtype, P1, P2, c, alpha, stream, 0u);
}

kq_status kq_workspace_size(const kq_plan *p, int64_t T, size_t *bytes) {
  if (!p || !bytes || T < 0 || (p->n && T > ((int64_t)1 << 40) / p->n)) return KQ_ERR_INVALID_ARG;
  *bytes = kq_ws_bytes(p, T);
  return KQ_OK;
}

kq_status kq_transform_quant(const kq_plan *p, const void *X, int64_t T, int64_t ldx,
                             uint8_t *codes, void *scales, float *y_debug, void *stream) {
  return kq_transform_quant_ws(p, X, T, ldx, codes, scales, y_debug, nullptr, 0, stream);
}

static kq_status transform_impl(const kq_plan *p, const void *X, int64_t T, int64_t ldx,
                                uint8_t *codes, void *scales, float *y_debug, void *workspace,
                                size_t workspace_bytes, void *stream) {
  if (!p || T < 0) return KQ_ERR_INVALID_ARG;
  if (T == 0) return KQ_OK;
  if (!X || !codes || !scales) return KQ_ERR_INVALID_ARG;
  if (ldx < p->n) return KQ_ERR_INVALID_ARG;
  const size_t es = elem_size(p->x_dtype);
  if (!is_aligned(X, 16) || ((size_t)ldx * es) % 16 != 0) return KQ_ERR_ALIGNMENT;
  if (!is_aligned(codes, 16) || !is_aligned(scales, elem_size(p->scale_dtype)))
    return KQ_ERR_ALIGNMENT;
  if (y_debug && !is_aligned(y_debug, 16)) return KQ_ERR_ALIGNMENT;
  if (T > ((int64_t)1 << 40) / p->n) return KQ_ERR_INVALID_ARG;
  if (p->per_row && T * p->n1 >= ((int64_t)1 << 31)) return KQ_ERR_UNSUPPORTED;
  const size_t need = kq_ws_bytes(p, T);
  if (need) {  // the two-kernel designs pass an intermediate through this workspace
    if (!workspace || workspace_bytes < need) return KQ_ERR_WORKSPACE;
    if (!is_aligned(workspace, 256)) return KQ_ERR_ALIGNMENT;
  } else {
    workspace = nullptr;
  }
  int dev = -1;  // the plan's buffers live on the device that was current at create time
  if (hipGetDevice(&dev) != hipSuccess || dev != p->device) return KQ_ERR_INVALID_ARG;
  hipError_t e;
  if (p->small_launch && T < p->small_max_T) {
    kq_plan v = *p;  // the same plan seen through the small-batch variant's operands
    v.p2op = p->small_p2op;
    v.grid_cap = p->small_grid_cap;
    e = p->small_launch(&v, X, T, ldx, codes, scales, y_debug, nullptr,
                        static_cast<hipStream_t>(stream));
  } else {
    e = p->launch(p, X, T, ldx, codes, scales, y_debug, workspace, static_cast<hipStream_t>(stream));
  }
  return e == hipSuccess ? KQ_OK : KQ_ERR_HIP;
}

kq_status kq_transform_quant_ws(const kq_plan *p, const void *X, int64_t T, int64_t ldx,
                                uint8_t *codes, void *scales, float *y_debug, void *workspace,
                                size_t workspace_bytes, void *stream) {
  const kq_status st = transform_impl(p, X, T, ldx, codes, scales, y_debug, workspace,
                                      workspace_bytes, stream);
  if (kq_log_on())
    kq_logf("transform T=%lld ldx=%lld on %s%s, workspace %zu B: %s", (long long)T,
            (long long)ldx, p ? kq_plan_kernel_name_for(p, T) : "(no plan)",
            y_debug ? " with y_debug" : "", workspace ? workspace_bytes : (size_t)0,
            kq_status_string(st));
  return st;
}

kq_status kq_transform_quant_noalloc(const kq_plan *p, const void *X, int64_t T, int64_t ldx,
                                     uint8_t *codes, void *scales, float *y_debug, void *stream) {
  if (!p || T < 0 || (p->n && T > ((int64_t)1 << 40) / p->n)) return KQ_ERR_INVALID_ARG;
  if (T == 0) return KQ_OK;
  const size_t need = kq_ws_bytes(p, T);
  if (need > kScratchBytes) return KQ_ERR_WORKSPACE;
  void *ws = nullptr;
  if (need) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return KQ_ERR_HIP;
    if (dev != p->device) return KQ_ERR_INVALID_ARG;
    const kq_status st = scratch_address(dev, &ws);
    if (st != KQ_OK) return st;
  }
  return kq_transform_quant_ws(p, X, T, ldx, codes, scales, y_debug, ws, need ? kScratchBytes : 0,
                               stream);
}

const char *kq_plan_kernel_name_for(const kq_plan *p, int64_t T) {
  if (!p) return "";
  return (p->small_launch && T < p->small_max_T) ? p->small_kname : p->kname;
}

kq_status kq_destroy(kq_plan *p) {
  if (!p) return KQ_OK;
  free_plan_buffers(p);
  free(p);
  return KQ_OK;
}

float kq_plan_clip_ratio(const kq_plan *p) { return p ? p->clip : 0.0f; }

const char *kq_plan_kernel_name(const kq_plan *p) { return p ? p->kname : ""; }

}  // extern "C"
