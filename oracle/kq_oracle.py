"""CPU oracle for the Kronecker-factored activation transform + per-token INT4 quantizer.

TEST INFRASTRUCTURE ONLY. This module is the slow, plainly written definition that the
GPU path is checked against. Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. It never imports the product package
(``kronecker_factored_transforms_amd``) and the product never imports it; the two share
no code. Inputs come from the caller as plain NumPy arrays.

Sources (web pages, cited by title and section):
  [KP]  "Kronecker Product" -- Definition; Why It Matters for LLM Quantization;
        Implementation Notes.
  [FQ]  "FlatQuant: Fast Learnable Affine Quantization" -- Symbol Map; Deep Dive:
        Kronecker factorization; Per-channel scaling and learnable clipping;
        The fused kernel (Figure 8); Putting It Together.
  [QuIP] "Quantifying Incoherence in the QuIP Method" (orthogonal factors, inverse).
  [HR]  "High-Rate Quantized Matrix Multiplication I" -- Technical Summary: INT
        multipliers with absmax scaling; high-rate uniform-noise model.

What is computed (per token t, x_t of length n = n1*n2):
  1. x^_t = x_t * c (elementwise, optional per-channel vector)        [FQ Symbol Map: diag(c)]
  2. V_t = x^_t viewed as an n1 x n2 matrix, row-major: V_t[i,k] = x^_t[i*n2 + k]
                                                                       [FQ Symbol Map: X~ is k x n1 x n2]
  3. Y_t = P1^T V_t P2, which equals x^_t (P1 (x) P2)                  [KP Why It Matters; FQ Kronecker factorization]
  4. per-token absmax a_t, clip ratio sigmoid(alpha), step s_t, RTN to symmetric INT4,
     clamp to [-8, 7], two codes per byte.                             [FQ TL;DR (RTN), Symbol Map (Q, alpha_a),
                                                                        Per-channel scaling and learnable clipping;
                                                                        HR absmax INT]

Readings where the pages leave a step open (each is a convention of this library, stated
once here and relied on by every function below):
  R1  The left factor enters transposed (P1^T). [FQ] writes P1^T in the factorization
      equation and in "Putting It Together"; the fused-kernel paragraph drops the
      transpose, which only agrees for symmetric P1.
  R2  vec() is the row-major flatten with the n1 axis outer, so that x (P1 (x) P2) =
      vec_r(P1^T V P2) holds with the index formula of [KP Definition].
  R3  c multiplies x before the transform (x^ = x * c). NULL/None means all ones.
  R4  One scale per token (the workloads state per-token quantization).
  R5  Symmetric INT4: divisor 7 = 2^(4-1) - 1, codes clamped to [-8, 7].
  R6  Round to nearest, ties to even (numpy.rint).
  R7  The clip ratio sigmoid(alpha) multiplies the absmax; values beyond clip*absmax
      saturate through the clamp. sigmoid is evaluated once, in double, then rounded to
      fp32.
  R8  Scale: s32 = fp32(fp32(clip * a) / 7), stored as fp16 (RNE) by default (or kept
      fp32); codes are computed with the *stored* scale: inv = fp32(1 / s),
      q = clamp(rint(fp32(y * inv)), -8, 7). Every step is one IEEE-rounded fp32 op.
  R9  A token whose stored scale is 0 (all-zero token, clip 0, or underflow) gets all
      codes 0. A stored fp32 step so small that fp32(1 / s) overflows (s <= 2^-128) is an
      underflow too: it is stored as 0 and its codes are 0 (an fp16 step never reaches
      that range: its smallest nonzero value is 2^-24). Non-finite inputs are outside the
      contract.
  R10 Element 2m goes in the low nibble of byte m, element 2m+1 in the high nibble,
      each as a 4-bit two's-complement value, in row-major Y order (index j*n2 + l).

Beyond the INT4 path the module also defines, with the same conventions:
  - INT8 codes (quantize_per_token(..., bits=8), pack_int8): divisor 127, clamp to
    [-128, 127], one two's-complement byte per value [FQ How we know: beyond dense W4A4,
    mixed precision at W8A8];
  - the weight side and the consumer (weight_factors, int4_gemm): the rows of W take the
    factors P1^-T and P2^-T so that (X P)(P^-1 W^T) = X W^T, and the INT4 x INT4 product
    is the integer dot product times both scales [FQ Learning the affine transformation;
    HR Technical Summary].

Every function below is pinned by tests that do not re-type its formula (brute-force
definition loops, library Kronecker products, closed forms for identity/permutation
factors, orthogonal norm and inverse invariants, exact power-of-two cases against
an independent library quantizer, and the quantization error bound).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "kron_by_definition",
    "kron_library",
    "transform_dense",
    "transform",
    "inverse_transform",
    "clip_ratio",
    "quantize_per_token",
    "weight_factors",
    "int4_gemm",
    "pack_int8",
    "pack_int4",
    "unpack_int4",
    "dequantize",
    "transform_quant",
]


# ----------------------------------------------------------------------------------------
# Input decoding
# ----------------------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 numbers given as their 16-bit patterns (uint16).

    A bfloat16 is the upper half of an IEEE binary32, so the pattern shifted left by 16
    bits is the binary32 with the same value; widening that to float64 is exact.
    """
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    f32 = (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f32.astype(np.float64)


def _as_f64(a, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    if dtype == "fp32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "fp64":
        return np.asarray(a, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------------------
# Kronecker product
# ----------------------------------------------------------------------------------------
def kron_by_definition(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """A (x) B from the entry formula of [KP Definition], written as explicit loops.

    For A (m x n) and B (p x q) the product is mp x nq and, with 0-based indices, the
    entry in row i*p + k, column j*q + l is a[i, j] * b[k, l]. Pure Python loops: meant
    for the tiny shapes the tests use.
    """
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    m, n = A.shape
    p, q = B.shape
    K = np.zeros((m * p, n * q), dtype=np.float64)
    for i in range(m):
        for j in range(n):
            for k in range(p):
                for l in range(q):
                    K[i * p + k, j * q + l] = A[i, j] * B[k, l]
    return K


def kron_library(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """A (x) B via numpy.kron, the library routine named in [KP Implementation Notes]."""
    return np.kron(np.asarray(A, dtype=np.float64), np.asarray(B, dtype=np.float64))


# ----------------------------------------------------------------------------------------
# The transform
# ----------------------------------------------------------------------------------------
def _scaled_tokens(X, dtype, c):
    x = _as_f64(X, dtype)
    if x.ndim != 2:
        raise ValueError("X must be [T, n]")
    if c is not None:
        cc = np.asarray(c, dtype=np.float32).astype(np.float64)
        if cc.shape != (x.shape[1],):
            raise ValueError("c must have length n")
        # [FQ Per-channel scaling and learnable clipping]: diag(c) acts on the input
        # before the transform (reading R3). bf16*fp32 products are exact in float64.
        x = x * cc[None, :]
    return x


def transform_dense(X, P1, P2, c=None, dtype="fp64") -> np.ndarray:
    """Y = x^ (P1 (x) P2) with the n x n Kronecker matrix materialised (tiny n only).

    This is the left-hand side of the identity in [KP Why It Matters] / [FQ Kronecker
    factorization]: the whole transform P = P1 (x) P2 applied to each token as a row
    vector. The per-channel scale enters as the diagonal matrix diag(c) multiplying the
    row vector before P (reading R3). Returns float64 [T, n].
    """
    x = _as_f64(X, dtype)
    p1 = _as_f64(P1, dtype)
    p2 = _as_f64(P2, dtype)
    n = p1.shape[0] * p2.shape[0]
    if x.shape[1] != n:
        raise ValueError("n must equal n1*n2")
    if n > 4096:
        raise ValueError("transform_dense materialises an n x n matrix; use n <= 4096")
    if c is not None:
        D = np.diag(np.asarray(c, dtype=np.float32).astype(np.float64))
        x = x @ D
    return x @ kron_library(p1, p2)


def transform(X, P1, P2, c=None, dtype="fp64") -> np.ndarray:
    """Y_t = P1^T V_t P2 for every token, in float64 (the factored form).

    [FQ Kronecker factorization]: the transform is applied as two small contractions on
    the 3-D view X~ (T x n1 x n2): the mode-1 product with P1^T and the mode-2 product
    with P2 (reading R1 for the transpose, R2 for the row-major view). Inputs are the
    exact stored values (bf16 bit patterns, fp32 or fp64); everything after decoding is
    float64. The two contractions use numpy.matmul as the library primitive.
    Returns float64 [T, n] in row-major Y order (index j*n2 + l).
    """
    x = _scaled_tokens(X, dtype, c)
    p1 = _as_f64(P1, dtype)
    p2 = _as_f64(P2, dtype)
    n1, n2 = p1.shape[0], p2.shape[0]
    if p1.shape != (n1, n1) or p2.shape != (n2, n2):
        raise ValueError("P1 must be n1 x n1 and P2 n2 x n2")
    T, n = x.shape
    if n != n1 * n2:
        raise ValueError("n must equal n1*n2")
    V = x.reshape(T, n1, n2)                      # V[t, i, k] = x^[t, i*n2 + k]
    Y = np.matmul(np.matmul(p1.T, V), p2)         # P1^T V_t P2
    return Y.reshape(T, n)


def inverse_transform(Y, P1, P2, c=None) -> np.ndarray:
    """Undo the transform: x = vec_r(P1^{-T} Y_t P2^{-1}) / c, in float64.

    [FQ Kronecker factorization] writes the weight side with P1^{-1} and P2^{-1}: the
    inverse of P1 (x) P2 is P1^{-1} (x) P2^{-1}. For orthogonal factors the inverse is
    the transpose [QuIP]. Uses numpy.linalg.solve as the library primitive.
    """
    y = np.asarray(Y, dtype=np.float64)
    p1 = np.asarray(P1, dtype=np.float64)
    p2 = np.asarray(P2, dtype=np.float64)
    n1, n2 = p1.shape[0], p2.shape[0]
    T = y.shape[0]
    Yt = y.reshape(T, n1, n2)
    # A = P1^{-T} Y  <=>  P1^T A = Y ;  V = A P2^{-1}  <=>  P2^T V^T = A^T
    A = np.linalg.solve(p1.T[None, :, :], Yt)
    Vt = np.linalg.solve(p2.T[None, :, :], np.swapaxes(A, 1, 2))
    x = np.swapaxes(Vt, 1, 2).reshape(T, n1 * n2)
    if c is not None:
        x = x / np.asarray(c, dtype=np.float32).astype(np.float64)[None, :]
    return x


# ----------------------------------------------------------------------------------------
# The quantizer
# ----------------------------------------------------------------------------------------
def clip_ratio(alpha: float) -> np.float32:
    """sigmoid(alpha) evaluated in double with the host libm exp, rounded to fp32.

    [FQ Symbol Map / Per-channel scaling and learnable clipping]: the activation clip
    threshold is a learnable scalar per tensor mapped into (0, 1) by a sigmoid
    (reading R7). +inf gives exactly 1, -inf gives 0.
    """
    a = float(alpha)
    if math.isnan(a):
        raise ValueError("alpha is NaN")
    if a == math.inf:
        return np.float32(1.0)
    if a == -math.inf:
        return np.float32(0.0)
    if a >= 0:
        v = 1.0 / (1.0 + math.exp(-a))
    else:
        e = math.exp(a)
        v = e / (1.0 + e)
    return np.float32(v)


def quantize_per_token(Y32, clip, scale_dtype: str = "fp16", bits: int = 4):
    """Per-token symmetric b-bit round-to-nearest of an fp32 [T, n] tensor (b = 4 or 8).

    [FQ TL;DR]: plain round-to-nearest (RTN) quantization; [FQ Symbol Map]: Q(.) maps
    values to b-bit integer points with step s; [HR absmax INT]: the step comes from the
    l-infinity norm (absmax) of the vector. With M = 2^(b-1) - 1 (7 for INT4, 127 for
    INT8), steps (readings R4-R9), each one rounded fp32 (or fp16) operation:
        a   = max_k |y_k|                          (exact)
        s32 = fp32( fp32(clip * a) / M )
        s   = fp16_rne(s32)   (or s32 when scale_dtype == "fp32")
        s == 0, or fp32(1 / s) not finite (then s is stored as 0) -> all codes 0
        inv = fp32(1 / s);  q = clamp(rint(fp32(y * inv)), -M - 1, M)
    Returns (q int8 [T, n], scales float16|float32 [T]).
    """
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    M = np.float32(2 ** (bits - 1) - 1)
    y = np.asarray(Y32)
    if y.dtype != np.float32:
        raise TypeError("the quantizer takes the fp32 transformed tensor")
    if y.ndim != 2:
        raise ValueError("Y must be [T, n]")
    clip32 = np.float32(clip)
    T = y.shape[0]
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        a = np.abs(y).max(axis=1) if y.shape[1] else np.zeros(T, np.float32)
        a = a.astype(np.float32)
        s32 = (clip32 * a).astype(np.float32) / M
        s32 = s32.astype(np.float32)
        if scale_dtype == "fp16":
            s_store = s32.astype(np.float16)
        elif scale_dtype == "fp32":
            s_store = s32
        else:
            raise ValueError("scale_dtype must be 'fp16' or 'fp32'")
        s_f = s_store.astype(np.float32)
        zero = s_f == np.float32(0.0)
        inv = (np.float32(1.0) / np.where(zero, np.float32(1.0), s_f)).astype(np.float32)
        # reading R9: a step whose reciprocal overflows fp32 counts as underflowed
        tiny = ~np.isfinite(inv)
        if tiny.any():
            s_store = np.where(tiny, np.zeros_like(s_store), s_store)
            zero = zero | tiny
            inv = np.where(tiny, np.float32(0.0), inv).astype(np.float32)
        v = (y * inv[:, None]).astype(np.float32)
        q = np.rint(v)
        q = np.clip(q, -M - 1, M)
        q = np.where(zero[:, None], 0.0, q)
    return q.astype(np.int8), s_store


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Two signed 4-bit codes per byte: element 2m low nibble, 2m+1 high (reading R10).

    [FQ The fused kernel]: only the packed low-bit tile is written out.
    """
    q = np.asarray(q)
    if q.shape[-1] % 2:
        raise ValueError("need an even number of codes per row")
    if q.size and (q.min() < -8 or q.max() > 7):
        raise ValueError("codes outside [-8, 7]")
    u = (q.astype(np.int16) & 0xF).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


def pack_int8(q: np.ndarray) -> np.ndarray:
    """INT8 codes stored as bytes (two's complement), one per element, row-major order."""
    return np.ascontiguousarray(np.asarray(q, dtype=np.int8)).view(np.uint8)


def unpack_int4(codes: np.ndarray) -> np.ndarray:
    """Inverse of pack_int4: bytes -> signed codes in [-8, 7] (int8)."""
    b = np.asarray(codes, dtype=np.uint8)
    lo = (b & 0xF).astype(np.int8)
    hi = (b >> 4).astype(np.int8)
    lo = np.where(lo >= 8, lo - 16, lo).astype(np.int8)
    hi = np.where(hi >= 8, hi - 16, hi).astype(np.int8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """q * s per token in float64 (what an INT4 consumer reconstructs)."""
    q = unpack_int4(codes).astype(np.float64)
    return q * np.asarray(scales).astype(np.float64)[:, None]


# ----------------------------------------------------------------------------------------
# Whole path
# ----------------------------------------------------------------------------------------
def transform_quant(X, P1, P2, c, alpha, dtype, scale_dtype="fp16"):
    """The full hot path on the CPU: float64 transform, then the fp32 quantizer.

    [FQ Putting It Together, step 3]: reshape, apply P1^T . P2, quantize, keep only
    the packed INT4 tile. The transformed tensor is rounded once from float64 to fp32
    before quantization. Returns (Y64 [T, n], codes uint8 [T, n/2], scales [T]).
    """
    Y = transform(X, P1, P2, c, dtype)
    q, s = quantize_per_token(Y.astype(np.float32), clip_ratio(alpha), scale_dtype)
    return Y, pack_int4(q), s


# ----------------------------------------------------------------------------------------
# Weight side and the INT4 consumer
def weight_factors(P1, P2):
    """Factors that transform the rows of a weight matrix W [N x n] so that the INT4 product
    of the two transformed sides reproduces X W^T.

    [FQ Learning the affine transformation]: the layer computes (X P)(P^-1 W^T); with
    [FQ Kronecker factorization] P = P1 (x) P2 and P^-1 = P1^-1 (x) P2^-1. Row j of
    (P^-1 W^T)^T = W P^-T is w_j (P1^-T (x) P2^-T) ([KP] Definition: (A (x) B)^T =
    A^T (x) B^T), i.e. the same transform as a token with factors P1^-T and P2^-T.
    float64 inputs and outputs.
    """
    P1 = np.asarray(P1, dtype=np.float64)
    P2 = np.asarray(P2, dtype=np.float64)
    return np.linalg.inv(P1).T, np.linalg.inv(P2).T


def _f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def int4_gemm(codes_x, scales_x, codes_w, scales_w, out_dtype: str = "fp32"):
    """The INT4 x INT4 product of two quantized operands with their per-row steps.

    acc[t, j] = sum_k qx[t, k] qw[j, k] exactly (integers), then in fp32, one rounding per
    step: out = fp32(fp32(acc) * sx[t]) * sw[j]; stored as fp32, or rounded to nearest
    even into bf16 (bit patterns, uint16) or fp16. [FQ Putting It Together]: the codes and
    steps of both sides feed an INT4 GEMM; [HR Technical Summary]: the product of two
    absmax-quantized matrices is the integer product times the two scale vectors.
    """
    qx = unpack_int4(codes_x).astype(np.int64)
    qw = unpack_int4(codes_w).astype(np.int64)
    acc = qx @ qw.T
    sx = np.asarray(scales_x).astype(np.float32)
    sw = np.asarray(scales_w).astype(np.float32)
    out = (acc.astype(np.float32) * sx[:, None]).astype(np.float32)
    out = (out * sw[None, :]).astype(np.float32)
    if out_dtype == "fp32":
        return out
    if out_dtype == "bf16":
        return _f32_to_bf16_bits(out)
    if out_dtype == "fp16":
        return out.astype(np.float16)
    raise ValueError(out_dtype)
