"""Seeded synthetic inputs for the Kronecker transform + INT4 quantizer.

This module only draws random numbers and stores them in the input dtypes; it holds none
of the method's arithmetic, so both the GPU path and the CPU oracle may consume what it
produces. Everything is NumPy (PCG64) on the host.

The workloads stand in for the activations the FlatQuant page talks about ("FlatQuant:
Fast Learnable Affine Quantization" -- Why This Exists: outlier channels and pivot tokens;
Kronecker factorization: hidden sizes 4096 / 8192 with factors such as (64, 128)). No real
model activations or weights are used.

Determinism: every tensor has its own SeedSequence child, keyed by (workload stream id,
tensor id[, chunk]). Activations are drawn in chunks of ``CHUNK`` tokens, each chunk from
its own child stream, so any token range can be regenerated on its own and the values do
not depend on how many tokens a caller asks for.
"""
from __future__ import annotations

import hashlib
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

CHUNK = 256  # tokens per activation chunk (one RNG child stream each)

# tensor ids inside a workload's seed space
_TID_X, _TID_PICKS, _TID_P1, _TID_P2, _TID_C, _TID_ALPHA = range(6)


@dataclass(frozen=True)
class Workload:
    name: str
    stream: int            # seed-space id of the workload
    T: int
    n1: int
    n2: int
    dtype: str             # "bf16" (uint16 bit patterns) or "fp32"
    x_kind: str            # "normal" | "student_t3" | "silu_gate"
    n_outliers: int = 0    # seeded outlier channels (scaled by outlier_scale)
    outlier_scale: float = 1.0
    fixed_outliers: tuple = ()      # explicit outlier channels (0-based)
    pivot_channels: int = 0          # token 0 gets this many seeded channels x pivot_scale
    pivot_scale: float = 1.0
    p_kind: str = "orthogonal"       # "orthogonal" | "near_identity"
    p_eps: float = 0.0               # near_identity: I + eps * N(0,1) / sqrt(n_i)
    c_kind: str | None = None        # None | "uniform" | "loguniform"
    c_lo: float = 1.0
    c_hi: float = 1.0
    alpha: float | None = None       # fixed clip logit; None -> drawn from N(alpha_mu, alpha_sd)
    alpha_mu: float = 2.0
    alpha_sd: float = 0.5
    scale_dtype: str = "fp16"
    per_row: bool = False            # identity left factor, one step per row of V

    @property
    def n(self) -> int:
        return self.n1 * self.n2


WORKLOADS = {
    # tiny case the oracle finishes instantly: fp32, 8x8 factors, two outlier channels
    "tiny_fp32_n64": Workload(
        "tiny_fp32_n64", 1, T=16, n1=8, n2=8, dtype="fp32", x_kind="normal",
        fixed_outliers=(3, 40), outlier_scale=20.0, p_kind="orthogonal",
        alpha=math.inf),
    # LLaMA-7B-shaped attention input: hidden 4096 as 64x64, pivot token, per-channel c
    "attn_n4096": Workload(
        "attn_n4096", 2, T=2048, n1=64, n2=64, dtype="bf16", x_kind="normal",
        n_outliers=4, outlier_scale=50.0, pivot_channels=2, pivot_scale=200.0,
        p_kind="near_identity", p_eps=0.1, c_kind="uniform", c_lo=0.5, c_hi=2.0,
        alpha=None),
    # hidden 8192 with the (64, 128) factors, heavy-tailed activations
    "hidden_n8192": Workload(
        "hidden_n8192", 3, T=16384, n1=64, n2=128, dtype="bf16", x_kind="student_t3",
        n_outliers=8, outlier_scale=30.0, p_kind="orthogonal", alpha=3.0),
    # MLP down-projection input: 14336 = 112 x 128, SiLU-gated activations, per-channel c
    "down_proj_n14336": Workload(
        "down_proj_n14336", 4, T=8192, n1=112, n2=128, dtype="bf16", x_kind="silu_gate",
        p_kind="near_identity", p_eps=0.05, c_kind="loguniform", c_lo=0.25, c_hi=4.0,
        alpha=None),
    # decode-shaped and long-prefill runs over the same hidden-8192 activation stream
    "decode_n8192_t64": Workload(
        "decode_n8192_t64", 5, T=64, n1=64, n2=128, dtype="bf16", x_kind="student_t3",
        n_outliers=8, outlier_scale=30.0, p_kind="orthogonal", alpha=3.0),
    "prefill_n8192_t65536": Workload(
        "prefill_n8192_t65536", 5, T=65536, n1=64, n2=128, dtype="bf16",
        x_kind="student_t3", n_outliers=8, outlier_scale=30.0, p_kind="orthogonal",
        alpha=3.0),
    # keys of a grouped-query attention layer ahead of the KV cache: 8 heads of 128 per
    # token (V = 8 x 128, identity left factor, one step per head), 64k-token prefill; a few
    # outlier channels inside the head dimension
    "kv_h8_d128": Workload(
        "kv_h8_d128", 7, T=65536, n1=8, n2=128, dtype="bf16", x_kind="normal",
        n_outliers=4, outlier_scale=20.0, p_kind="orthogonal", alpha=3.0, per_row=True),
    # MLP down-projection input of a 7B-class model: 11008 = 86 x 128 (n1 not a multiple
    # of 16), SiLU-gated activations, per-channel c
    "ffn_n11008": Workload(
        "ffn_n11008", 8, T=8192, n1=86, n2=128, dtype="bf16", x_kind="silu_gate",
        p_kind="near_identity", p_eps=0.05, c_kind="loguniform", c_lo=0.25, c_hi=4.0,
        alpha=None),
    # DeepSeek-V3-class hidden size 7168 with the factors that minimise n1 + n2 (64 x 112:
    # n2 is an odd multiple of 16), heavy-tailed activations
    "hidden_n7168": Workload(
        "hidden_n7168", 9, T=16384, n1=64, n2=112, dtype="bf16", x_kind="student_t3",
        n_outliers=8, outlier_scale=30.0, p_kind="orthogonal", alpha=3.0),
    # DeepSeek-V3-class dense FFN down-projection input, 18432 = 128 x 144
    "ffn_n18432": Workload(
        "ffn_n18432", 10, T=4096, n1=128, n2=144, dtype="bf16", x_kind="silu_gate",
        p_kind="orthogonal", alpha=3.0),
    # a larger factor than 128: the 70B-class FFN down-projection input, 28672 = 128 x 224
    "down_proj_n28672": Workload(
        "down_proj_n28672", 6, T=4096, n1=128, n2=224, dtype="bf16", x_kind="silu_gate",
        p_kind="orthogonal", alpha=3.0),
    # the same input with a per-channel scale: n2 > 128 with c has only the two-kernel
    # designs for factors beyond the on-chip memory
    "down_proj_n28672_c": Workload(
        "down_proj_n28672_c", 11, T=4096, n1=128, n2=224, dtype="bf16", x_kind="silu_gate",
        p_kind="near_identity", p_eps=0.05, c_kind="loguniform", c_lo=0.25, c_hi=4.0,
        alpha=None),
    # both factors above 128: a 72B-class FFN down-projection input, 29568 = 168 x 176
    "down_proj_n29568": Workload(
        "down_proj_n29568", 12, T=4096, n1=168, n2=176, dtype="bf16", x_kind="silu_gate",
        p_kind="orthogonal", alpha=3.0),
    # fp32 activations of hidden size 4096 (64 x 64): the fp32 path on the matrix cores
    "fp32_n4096": Workload(
        "fp32_n4096", 14, T=2048, n1=64, n2=64, dtype="fp32", x_kind="normal",
        n_outliers=4, outlier_scale=20.0, p_kind="orthogonal", alpha=3.0),
    # the largest factors built: 65536 = 256 x 256 (heavy-tailed activations)
    "hidden_n65536": Workload(
        "hidden_n65536", 13, T=2048, n1=256, n2=256, dtype="bf16", x_kind="student_t3",
        n_outliers=8, outlier_scale=30.0, p_kind="orthogonal", alpha=3.0),
}


@dataclass
class Inputs:
    wl: Workload
    X: np.ndarray          # [T, n] uint16 (bf16 bits) or float32
    P1: np.ndarray         # [n1, n1] same storage dtype as X
    P2: np.ndarray         # [n2, n2]
    c: np.ndarray | None   # [n] float32 or None
    alpha: float           # clip logit (an fp32-representable value, or +-inf)
    token_ids: np.ndarray  # which tokens of the stream X holds

    @property
    def T(self):
        return self.X.shape[0]


# ----------------------------------------------------------------------------------------
def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=seed, spawn_key=key)))


def to_bf16_bits(a) -> np.ndarray:
    """Round to bfloat16 (round-to-nearest-even via binary32) and return uint16 patterns."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(a, dtype):
    if dtype == "bf16":
        return to_bf16_bits(a)
    if dtype == "fp32":
        return np.asarray(a, dtype=np.float64).astype(np.float32)
    raise ValueError(dtype)


def _picks(wl: Workload, seed: int):
    rng = _rng(seed, wl.stream, _TID_PICKS)
    n = wl.n
    out = list(wl.fixed_outliers)
    if wl.n_outliers:
        out = sorted(int(v) for v in rng.choice(n, size=wl.n_outliers, replace=False))
    piv = []
    if wl.pivot_channels:
        piv = sorted(int(v) for v in rng.choice(n, size=wl.pivot_channels, replace=False))
    return out, piv


def outlier_channels(wl: Workload, seed: int = 0):
    """(outlier channels, pivot channels) of a workload, 0-based."""
    return _picks(wl, seed)


def _draw_chunk(wl: Workload, seed: int, ci: int, outl, piv) -> np.ndarray:
    rng = _rng(seed, wl.stream, _TID_X, ci)
    shape = (CHUNK, wl.n)
    if wl.x_kind == "normal":
        x = rng.standard_normal(shape)
    elif wl.x_kind == "student_t3":
        x = rng.standard_t(3.0, size=shape)
    elif wl.x_kind == "silu_gate":
        g = rng.standard_normal(shape)
        u = rng.standard_normal(shape)
        x = g / (1.0 + np.exp(-g)) * u
    else:
        raise ValueError(wl.x_kind)
    if outl:
        x[:, outl] *= wl.outlier_scale
    if piv and ci == 0:
        x[0, piv] *= wl.pivot_scale
    return _store(x, wl.dtype)


def make_tokens(wl: Workload, token_ids, seed: int = 0, threads: int | None = None) -> np.ndarray:
    """Rows `token_ids` of the workload's activation stream (only their chunks are drawn)."""
    tid = np.asarray(token_ids, dtype=np.int64)
    outl, piv = _picks(wl, seed)
    chunks = np.unique(tid // CHUNK)
    threads = threads or min(8, os.cpu_count() or 1)
    dt = np.uint16 if wl.dtype == "bf16" else np.float32
    out = np.empty((tid.size, wl.n), dtype=dt)

    def work(ci):
        blk = _draw_chunk(wl, seed, int(ci), outl, piv)
        sel = np.nonzero(tid // CHUNK == ci)[0]
        out[sel] = blk[tid[sel] - ci * CHUNK]

    if len(chunks) == 1 or threads == 1:
        for ci in chunks:
            work(ci)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, chunks))
    return out


def _factor(wl: Workload, seed: int, which: int, n_i: int) -> np.ndarray:
    rng = _rng(seed, wl.stream, which)
    G = rng.standard_normal((n_i, n_i))
    if wl.p_kind == "orthogonal":
        # Haar-distributed orthogonal matrix: QR of a Gaussian with the column signs fixed
        # by sign(diag(R)) (Mezzadri, "How to generate random matrices from the classical
        # compact groups", 2007).
        Q, R = np.linalg.qr(G)
        d = np.sign(np.diag(R))
        d[d == 0] = 1.0
        P = Q * d[None, :]
    elif wl.p_kind == "near_identity":
        P = np.eye(n_i) + wl.p_eps * G / math.sqrt(n_i)
    else:
        raise ValueError(wl.p_kind)
    return _store(P, wl.dtype)


def make(name_or_wl, seed: int = 0, T: int | None = None, token_ids=None) -> Inputs:
    """All inputs of a workload. `T` overrides the token count (first T tokens of the
    stream); `token_ids` selects arbitrary tokens of the stream instead."""
    wl = WORKLOADS[name_or_wl] if isinstance(name_or_wl, str) else name_or_wl
    if token_ids is None:
        T = wl.T if T is None else int(T)
        token_ids = np.arange(T, dtype=np.int64)
    else:
        token_ids = np.asarray(token_ids, dtype=np.int64)
    X = make_tokens(wl, token_ids, seed) if token_ids.size else np.empty(
        (0, wl.n), dtype=np.uint16 if wl.dtype == "bf16" else np.float32)
    P1 = _factor(wl, seed, _TID_P1, wl.n1)
    P2 = _factor(wl, seed, _TID_P2, wl.n2)
    c = None
    if wl.c_kind is not None:
        rng = _rng(seed, wl.stream, _TID_C)
        if wl.c_kind == "uniform":
            c = rng.uniform(wl.c_lo, wl.c_hi, size=wl.n)
        elif wl.c_kind == "loguniform":
            c = np.exp(rng.uniform(math.log(wl.c_lo), math.log(wl.c_hi), size=wl.n))
        else:
            raise ValueError(wl.c_kind)
        c = c.astype(np.float32)
    if wl.alpha is None:
        alpha = float(np.float32(_rng(seed, wl.stream, _TID_ALPHA).normal(wl.alpha_mu, wl.alpha_sd)))
    else:
        alpha = float(np.float32(wl.alpha)) if math.isfinite(wl.alpha) else float(wl.alpha)
    return Inputs(wl, X, P1, P2, c, alpha, token_ids)


def with_tokens(wl: Workload, T: int) -> Workload:
    return replace(wl, T=int(T))


def signed_permutation(n: int, rng: np.random.Generator) -> np.ndarray:
    """A random signed permutation matrix (entries 0 / +-1), as float64."""
    perm = rng.permutation(n)
    sign = rng.choice([-1.0, 1.0], size=n)
    P = np.zeros((n, n))
    P[np.arange(n), perm] = sign
    return P


def sha256(a) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
