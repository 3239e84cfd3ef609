"""Feasibility of the bf16 tolerance, on the CPU.

The bf16 path multiplies bf16 operands with fp32 accumulation in both stages, rounds the
stage-1 result Z to bf16 to feed stage 2, and with a per-channel scale splits
x_hat = fp32(x c) into bf16 hi + lo words. This file emulates exactly those roundings in
numpy (the accumulation order inside an MFMA aside) and compares the result with the
fp64 oracle on every bf16 workload:

- the emulated pipeline stays inside the 2e-3 relative-L2 gate with margin, so the gate
  is one the design can meet and not one a kernel passes by luck;
- rounding x_hat once to bf16 instead of splitting it would not meet the gate on the
  workloads with a per-channel scale, which is why the path splits it.
"""
import numpy as np
import pytest

from kronecker_factored_transforms_amd import synth as S
from oracle import kq_oracle as O

GATE = 2e-3
BF16_WORKLOADS = ["attn_n4096", "hidden_n8192", "down_proj_n14336", "decode_n8192_t64",
                  "down_proj_n28672", "ffn_n11008", "hidden_n7168", "ffn_n18432"]


def _bf16(a64):
    return O.bf16_bits_to_f64(S.to_bf16_bits(a64))


def _emulate(inp, split_c=True):
    wl = inp.wl
    X = O.bf16_bits_to_f64(inp.X)
    if inp.c is not None:
        xh = (X.astype(np.float32) * inp.c.astype(np.float32)).astype(np.float32)
        hi = _bf16(xh.astype(np.float64))
        A = hi
        if split_c:
            A = hi + _bf16((xh - hi.astype(np.float32)).astype(np.float64))
    else:
        A = X
    T = A.shape[0]
    P1 = O.bf16_bits_to_f64(inp.P1)
    P2 = O.bf16_bits_to_f64(inp.P2)
    Z = (A.reshape(T, wl.n1, wl.n2) @ P2).astype(np.float32).astype(np.float64)
    Y = np.einsum("ji,tjk->tik", P1, _bf16(Z))  # P1^T Z
    return Y.astype(np.float32).astype(np.float64).reshape(T, -1)


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("name", BF16_WORKLOADS)
def test_bf16_pipeline_meets_the_gate_with_margin(name):
    inp = S.make(name, T=64)
    Y = O.transform(inp.X, inp.P1, inp.P2, inp.c, inp.wl.dtype)
    rel = _rel(_emulate(inp), Y)
    # two bf16 roundings of unit-variance data: about 2 * 2^-9 / sqrt(3) in quadrature
    assert 1.2e-3 < rel < 0.9 * GATE, f"{name}: {rel:.3e}"


@pytest.mark.parametrize("name", ["attn_n4096", "down_proj_n14336"])
def test_per_channel_scale_needs_the_hi_lo_split(name):
    inp = S.make(name, T=64)
    assert inp.c is not None
    Y = O.transform(inp.X, inp.P1, inp.P2, inp.c, inp.wl.dtype)
    split = _rel(_emulate(inp, split_c=True), Y)
    single = _rel(_emulate(inp, split_c=False), Y)
    assert split < 0.9 * GATE < GATE < single, (split, single)
