"""GPU parity of the row-split kernel with a per-channel scale (n2 = 64): a token's 16-row
blocks on their own waves, each with its own power-of-two scale for x^ (from its rows'
bound), Z passed between the waves through LDS on one reference scale. Every case checks
Y against the fp64 oracle (2e-3 rel-L2), codes and steps bit-exact against the oracle
quantizer on the GPU's own Y, and the launch without the debug output writing the same
codes."""
import math
from dataclasses import replace

import numpy as np
import pytest

import kqtest as K
from kronecker_factored_transforms_amd import binding as B
from kronecker_factored_transforms_amd import synth as S
from oracle import kq_oracle as O

pytestmark = pytest.mark.gpu

FLAG = B.KQ_FLAG_SPLIT_RSPLIT


def _workload(n1, **kw):
    return replace(S.WORKLOADS["attn_n4096"], n1=n1, n2=64, n_outliers=4, pivot_channels=0, **kw)


def _run(inp, plan, X):
    import torch
    codes, scales, y = K.run(plan, X, y_debug=True)
    codes2, scales2 = K.run(plan, X, y_debug=False)
    assert torch.equal(codes, codes2) and torch.equal(scales, scales2)
    return codes, scales, y


@pytest.mark.parametrize("n1", [16, 32, 48, 64])
@pytest.mark.parametrize("T", [1, 77, 3 * 2048 + 77])
def test_rsplit_parity_every_token(gpu, n1, T):
    """T = 6221 gives every workgroup several tokens (the next token's rows prefetched by
    each wave while the current one is computed); every token is checked."""
    inp = S.make(_workload(n1), T=T)
    plan, X = K.make_plan(inp, flags=FLAG)
    assert plan.kernel == f"fused_mfma_bf16_rsplit_{n1}x64_c", plan.kernel
    codes, scales, y = _run(inp, plan, X)
    rel, worst = K.check_all_tokens_chunked(inp, plan, codes, scales, y)
    print(f"[rsplit] {n1}x64 T={T} rel-L2 {rel:.3e} worst token {worst:.3e}", flush=True)


def test_rsplit_blocks_of_very_different_magnitude(gpu):
    """Each 16-row block picks its own scale for x^: blocks scaled by 2^40, 1, 2^-40 and
    2^-100 within one token (and the reverse order) must give the same relative error as
    ordinary tokens, and the exact codes of the oracle quantizer on the GPU's Y."""
    T = 64
    inp = S.make(_workload(64), T=T)
    X = O.bf16_bits_to_f64(inp.X).reshape(T, 64, 64)
    f = np.array([2.0 ** 40, 1.0, 2.0 ** -40, 2.0 ** -100])
    fac = np.where(np.arange(T)[:, None] % 2 == 0, f[None, :], f[None, ::-1])  # [T, 4]
    Xs = X * np.repeat(fac, 16, axis=1)[:, :, None]
    inp.X = S.to_bf16_bits(Xs.reshape(T, -1))
    plan, Xd = K.make_plan(inp, flags=FLAG)
    codes, scales, y = _run(inp, plan, Xd)
    rel, worst = K.check_all_tokens_chunked(inp, plan, codes, scales, y)
    print(f"[rsplit] mixed-magnitude blocks: rel-L2 {rel:.3e} worst token {worst:.3e}", flush=True)


@pytest.mark.parametrize("case", ["fp32_scales", "clip_zero", "zero_tokens", "zero_block", "strided"])
def test_rsplit_edge_cases(gpu, case):
    import torch
    wl = _workload(64, alpha=-math.inf) if case == "clip_zero" else _workload(64)
    T = 301
    inp = S.make(wl, T=T)
    if case == "zero_tokens":
        X0 = inp.X.copy()
        X0[[0, 150, T - 1]] = 0
        inp.X = X0
    if case == "zero_block":  # one 16-row block of some tokens all zero
        X0 = inp.X.copy().reshape(T, 64, 64)
        X0[::3, 16:32] = 0
        inp.X = X0.reshape(T, -1)
    sd = "fp32" if case == "fp32_scales" else inp.wl.scale_dtype
    plan, X = K.make_plan(inp, scale_dtype=sd, flags=FLAG)
    codes, scales, y = _run(inp, plan, X)
    K.check_plan_against_oracle(inp, plan, codes, scales, y)
    s = K.np_scales(scales)
    cn = codes.cpu().numpy()
    if case == "clip_zero":
        assert np.all(s == 0) and np.all(cn == 0)
    if case == "zero_tokens":
        assert np.all(s[[0, 150, T - 1]] == 0) and np.all(cn[[0, 150, T - 1]] == 0)
    if case == "strided":
        n = plan.n
        wide = torch.zeros((T, n + 96), dtype=torch.bfloat16, device=gpu)
        wide[:, 48:48 + n] = X
        c2, s2 = plan(wide[:, 48:48 + n])
        assert torch.equal(c2, codes) and torch.equal(s2, scales)


@pytest.mark.parametrize("n1", [16, 32, 48, 64])
def test_rsplit_matches_the_stream_split_bit_for_bit(gpu, n1):
    """The same roundings, scales and MFMA order as the stream kernel with c: a token gets
    the same Y, codes and step whichever of the two a call runs (a plan picks by batch
    size), including tokens scaled far outside fp16's range."""
    import torch
    T = 203
    inp = S.make(_workload(n1), T=T)
    x = O.bf16_bits_to_f64(inp.X)
    x[1::5] *= 2.0 ** 40
    x[2::5] *= 2.0 ** -60
    inp.X = S.to_bf16_bits(x)
    rp, X = K.make_plan(inp, flags=FLAG)
    sp, _ = K.make_plan(inp, flags=B.KQ_FLAG_SPLIT_STREAM)
    a = K.run(rp, X, y_debug=True)
    b = K.run(sp, X, y_debug=True)
    assert all(torch.equal(u, v) for u, v in zip(a, b))
