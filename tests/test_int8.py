"""GPU tests of INT8 plans (KQ_FLAG_INT8): the same transform, codes from the b = 8
quantizer (divisor 127, clamp to [-128, 127], one byte per value). Codes and scales must
be bit-exact against the oracle quantizer on the GPU's own fp32 Y; Y within the bf16
tolerance of the fp64 oracle."""
from dataclasses import replace

import numpy as np
import pytest

import kqtest as K
from kronecker_factored_transforms_amd import binding as B
from kronecker_factored_transforms_amd import synth as S
from oracle import kq_oracle as O

pytestmark = pytest.mark.gpu


def _plan(inp, dev="cuda:0", scale_dtype=None):
    X, P1, P2, c = K.device_inputs(inp, dev)
    return B.Plan(P1, P2, c, inp.alpha, scale_dtype or inp.wl.scale_dtype, bits=8), X


def _check(inp, codes, scales, y, clip, token_ids=None, scale_dtype=None):
    X = inp.X if token_ids is None else inp.X[token_ids]
    Y = O.transform(X, inp.P1, inp.P2, inp.c, inp.wl.dtype)
    rel = K.rel_l2(y, Y)
    assert rel <= K.TOL[inp.wl.dtype], f"rel-L2 {rel:.3e}"
    q, s = O.quantize_per_token(np.ascontiguousarray(y, np.float32), np.float32(clip),
                                scale_dtype or inp.wl.scale_dtype, bits=8)
    assert np.array_equal(np.asarray(codes), O.pack_int8(q)), "codes differ"
    assert np.array_equal(np.asarray(scales).view(np.uint8), s.view(np.uint8)), "scales differ"


SHAPES = [(64, 128, False), (64, 64, True), (32, 128, False), (16, 64, True), (48, 64, False),
          (16, 128, False)]


@pytest.mark.parametrize("n1,n2,with_c", SHAPES)
@pytest.mark.parametrize("T", [1, 203])
def test_int8_parity(gpu, n1, n2, with_c, T):
    import torch
    base = S.WORKLOADS["attn_n4096"] if with_c else S.WORKLOADS["hidden_n8192"]
    wl = replace(base, n1=n1, n2=n2, n_outliers=4, pivot_channels=0)
    inp = S.make(wl, T=T)
    plan, X = _plan(inp)
    # small batches of the stream shapes without c run on the pair split
    small = f"fused_mfma_bf16_pair_{n1}x{n2}_int8" if not with_c else plan.kernel
    assert plan.kernel.endswith("_int8") and plan.kernel_for(T) == small
    codes, scales, y = K.run(plan, X, y_debug=True)
    codes2, scales2 = K.run(plan, X, y_debug=False)
    assert torch.equal(codes, codes2) and torch.equal(scales, scales2)
    assert tuple(codes.shape) == (T, n1 * n2)
    _check(inp, codes.cpu().numpy(), K.np_scales(scales), y.cpu().numpy(), plan.clip)


@pytest.mark.parametrize("n1,n2", [(64, 128), (16, 64), (48, 128)])
@pytest.mark.parametrize("T", [1, 77, 1500])
def test_int8_pair_split(gpu, n1, n2, T):
    """INT8 codes from the pair split (two waves per token), forced with its flag at any
    T, and the same codes from the default plan, which runs it below about four tokens
    per CU and the stream kernel above."""
    import torch
    wl = replace(S.WORKLOADS["hidden_n8192"], n1=n1, n2=n2, n_outliers=4, pivot_channels=0)
    inp = S.make(wl, T=T)
    X, P1, P2, c = K.device_inputs(inp)
    pair = B.Plan(P1, P2, None, inp.alpha, inp.wl.scale_dtype, bits=8, flags=B.KQ_FLAG_SPLIT_PAIR)
    assert pair.kernel == f"fused_mfma_bf16_pair_{n1}x{n2}_int8"
    codes, scales, y = K.run(pair, X, y_debug=True)
    codes2, scales2 = K.run(pair, X, y_debug=False)
    assert torch.equal(codes, codes2) and torch.equal(scales, scales2)
    _check(inp, codes.cpu().numpy(), K.np_scales(scales), y.cpu().numpy(), pair.clip)
    dflt, _ = _plan(inp)
    c3, s3 = K.run(dflt, X, y_debug=False)
    assert torch.equal(codes, c3) and torch.equal(scales, s3)


def test_int8_full_size_sampled(gpu):
    import torch
    inp = S.make("hidden_n8192")
    plan, X = _plan(inp)
    codes, scales = K.run(plan, X, y_debug=False)
    rng = np.random.default_rng(8)
    ids = np.unique(np.concatenate([[0, inp.wl.T - 1], rng.integers(0, inp.wl.T, 200)]))
    sub = S.make("hidden_n8192", token_ids=ids)
    Xs = K.torch_from(sub.X, "bf16").to("cuda:0")
    cs, ss, ys = K.run(plan, Xs, y_debug=True)
    idx = torch.from_numpy(ids).cuda()
    assert torch.equal(codes[idx], cs) and torch.equal(scales[idx], ss)
    _check(sub, cs.cpu().numpy(), K.np_scales(ss), ys.cpu().numpy(), plan.clip)


# Shapes whose default kernel is a register kernel, which has no INT8 epilogue: n2 = 32,
# and 16..48 x 128 with a per-channel scale.
INT8_LEFT_OUT = [(16, 32, False), (32, 32, True), (16, 128, True), (32, 128, True),
                 (48, 128, True)]


@pytest.mark.parametrize("n1,n2,with_c", INT8_LEFT_OUT)
def test_int8_unsupported_shapes(gpu, n1, n2, with_c):
    import torch
    wl = replace(S.WORKLOADS["hidden_n8192"], n1=n1, n2=n2, n_outliers=2, pivot_channels=0)
    inp = S.make(wl, T=4)
    X, P1, P2, c = K.device_inputs(inp)
    c = torch.ones(n1 * n2, dtype=torch.float32, device=gpu) if with_c else None
    with pytest.raises(B.KqError) as e:
        B.kq_create(n1, n2, "bf16", "fp16", P1, P2, c, 1.0, None, B.KQ_FLAG_INT8)
    assert e.value.status == B.KQ_ERR_UNSUPPORTED


COLS_SHAPES = [(112, 128, True), (86, 128, True), (108, 128, False), (96, 128, True),
               (128, 128, True), (64, 128, True), (80, 128, False), (128, 224, False),
               (128, 160, False), (128, 256, False), (64, 112, True), (128, 144, False),
               (32, 48, True), (56, 64, True), (56, 64, False), (64, 104, True),
               (64, 104, False), (40, 64, True), (64, 88, False), (64, 96, True),
               (80, 112, False)]


@pytest.mark.parametrize("n1,n2,with_c", COLS_SHAPES)
@pytest.mark.parametrize("T", [1, 203])
def test_int8_cols_parity(gpu, n1, n2, with_c, T):
    """INT8 codes from the column kernel (two workgroups per CU, column halves, padded
    n1, P2 in registers or L2 for n2 > 128), e.g. down-projection inputs kept at 8 bits."""
    import torch
    base = S.WORKLOADS["down_proj_n14336"] if with_c else S.WORKLOADS["hidden_n8192"]
    wl = replace(base, n1=n1, n2=n2, n_outliers=4, pivot_channels=0)
    inp = S.make(wl, T=T)
    plan, X = _plan(inp)
    assert plan.kernel == f"fused_mfma_bf16_cols_{n1}x{n2}{'_c' if with_c else ''}_int8", plan.kernel
    codes, scales, y = K.run(plan, X, y_debug=True)
    codes2, scales2 = K.run(plan, X, y_debug=False)
    assert torch.equal(codes, codes2) and torch.equal(scales, scales2)
    assert tuple(codes.shape) == (T, n1 * n2)
    _check(inp, codes.cpu().numpy(), K.np_scales(scales), y.cpu().numpy(), plan.clip)


@pytest.mark.parametrize("name", ["down_proj_n14336", "down_proj_n28672"])
def test_int8_cols_strided_and_full_size_sampled(gpu, name):
    """Full-size INT8 run in the bench's launch configuration, sampled tokens checked
    against the oracle; the same codes through a row stride larger than the row."""
    import torch
    inp = S.make(name)
    plan, X = _plan(inp)
    codes, scales = K.run(plan, X, y_debug=False)
    n = inp.wl.n
    T = 3 * 256 + 77
    wide = torch.zeros((T, n + 64), dtype=torch.bfloat16, device=gpu)
    wide[:, 32:32 + n] = X[:T]
    c2, s2 = K.run(plan, wide[:, 32:32 + n], y_debug=False)
    assert torch.equal(c2, codes[:T]) and torch.equal(s2, scales[:T])
    rng = np.random.default_rng(9)
    ids = np.unique(np.concatenate([[0, inp.wl.T - 1], rng.integers(0, inp.wl.T, 100)]))
    sub = S.make(name, token_ids=ids)
    Xs = K.torch_from(sub.X, "bf16").to("cuda:0")
    cs, ss, ys = K.run(plan, Xs, y_debug=True)
    idx = torch.from_numpy(ids).cuda()
    assert torch.equal(codes[idx], cs) and torch.equal(scales[idx], ss)
    _check(sub, cs.cpu().numpy(), K.np_scales(ss), ys.cpu().numpy(), plan.clip)


@pytest.mark.parametrize("n1,n2,T", [(8, 128, 777), (3, 64, 41), (1, 128, 5), (32, 128, 129)])
@pytest.mark.parametrize("alpha", [3.0, 0.0])
def test_int8_per_row_parity(gpu, n1, n2, T, alpha):
    """Per-row plans with INT8 codes (a per-head transform ahead of an 8-bit KV cache):
    one byte per value in row-major Y order, one step per row, bit-exact against the
    oracle quantizer applied to each row of the GPU's own Y."""
    import torch
    wl = replace(S.WORKLOADS["kv_h8_d128"], n1=n1, n2=n2, n_outliers=3, alpha=alpha)
    inp = S.make(wl, T=T)
    _, _, P2, _ = K.device_inputs(inp)
    plan = B.Plan(None, P2, None, inp.alpha, inp.wl.scale_dtype, n1=n1, bits=8)
    assert plan.kernel == f"fused_mfma_bf16_rows_{n2}_int8"
    X = K.torch_from(inp.X, "bf16").to("cuda:0")
    codes, scales, y = K.run(plan, X, y_debug=True)
    codes2, scales2 = K.run(plan, X, y_debug=False)
    assert torch.equal(codes, codes2) and torch.equal(scales, scales2)
    assert tuple(codes.shape) == (T, n1 * n2) and tuple(scales.shape) == (T, n1)
    eye = S.to_bf16_bits(np.eye(n1))
    Y = O.transform(inp.X, eye, inp.P2, None, "bf16")
    assert K.rel_l2(y.cpu().numpy(), Y) <= 1e-5
    rows = np.ascontiguousarray(y.cpu().numpy(), dtype=np.float32).reshape(T * n1, n2)
    q, s = O.quantize_per_token(rows, np.float32(plan.clip), inp.wl.scale_dtype, bits=8)
    assert np.array_equal(codes.cpu().numpy(), O.pack_int8(q).reshape(T, -1)), "codes differ"
    assert np.array_equal(K.np_scales(scales).reshape(-1).view(np.uint8), s.view(np.uint8))
    if alpha == 0.0:  # clip 0.5: the clamp to [-128, 127] is reached
        qq = codes.cpu().numpy().view(np.int8)
        assert qq.max() == 127 and qq.min() == -128
