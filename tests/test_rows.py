"""GPU tests of per-row plans (KQ_FLAG_PER_ROW): identity left factor, one INT4 step per
row of V, e.g. per attention head of a key or value vector ahead of a quantized KV cache
("FlatQuant" page, Symbol Map: P_h, P_v). The oracle is the same transform with P1 = I
and the same per-token quantizer applied to every row of n2 values."""
from dataclasses import replace

import numpy as np
import pytest

import kqtest as K
from kronecker_factored_transforms_amd import binding as B
from kronecker_factored_transforms_amd import synth as S
from oracle import kq_oracle as O

pytestmark = pytest.mark.gpu

TOL_ROWS = 1e-5  # one bf16 x bf16 MFMA stage with fp32 accumulation: no bf16 intermediate


def _plan(inp, dev="cuda:0", scale_dtype=None):
    _, _, P2, _ = K.device_inputs(inp, dev)
    return B.Plan(None, P2, None, inp.alpha, scale_dtype or inp.wl.scale_dtype, n1=inp.wl.n1)


def _check(inp, codes, scales, y, clip, token_ids=None, scale_dtype=None):
    n1, n2 = inp.wl.n1, inp.wl.n2
    X = inp.X if token_ids is None else inp.X[token_ids]
    eye = S.to_bf16_bits(np.eye(n1))  # factors are given as bf16 bit patterns
    Y = O.transform(X, eye, inp.P2, None, inp.wl.dtype)
    rel = K.rel_l2(y, Y)
    assert rel <= TOL_ROWS, f"rel-L2 {rel:.3e}"
    T = X.shape[0]
    rows = np.ascontiguousarray(y, dtype=np.float32).reshape(T * n1, n2)
    q, s = O.quantize_per_token(rows, np.float32(clip), scale_dtype or inp.wl.scale_dtype)
    assert np.array_equal(np.asarray(codes), O.pack_int4(q).reshape(T, -1)), "codes differ"
    sv = np.asarray(scales).reshape(-1)
    assert np.array_equal(sv.view(np.uint8), s.view(np.uint8)), "scales differ"
    return rel


@pytest.mark.parametrize("n1,n2,T", [(8, 128, 777), (8, 128, 1), (8, 128, 3), (1, 128, 37),
                                     (3, 128, 50), (32, 128, 129), (8, 64, 300), (5, 64, 7)])
@pytest.mark.parametrize("scale_dtype", ["fp16", "fp32"])
def test_rows_parity(gpu, n1, n2, T, scale_dtype):
    import torch
    wl = replace(S.WORKLOADS["kv_h8_d128"], n1=n1, n2=n2, n_outliers=3)
    inp = S.make(wl, T=T)
    plan = _plan(inp, scale_dtype=scale_dtype)
    assert plan.kernel == f"fused_mfma_bf16_rows_{n2}"
    X = K.torch_from(inp.X, "bf16").to("cuda:0")
    codes, scales, y = K.run(plan, X, y_debug=True)
    codes2, scales2 = K.run(plan, X, y_debug=False)
    assert torch.equal(codes, codes2) and torch.equal(scales, scales2)
    assert tuple(scales.shape) == (T, n1)
    _check(inp, codes.cpu().numpy(), K.np_scales(scales), y.cpu().numpy(), plan.clip,
           scale_dtype=scale_dtype)


@pytest.mark.parametrize("n1,n2,T", [(8, 128, 300), (3, 64, 41)])
@pytest.mark.parametrize("alpha", [0.0, 2.0])
def test_rows_parity_clamped(gpu, n1, n2, T, alpha):
    """Clip ratios below 0.935 (sigmoid(0) = 0.5, sigmoid(2) = 0.88): the clamp to [-8, 7]
    changes codes, so the kernel must take its clamping quantizer."""
    wl = replace(S.WORKLOADS["kv_h8_d128"], n1=n1, n2=n2, n_outliers=3, alpha=alpha)
    inp = S.make(wl, T=T)
    plan = _plan(inp)
    assert plan.clip < 0.935
    X = K.torch_from(inp.X, "bf16").to("cuda:0")
    codes, scales, y = K.run(plan, X, y_debug=True)
    _check(inp, codes.cpu().numpy(), K.np_scales(scales), y.cpu().numpy(), plan.clip)
    # some codes sit at the clamp bound -8 (nibble 8) or 7
    nib = np.concatenate([codes.cpu().numpy() & 15, codes.cpu().numpy() >> 4]).ravel()
    assert np.any(nib == 7) and np.any(nib == 8)


def test_rows_strided_tokens(gpu):
    """Rows of a token sit at t * ldx + i * n2 (e.g. the key slice of a fused QKV output)."""
    import torch
    inp = S.make("kv_h8_d128", T=201)
    n = inp.wl.n
    plan = _plan(inp)
    big = torch.zeros((201, 3 * n), dtype=torch.bfloat16, device="cuda:0")
    big[:, n:2 * n] = K.torch_from(inp.X, "bf16").to("cuda:0")
    X = big[:, n:2 * n]
    assert X.stride(0) == 3 * n
    codes, scales, y = K.run(plan, X, y_debug=True)
    _check(inp, codes.cpu().numpy(), K.np_scales(scales), y.cpu().numpy(), plan.clip)


def test_rows_full_size_sampled(gpu):
    """The 64k-token workload in the benchmark's launch; sampled tokens against the oracle."""
    import torch
    inp = S.make("kv_h8_d128")
    plan = _plan(inp)
    X = K.torch_from(inp.X, "bf16").to("cuda:0")
    codes, scales = K.run(plan, X, y_debug=False)
    rng = np.random.default_rng(3)
    ids = np.unique(np.concatenate([[0, inp.wl.T - 1], rng.integers(0, inp.wl.T, 300)]))
    sub = S.make("kv_h8_d128", token_ids=ids)
    Xs = K.torch_from(sub.X, "bf16").to("cuda:0")
    cs, ss, ys = K.run(plan, Xs, y_debug=True)
    # the same tokens give the same codes inside the full launch
    assert torch.equal(codes[torch.from_numpy(ids).cuda()], cs)
    assert torch.equal(scales[torch.from_numpy(ids).cuda()], ss)
    _check(sub, cs.cpu().numpy(), K.np_scales(ss), ys.cpu().numpy(), plan.clip)


def test_rows_argument_errors(gpu):
    import torch
    inp = S.make("kv_h8_d128", T=4)
    X, P1, P2, _ = K.device_inputs(inp)
    # P1 given with the flag, or missing without it
    with pytest.raises(B.KqError) as e:
        B.kq_create(8, 128, "bf16", "fp16", P1, P2, None, 3.0, None, B.KQ_FLAG_PER_ROW)
    assert e.value.status == B.KQ_ERR_INVALID_ARG
    with pytest.raises(B.KqError) as e:
        B.kq_create(8, 128, "bf16", "fp16", None, P2, None, 3.0, None, 0)
    assert e.value.status == B.KQ_ERR_INVALID_ARG
    c = torch.ones(1024, dtype=torch.float32, device="cuda:0")
    with pytest.raises(B.KqError) as e:
        B.kq_create(8, 128, "bf16", "fp16", None, P2, c, 3.0, None, B.KQ_FLAG_PER_ROW)
    assert e.value.status == B.KQ_ERR_INVALID_ARG
    with pytest.raises(B.KqError) as e:   # no rows kernel for n2 = 32
        B.kq_create(8, 32, "bf16", "fp16", None, P2[:32, :32].contiguous(), None, 3.0, None,
                    B.KQ_FLAG_PER_ROW)
    assert e.value.status == B.KQ_ERR_UNSUPPORTED
