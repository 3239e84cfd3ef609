"""GPU tests of the weight side: the INT4 x INT4 consumer (kq_int4_gemm) and the weight-side
factors (kq_weight_factor), through the C ABI.

Parity: bit-exact against the oracle's integer product with the fp32 epilogue (every
output dtype, both scale dtypes, ragged T and N around the 256 x 256 workgroup tile, and
exact multiples of it).
End to end ("FlatQuant" page, Learning the affine transformation: (X P)(P^-1 W^T) =
X W^T): activations through a kq plan with (P1, P2), weight rows through a kq plan with
(P1^-T, P2^-T), then the INT4 GEMM; the result must equal the oracle GEMM of the same
codes bit for bit, and approximate X W^T as closely as the oracle's own quantized path.
"""
import numpy as np
import pytest

import kqtest as K
from kronecker_factored_transforms_amd import binding as B
from kronecker_factored_transforms_amd import synth as S
from oracle import kq_oracle as O

pytestmark = pytest.mark.gpu


def _codes(rng, rows, k):
    return O.pack_int4(rng.integers(-8, 8, size=(rows, k)).astype(np.int8))


def _to_np(out):
    import torch
    if out.dtype == torch.bfloat16:
        return out.cpu().view(torch.int16).numpy().view(np.uint16)
    if out.dtype == torch.float16:
        return out.cpu().view(torch.int16).numpy().view(np.float16)
    return out.cpu().numpy()


@pytest.mark.parametrize("T,N,Kc", [(1, 4, 256), (37, 52, 512), (256, 256, 256),
                                    (300, 520, 1024), (512, 512, 512), (513, 260, 8192),
                                    (769, 772, 1024)])
@pytest.mark.parametrize("out_dtype", ["fp32", "bf16", "fp16"])
@pytest.mark.parametrize("scale_dtype", ["fp16", "fp32"])
def test_int4_gemm_bit_exact(gpu, T, N, Kc, out_dtype, scale_dtype):
    import torch
    rng = np.random.default_rng(T * 7 + N + Kc)
    cx, cw = _codes(rng, T, Kc), _codes(rng, N, Kc)
    sdt = np.float16 if scale_dtype == "fp16" else np.float32
    sx = rng.uniform(1e-3, 0.5, T).astype(sdt)
    sw = rng.uniform(1e-3, 0.5, N).astype(sdt)
    tdt = torch.float16 if scale_dtype == "fp16" else torch.float32
    dev = "cuda:0"
    out = B.int4_gemm(torch.from_numpy(cx).to(dev), torch.from_numpy(sx.view(np.int16) if sdt == np.float16 else sx).view(tdt).to(dev),
                      torch.from_numpy(cw).to(dev), torch.from_numpy(sw.view(np.int16) if sdt == np.float16 else sw).view(tdt).to(dev),
                      out_dtype)
    torch.cuda.synchronize()
    ref = O.int4_gemm(cx, sx, cw, sw, out_dtype)
    got = _to_np(out)
    assert got.shape == ref.shape
    if not np.array_equal(got.view(np.uint8), np.ascontiguousarray(ref).view(np.uint8)):
        bad = np.argwhere(got != ref)
        t, j = bad[0]
        raise AssertionError(f"{len(bad)} outputs differ; first [{t},{j}]: {got[t, j]!r} vs {ref[t, j]!r}")


def test_int4_gemm_strided_rows_and_output(gpu):
    """Row strides larger than the rows (ldxq, ldwq, ldo) and zero sizes."""
    import torch
    rng = np.random.default_rng(5)
    T, N, Kc = 70, 36, 512
    cx = np.zeros((T, Kc // 2 + 48), np.uint8)
    cw = np.zeros((N, Kc // 2 + 16), np.uint8)
    cx[:, :Kc // 2] = _codes(rng, T, Kc)
    cw[:, :Kc // 2] = _codes(rng, N, Kc)
    sx = rng.uniform(0.01, 1, T).astype(np.float32)
    sw = rng.uniform(0.01, 1, N).astype(np.float32)
    dev = "cuda:0"
    dx, dw = torch.from_numpy(cx).to(dev), torch.from_numpy(cw).to(dev)
    dsx, dsw = torch.from_numpy(sx).to(dev), torch.from_numpy(sw).to(dev)
    out = torch.full((T, N + 12), -1.0, dtype=torch.float32, device=dev)
    B.kq_int4_gemm(dx, cx.shape[1], dsx, T, dw, cw.shape[1], dsw, N, Kc, "fp32", "fp32", out,
                   N + 12)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = O.int4_gemm(cx[:, :Kc // 2], sx, cw[:, :Kc // 2], sw)
    assert np.array_equal(got[:, :N], ref)
    assert np.all(got[:, N:] == -1.0)  # nothing written past the N columns
    B.kq_int4_gemm(dx, cx.shape[1], dsx, 0, dw, cw.shape[1], dsw, N, Kc, "fp32", "fp32", out, N + 12)
    B.kq_int4_gemm(dx, cx.shape[1], dsx, T, dw, cw.shape[1], dsw, 0, Kc, "fp32", "fp32", out, N + 12)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), got)


def _ulp(v, mant_bits):
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - mant_bits), 0.0)


@pytest.mark.parametrize("m", [1, 8, 64, 112, 128, 256])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_weight_factor_is_the_inverse_transpose(gpu, m, dtype):
    """kq_weight_factor(P) against the oracle's inv(P)^T in fp64 (LAPACK's LU inverse, a
    different algorithm from the library's Gauss-Jordan): every entry within half a unit
    in the last place of the dtype, plus a margin for the fp64 error of the two
    eliminations; non-symmetric P, so a missing transpose fails."""
    import torch
    rng = np.random.default_rng(m * 3 + (dtype == "bf16"))
    P = np.eye(m) + 0.3 * rng.standard_normal((m, m)) / np.sqrt(m)
    dev = "cuda:0"
    if dtype == "bf16":
        Pb = S.to_bf16_bits(P)
        Pd = O.bf16_bits_to_f64(Pb)
        tP = K.torch_from(Pb, "bf16").to(dev)
    else:
        Pf = P.astype(np.float32)
        Pd = Pf.astype(np.float64)
        tP = torch.from_numpy(Pf).to(dev)
    out = B.weight_factor(tP)
    torch.cuda.synchronize()
    if dtype == "bf16":
        got = O.bf16_bits_to_f64(out.cpu().view(torch.int16).numpy().view(np.uint16))
    else:
        got = out.cpu().numpy().astype(np.float64)
    ref = O.weight_factors(Pd, Pd)[0]
    assert m == 1 or not np.allclose(ref, ref.T)
    tol = 0.5 * _ulp(ref, 7 if dtype == "bf16" else 23) + 1e-9 * np.abs(ref).max()
    err = np.abs(got - ref)
    assert np.all(err <= tol), (float(err.max()), np.unravel_index(np.argmax(err - tol), err.shape))
    # in place: out may be P itself
    B.kq_weight_factor(tP, m, tP.dtype, tP)
    torch.cuda.synchronize()
    assert torch.equal(tP.cpu(), out.cpu())


def test_weight_factor_refuses_singular_factors(gpu):
    import torch
    dev = "cuda:0"
    with pytest.raises(B.KqError) as e:
        B.weight_factor(torch.zeros((16, 16), dtype=torch.float32, device=dev))
    assert e.value.status == B.KQ_ERR_INVALID_ARG
    P = torch.eye(64, dtype=torch.bfloat16) + 0.05 * torch.randn(64, 64).to(torch.bfloat16)
    P[5] = 0  # a zero row of P: column 5 of P^T stays zero through the elimination
    with pytest.raises(B.KqError) as e:
        B.weight_factor(P.to(dev))
    assert e.value.status == B.KQ_ERR_INVALID_ARG
    # a regular factor afterwards still works
    assert torch.isfinite(B.weight_factor(torch.eye(8, device=dev)).float()).all()


def test_w4a4_layer_end_to_end(gpu):
    """Activations (hidden 8192, 64 x 128 orthogonal factors) and a synthetic weight matrix
    through their transforms and the INT4 GEMM."""
    import torch
    inp = S.make("hidden_n8192", T=300)
    n, N = inp.wl.n, 512
    rng = np.random.default_rng(21)
    W = S.to_bf16_bits(rng.standard_normal((N, n)) / np.sqrt(n))
    # weight-side factors (P^-1)^T from the library, from the bf16 activation factors
    dev = "cuda:0"
    plan_x, X = K.make_plan(inp)
    tQ1 = B.weight_factor(K.torch_from(inp.P1, "bf16").to(dev))
    tQ2 = B.weight_factor(K.torch_from(inp.P2, "bf16").to(dev))
    plan_w = B.Plan(tQ1, tQ2, None, float("inf"), "fp16")
    # the oracle's own weight-side factors, rounded to bf16, for its reference path
    Q1, Q2 = O.weight_factors(O.bf16_bits_to_f64(inp.P1), O.bf16_bits_to_f64(inp.P2))
    Q1b, Q2b = S.to_bf16_bits(Q1), S.to_bf16_bits(Q2)
    xq, sx = plan_x(X)
    wq, sw = plan_w(K.torch_from(W, "bf16").to(dev))
    out = B.int4_gemm(xq, sx, wq, sw, "fp32")
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    # the GEMM of the GPU's own codes: bit-exact
    cxn, cwn = xq.cpu().numpy(), wq.cpu().numpy()
    sxn, swn = K.np_scales(sx), K.np_scales(sw)
    assert np.array_equal(got, O.int4_gemm(cxn, sxn, cwn, swn))
    # the whole layer on the CPU from the same inputs
    Xf, Wf = O.bf16_bits_to_f64(inp.X), O.bf16_bits_to_f64(W)
    ref = Xf @ Wf.T
    _, ocx, osx = O.transform_quant(inp.X, inp.P1, inp.P2, None, inp.alpha, "bf16")
    _, ocw, osw = O.transform_quant(W, Q1b, Q2b, None, float("inf"), "bf16")
    oracle_out = O.int4_gemm(ocx, osx, ocw, osw).astype(np.float64)
    rel_gpu = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    rel_oracle = np.linalg.norm(oracle_out - ref) / np.linalg.norm(ref)
    print(f"[w4a4] rel error vs X W^T: gpu {rel_gpu:.4f}, oracle {rel_oracle:.4f}", flush=True)
    assert rel_gpu <= 1.02 * rel_oracle + 1e-3
    assert rel_gpu < 0.3
