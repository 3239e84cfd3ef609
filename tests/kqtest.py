"""Helpers shared by the GPU tests: move seeded inputs to the device, run the HIP path
through the C ABI, and compare with the oracle."""
import math

import numpy as np

from kronecker_factored_transforms_amd import binding as B
from kronecker_factored_transforms_amd import synth as S
from oracle import kq_oracle as O

TOL = {"bf16": 2e-3, "fp32": 1e-5}   # rel-L2 of the transformed tensor vs the fp64 oracle


def torch_from(a, dtype_name):
    import torch
    if dtype_name == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))


def device_inputs(inp, dev="cuda:0"):
    d = inp.wl.dtype
    X = torch_from(inp.X, d).to(dev)
    P1 = torch_from(inp.P1, d).to(dev)
    P2 = torch_from(inp.P2, d).to(dev)
    c = None
    if inp.c is not None:
        import torch
        c = torch.from_numpy(inp.c).to(dev)
    return X, P1, P2, c


def make_plan(inp, dev="cuda:0", scale_dtype=None, flags=0, P1=None, P2=None, c="inp"):
    X, dP1, dP2, dc = device_inputs(inp, dev)
    plan = B.Plan(dP1 if P1 is None else P1, dP2 if P2 is None else P2,
                  dc if isinstance(c, str) else c, inp.alpha,
                  scale_dtype or inp.wl.scale_dtype, flags=flags)
    return plan, X


def run(plan, X, y_debug=True):
    import torch
    out = plan(X, y_debug=y_debug)
    torch.cuda.synchronize()
    return out


def np_scales(s):
    import torch
    if s.dtype == torch.float16:
        return s.cpu().view(torch.int16).numpy().view(np.float16)
    return s.cpu().numpy()


def rel_l2(y, Y):
    y = np.asarray(y, dtype=np.float64)
    Y = np.asarray(Y, dtype=np.float64)
    den = np.linalg.norm(Y)
    return float(np.linalg.norm(y - Y) / den) if den else float(np.linalg.norm(y))


def oracle_quant_bits(y, clip, scale_dtype):
    """Oracle quantizer on the GPU's own fp32 Y: (packed codes, scales)."""
    q, s = O.quantize_per_token(np.ascontiguousarray(y, dtype=np.float32), np.float32(clip), scale_dtype)
    return O.pack_int4(q), s


def assert_quant_bit_exact(codes, scales, y, clip, scale_dtype):
    oc, os_ = oracle_quant_bits(y, clip, scale_dtype)
    codes = np.asarray(codes)
    if not np.array_equal(codes, oc):
        bad = np.argwhere(codes != oc)
        t, m = bad[0]
        raise AssertionError(
            f"{len(bad)} code bytes differ; first at token {t} byte {m}: gpu {codes[t, m]:#04x} "
            f"oracle {oc[t, m]:#04x} (y = {y[t, 2 * m]!r}, {y[t, 2 * m + 1]!r})")
    sv = np.asarray(scales)
    assert sv.dtype == os_.dtype
    assert np.array_equal(sv.view(np.uint8), os_.view(np.uint8)), "scales differ"


def check_against_oracle(inp, codes, scales, y, clip, token_ids=None, scale_dtype=None):
    """Transform within tolerance of the fp64 oracle; codes/scales bit-exact vs the oracle
    quantizer on the GPU's y. `token_ids` selects which rows of inp.X the outputs are."""
    sd = scale_dtype or inp.wl.scale_dtype
    X = inp.X if token_ids is None else inp.X[token_ids]
    Y = O.transform(X, inp.P1, inp.P2, inp.c, inp.wl.dtype)
    rel = rel_l2(y, Y)
    assert rel <= TOL[inp.wl.dtype], f"rel-L2 {rel:.3e} > {TOL[inp.wl.dtype]:.0e}"
    assert_quant_bit_exact(codes, scales, y, clip, sd)
    assert clip == float(O.clip_ratio(inp.alpha)) or (math.isinf(inp.alpha) and clip in (0.0, 1.0))
    return rel


def check_plan_against_oracle(inp, plan, codes, scales, y):
    """Any plan's outputs for inp.X: a Kronecker plan (within the dtype's tolerance of the
    fp64 oracle) or a per-row plan (identity left factor, one step per row of n2 values,
    within 1e-5), with INT4 or INT8 codes bit-exact against the oracle quantizer applied
    to the GPU's own y. Arguments are torch tensors."""
    import torch
    n1, n2 = inp.wl.n1, inp.wl.n2
    T = inp.X.shape[0]
    y = y.cpu().numpy()
    sd = "fp16" if plan.scale_dtype == torch.float16 else "fp32"
    if plan.per_row:
        Y = O.transform(inp.X, S.to_bf16_bits(np.eye(n1)), inp.P2, None, inp.wl.dtype)
        tol, rows = 1e-5, y.reshape(T * n1, n2)
    else:
        Y = O.transform(inp.X, inp.P1, inp.P2, inp.c, inp.wl.dtype)
        tol, rows = TOL[inp.wl.dtype], y
    rel = rel_l2(y, Y)
    assert rel <= tol, f"rel-L2 {rel:.3e} > {tol:.0e}"
    q, s = O.quantize_per_token(np.ascontiguousarray(rows, dtype=np.float32),
                                np.float32(plan.clip), sd, bits=plan.bits)
    packed = (O.pack_int4(q) if plan.bits == 4 else O.pack_int8(q)).reshape(T, -1)
    assert np.array_equal(codes.cpu().numpy(), packed), "codes differ"
    assert np.array_equal(np_scales(scales).reshape(-1).view(np.uint8), s.view(np.uint8)), \
        "scales differ"
    return rel


def check_all_tokens_chunked(inp, plan, codes, scales, y, chunk=4096):
    """Every token of a full-size call against the oracle, a chunk of tokens at a time (host
    memory stays bounded): the fp32 Y within the dtype's rel-L2 tolerance over the whole
    tensor (and the worst per-token rel-L2 reported), codes and steps bit-exact against the
    oracle quantizer on the GPU's own Y. Arguments are torch tensors of the whole call."""
    import torch
    T = int(codes.shape[0])
    sd = "fp16" if plan.scale_dtype == torch.float16 else "fp32"
    err2 = ref2 = 0.0
    worst = 0.0
    for a in range(0, T, chunk):
        b = min(T, a + chunk)
        yc = y[a:b].cpu().numpy()
        Y = O.transform(inp.X[a:b], inp.P1, inp.P2, inp.c, inp.wl.dtype)
        d = yc.astype(np.float64) - Y
        e_tok = np.einsum("ij,ij->i", d, d)
        r_tok = np.einsum("ij,ij->i", Y, Y)
        err2 += float(e_tok.sum())
        ref2 += float(r_tok.sum())
        nz = r_tok > 0
        if nz.any():
            worst = max(worst, float(np.sqrt((e_tok[nz] / r_tok[nz]).max())))
        q, s = O.quantize_per_token(np.ascontiguousarray(yc, dtype=np.float32), np.float32(plan.clip),
                                    sd, bits=plan.bits)
        packed = O.pack_int4(q) if plan.bits == 4 else O.pack_int8(q)
        cc = codes[a:b].cpu().numpy()
        if not np.array_equal(cc, packed):
            bad = np.argwhere(cc != packed)
            raise AssertionError(f"{len(bad)} code bytes differ; first at token {a + bad[0][0]}")
        assert np.array_equal(np_scales(scales[a:b]).view(np.uint8), s.view(np.uint8)), \
            f"scales differ in tokens {a}..{b}"
    rel = float(np.sqrt(err2 / ref2)) if ref2 else float(np.sqrt(err2))
    assert rel <= TOL[inp.wl.dtype], f"rel-L2 {rel:.3e} > {TOL[inp.wl.dtype]:.0e}"
    return rel, worst
