"""GPU edge cases and exact special cases of the HIP path (through the C ABI).

Exact cases: identity and signed-permutation factors have entries 0 / +-1, so every
product and sum in the bf16 MFMA pipeline is exact; the GPU's Y must then equal the
(permuted, sign-flipped) input bit for bit, and the codes must match the oracle's whole
pipeline, not only its quantizer on the GPU's Y ("Kronecker Product", Definition: a
signed permutation factor pair moves entry (i, k) of V to (s1(i), s2(k)))."""
import math
from dataclasses import replace

import numpy as np
import pytest

import kqtest as K
from kronecker_factored_transforms_amd import binding as B
from kronecker_factored_transforms_amd import synth as S
from oracle import kq_oracle as O

pytestmark = pytest.mark.gpu


def _factor_tensor(P, dtype_name, dev):
    arr = S.to_bf16_bits(P) if dtype_name == "bf16" else P.astype(np.float32)
    return K.torch_from(arr, dtype_name).to(dev)


@pytest.mark.parametrize("name", ["hidden_n8192", "attn_n4096", "down_proj_n14336"])
@pytest.mark.parametrize("kind", ["identity", "signed_perm"])
def test_exact_factors_reproduce_permuted_input(gpu, name, kind):
    wl = replace(S.WORKLOADS[name], c_kind=None)
    inp = S.make(wl, T=129)
    rng = np.random.default_rng(5)
    if kind == "identity":
        P1, P2 = np.eye(wl.n1), np.eye(wl.n2)
    else:
        P1, P2 = S.signed_permutation(wl.n1, rng), S.signed_permutation(wl.n2, rng)
    dP1, dP2 = _factor_tensor(P1, wl.dtype, gpu), _factor_tensor(P2, wl.dtype, gpu)
    plan, X = K.make_plan(inp, P1=dP1, P2=dP2, c=None)
    codes, scales, y = K.run(plan, X)
    x = S.bf16_bits_to_f32(inp.X).astype(np.float64)
    Y = O.transform(x, P1, P2)                       # exact: +-1 times bf16 values
    assert np.array_equal(y.cpu().numpy(), Y.astype(np.float32))
    _, oc, os_ = O.transform_quant(x, P1, P2, None, inp.alpha, "fp64")
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(K.np_scales(scales), os_)


@pytest.mark.parametrize("flags,kernel", [(B.KQ_FLAG_SPLIT_REG1, "fused_mfma_bf16_reg1_64x64_c"),
                                          (B.KQ_FLAG_SPLIT_COLS, "fused_mfma_bf16_cols_64x64_c"),
                                          (0, "fused_mfma_bf16_rsplit_64x64_c")])
def test_power_of_two_channel_scale_is_exact(gpu, flags, kernel):
    """c = powers of two with identity factors: x*c has x's 8 significant bits.
    - The register kernels split x*c into bf16 hi + lo: lo is zero and Y is x*c exactly.
    - The stream, column and row-split kernels run on fp16 operands after a per-token power-of-two
      scale 2^s (s = 0 unless the bound max|x| max|c| leaves [2^-8, 2^15)): Y is x*c
      exactly wherever fp16 holds x*c 2^s exactly (at or above 2^-17, where its subnormal
      grid is still fine enough for 8 bits), and within half of fp16's smallest step 2^-25
      (times 2^-s) below that."""
    wl = S.WORKLOADS["attn_n4096"]
    inp = S.make(wl, T=70)
    rng = np.random.default_rng(6)
    c = (2.0 ** rng.integers(-3, 4, wl.n)).astype(np.float32)
    import torch
    dP1 = _factor_tensor(np.eye(wl.n1), "bf16", gpu)
    dP2 = _factor_tensor(np.eye(wl.n2), "bf16", gpu)
    plan, X = K.make_plan(inp, P1=dP1, P2=dP2, c=torch.from_numpy(c).to(gpu), flags=flags)
    assert plan.kernel_for(70) == kernel, plan.kernel_for(70)
    codes, scales, y = K.run(plan, X)
    xf = S.bf16_bits_to_f32(inp.X).astype(np.float64)
    x = xf * c.astype(np.float64)
    yc = y.cpu().numpy().astype(np.float64)
    if "reg1" in kernel:  # the hi / lo split
        assert np.array_equal(yc, x)
    else:  # fp16 operands
        bound = (np.abs(xf).max(axis=1).astype(np.float32) * np.float32(np.abs(c).max())).astype(np.float64)
        e = np.floor(np.log2(bound))
        s = np.where((e >= -8) & (e < 15), 0.0, np.clip(14 - e, -126, 127))[:, None]
        big = np.abs(x) * 2.0 ** s >= 2.0 ** -17
        assert big.mean() > 0.999
        assert np.array_equal(yc[big], x[big])
        assert np.all(np.abs(yc - x)[~big] <= (2.0 ** (-25 - s) * np.ones_like(x))[~big])
    K.assert_quant_bit_exact(codes.cpu().numpy(), K.np_scales(scales), y.cpu().numpy(), plan.clip, "fp16")


@pytest.mark.parametrize("name", ["hidden_n8192", "attn_n4096"])
def test_c_of_ones_matches_no_c(gpu, name):
    """c = ones gives x^ = x exactly; the with-c kernels then differ from the plain ones only
    in carrying Z in fp16 (instead of bf16) to stage 2. Both match the oracle, and their
    codes agree except for values that sit near a rounding boundary (at most one step)."""
    import torch
    inp = S.make(replace(S.WORKLOADS[name], c_kind=None), T=200)
    p0, X = K.make_plan(inp, c=None)
    p1, _ = K.make_plan(inp, c=torch.ones(inp.wl.n, dtype=torch.float32, device=gpu))
    assert p1.kernel.endswith("_c") and not p0.kernel.endswith("_c")
    a = K.run(p0, X)
    b = K.run(p1, X)
    for codes, scales, y in (a, b):
        K.check_against_oracle(inp, codes.cpu().numpy(), K.np_scales(scales), y.cpu().numpy(),
                               p0.clip)
    qa = O.unpack_int4(a[0].cpu().numpy()).astype(int)
    qb = O.unpack_int4(b[0].cpu().numpy()).astype(int)
    assert np.abs(qa - qb).max() <= 1 and np.mean(qa != qb) < 0.02


@pytest.mark.parametrize("T", [1, 2, 3, 5, 63, 65, 127, 1025])
def test_ragged_token_counts(gpu, T):
    for name in ("attn_n4096", "hidden_n8192"):
        inp = S.make(name, T=T)
        plan, X = K.make_plan(inp)
        codes, scales, y = K.run(plan, X)
        assert codes.shape == (T, inp.wl.n // 2) and scales.shape == (T,)
        K.check_against_oracle(inp, codes.cpu().numpy(), K.np_scales(scales), y.cpu().numpy(), plan.clip)


def test_zero_tokens_and_zero_rows(gpu):
    import torch
    inp = S.make("hidden_n8192", T=9)
    X0 = inp.X.copy()
    X0[[0, 4, 8]] = 0
    inp.X = X0
    plan, X = K.make_plan(inp)
    codes, scales, y = K.run(plan, X)
    s = K.np_scales(scales)
    assert np.all(s[[0, 4, 8]] == 0) and np.all(codes.cpu().numpy()[[0, 4, 8]] == 0)
    K.check_against_oracle(inp, codes.cpu().numpy(), s, y.cpu().numpy(), plan.clip)
    # T == 0 enqueues nothing and succeeds
    e = torch.empty((0, inp.wl.n), dtype=torch.bfloat16, device=gpu)
    c0, s0 = plan(e)
    assert c0.shape == (0, inp.wl.n // 2) and s0.shape == (0,)


def test_strided_rows(gpu):
    import torch
    inp = S.make("hidden_n8192", T=100)
    plan, X = K.make_plan(inp)
    wide = torch.zeros((100, inp.wl.n + 64), dtype=torch.bfloat16, device=gpu)
    wide[:, 32:32 + inp.wl.n] = X
    Xs = wide[:, 32:32 + inp.wl.n]
    assert Xs.stride(0) == inp.wl.n + 64
    a = K.run(plan, Xs)
    b = K.run(plan, X)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])


@pytest.mark.parametrize("alpha", [-math.inf, -2.0, 0.0, 1.0, 7.0, math.inf])
def test_clip_logits(gpu, alpha):
    wl = replace(S.WORKLOADS["hidden_n8192"], alpha=alpha)
    inp = S.make(wl, T=64)
    plan, X = K.make_plan(inp)
    assert plan.clip == float(O.clip_ratio(alpha))
    codes, scales, y = K.run(plan, X)
    K.check_against_oracle(inp, codes.cpu().numpy(), K.np_scales(scales), y.cpu().numpy(), plan.clip)
    if alpha == -math.inf:
        assert np.all(K.np_scales(scales) == 0) and np.all(codes.cpu().numpy() == 0)


def test_fp32_scales(gpu):
    inp = S.make("attn_n4096", T=100)
    plan, X = K.make_plan(inp, scale_dtype="fp32")
    codes, scales, y = K.run(plan, X)
    import torch
    assert scales.dtype == torch.float32
    K.check_against_oracle(inp, codes.cpu().numpy(), K.np_scales(scales), y.cpu().numpy(), plan.clip,
                           scale_dtype="fp32")


@pytest.mark.parametrize("name,T", [("attn_n4096", 50), ("hidden_n8192", 40), ("tiny_fp32_n64", 16)])
def test_generic_kernel_parity(gpu, name, T):
    inp = S.make(name, T=T)
    plan, X = K.make_plan(inp, flags=B.KQ_FLAG_FORCE_GENERIC)
    assert plan.kernel == "generic_fp32_fma"
    codes, scales, y = K.run(plan, X)
    rel = K.check_against_oracle(inp, codes.cpu().numpy(), K.np_scales(scales), y.cpu().numpy(), plan.clip)
    assert rel <= 1e-5          # fp32 contractions, no bf16 intermediate


def test_shapes_without_an_mfma_variant_use_the_generic_kernel(gpu):
    wl = replace(S.WORKLOADS["attn_n4096"], n1=12, n2=40, c_kind=None)
    inp = S.make(wl, T=33)
    plan, X = K.make_plan(inp)
    assert plan.kernel == "generic_fp32_fma"
    codes, scales, y = K.run(plan, X)
    K.check_against_oracle(inp, codes.cpu().numpy(), K.np_scales(scales), y.cpu().numpy(), plan.clip)


def test_argument_errors(gpu):
    import torch
    inp = S.make("hidden_n8192", T=8)
    plan, X = K.make_plan(inp)
    n = inp.wl.n
    codes = torch.empty((8, n // 2), dtype=torch.uint8, device=gpu)
    scales = torch.empty((8,), dtype=torch.float16, device=gpu)
    raw = torch.empty((8 * n + 8,), dtype=torch.bfloat16, device=gpu)
    with pytest.raises(B.KqError) as e:      # X not 16-byte aligned
        B.kq_transform_quant(plan.handle, raw.data_ptr() + 2, 8, n, codes, scales)
    assert e.value.status == B.KQ_ERR_ALIGNMENT
    with pytest.raises(B.KqError) as e:      # ldx < n
        B.kq_transform_quant(plan.handle, X, 8, n - 8, codes, scales)
    assert e.value.status == B.KQ_ERR_INVALID_ARG
    with pytest.raises(B.KqError) as e:      # T < 0
        B.kq_transform_quant(plan.handle, X, -1, n, codes, scales)
    assert e.value.status == B.KQ_ERR_INVALID_ARG
    # every case below is refused on the host, before anything is launched
    cbytes = torch.empty((8 * n // 2 + 16,), dtype=torch.uint8, device=gpu)
    sbytes = torch.empty((32,), dtype=torch.uint8, device=gpu)
    ybuf = torch.empty((8 * n + 4,), dtype=torch.float32, device=gpu)
    bad = [
        ((X, 8, n + 1, codes, scales, None), B.KQ_ERR_ALIGNMENT),                    # row pitch not 16 B
        ((X, 8, n, cbytes.data_ptr() + 1, scales, None), B.KQ_ERR_ALIGNMENT),       # codes
        ((X, 8, n, codes, sbytes.data_ptr() + 1, None), B.KQ_ERR_ALIGNMENT),        # fp16 steps
        ((X, 8, n, codes, scales, ybuf.data_ptr() + 4), B.KQ_ERR_ALIGNMENT),        # y_debug
        ((X, (1 << 40) // n + 1, n, codes, scales, None), B.KQ_ERR_INVALID_ARG),    # T * n > 2^40
        ((0, 8, n, codes, scales, None), B.KQ_ERR_INVALID_ARG),                     # null X
        ((X, 8, n, 0, scales, None), B.KQ_ERR_INVALID_ARG),                         # null codes
    ]
    for args, status in bad:
        with pytest.raises(B.KqError) as e:
            B.kq_transform_quant(plan.handle, *args)
        assert e.value.status == status, args[1:3]
    B.kq_transform_quant(plan.handle, 0, 0, n, 0, 0)  # T = 0: nothing to do, no pointer read
    with pytest.raises(B.KqError) as e:
        B.Plan(K.torch_from(inp.P1, "bf16").to(gpu), K.torch_from(inp.P2, "bf16").to(gpu),
               alpha=float("nan"))
    assert e.value.status == B.KQ_ERR_INVALID_ARG


def test_repeated_runs_are_identical(gpu):
    import torch
    inp = S.make("down_proj_n14336", T=512)
    plan, X = K.make_plan(inp)
    ref = K.run(plan, X)
    for _ in range(3):
        out = K.run(plan, X)
        assert all(torch.equal(a, b) for a, b in zip(ref, out))


def test_small_batches_switch_to_the_pair_split(gpu):
    """A default 64x128 plan runs the pair split (two waves per token) below a token
    count and the stream split (one wave per token) from there on; both sides of the
    switch match the oracle and the debug-free launch."""
    inp = S.make("hidden_n8192", T=8)
    plan, _ = K.make_plan(inp)
    assert plan.kernel.startswith("fused_mfma_bf16_stream_"), plan.kernel
    assert plan.kernel_for(1).startswith("fused_mfma_bf16_pair_")
    assert plan.kernel_for(1 << 20) == plan.kernel
    lo, hi = 1, 1 << 20  # smallest T that runs the stream split
    while lo < hi:
        mid = (lo + hi) // 2
        if plan.kernel_for(mid) == plan.kernel:
            hi = mid
        else:
            lo = mid + 1
    print(f"[switch] stream from T={lo}", flush=True)
    for T in (lo - 1, lo):
        inp = S.make("hidden_n8192", T=T)
        plan, X = K.make_plan(inp)
        import torch
        codes, scales, y = K.run(plan, X, y_debug=True)
        codes2, scales2 = K.run(plan, X, y_debug=False)
        assert torch.equal(codes, codes2) and torch.equal(scales, scales2)
        K.check_against_oracle(inp, codes.cpu().numpy(), K.np_scales(scales), y.cpu().numpy(),
                               plan.clip)


@pytest.mark.parametrize("name,small", [("attn_n4096", "fused_mfma_bf16_rsplit_64x64_c"),
                                        ("hidden_n7168", "fused_mfma_bf16_cols_64x112")])
def test_small_batches_without_a_pair_split_use_the_row_or_column_split(gpu, name, small):
    """Stream plans with no pair variant switch to another split for small batches: the row
    split with c, the column split for rows of 112 values; both sides of the switch match
    the oracle, and the same tokens give the same codes on both sides."""
    import torch
    inp = S.make(name, T=8)
    plan, _ = K.make_plan(inp)
    assert plan.kernel.startswith("fused_mfma_bf16_stream_"), plan.kernel
    assert plan.kernel_for(8) == small and plan.kernel_for(1 << 20) == plan.kernel
    lo, hi = 1, 1 << 20
    while lo < hi:
        mid = (lo + hi) // 2
        if plan.kernel_for(mid) == plan.kernel:
            hi = mid
        else:
            lo = mid + 1
    inp = S.make(name, T=lo)
    plan, X = K.make_plan(inp)
    big_codes, big_scales, y = K.run(plan, X, y_debug=True)
    K.check_against_oracle(inp, big_codes.cpu().numpy(), K.np_scales(big_scales), y.cpu().numpy(),
                           plan.clip)
    c_small, s_small = K.run(plan, X[: lo - 1], y_debug=False)
    assert torch.equal(c_small, big_codes[: lo - 1]) and torch.equal(s_small, big_scales[: lo - 1])


# The kernels behind the padded and widened shapes, through the same edge cases: fp32
# steps, clip 0 (every code and step zero), a token of zeros among others, and T = 0.
EDGE_CASES = [
    ("hidden_n7168", 4, "fused_mfma_bf16_stream_64x112"),
    ("ffn_n11008", 4, "fused_mfma_bf16_cols_86x128_c"),
    ("ffn_n18432", 4, "fused_mfma_bf16_cols_128x144"),
    ("down_proj_n14336", 8, "fused_mfma_bf16_cols_112x128_c_int8"),
    ("hidden_n8192", 8, "fused_mfma_bf16_stream_64x128_int8"),
]


@pytest.mark.parametrize("name,bits,kernel", EDGE_CASES)
@pytest.mark.parametrize("case", ["fp32_scales", "clip_zero", "zero_token"])
def test_widened_kernels_edge_cases(gpu, name, bits, kernel, case):
    import torch
    wl = S.WORKLOADS[name]
    if case == "clip_zero":
        wl = replace(wl, alpha=-math.inf)
    T = 1100  # at or above the small-batch switch, so the named kernel runs
    inp = S.make(wl, T=T)
    if case == "zero_token":
        X0 = inp.X.copy()
        X0[[0, 517, T - 1]] = 0
        inp.X = X0
    X, P1, P2, c = K.device_inputs(inp)
    sd = "fp32" if case == "fp32_scales" else inp.wl.scale_dtype
    plan = B.Plan(P1, P2, c, inp.alpha, sd, bits=bits)
    assert plan.kernel_for(T) == kernel, plan.kernel_for(T)
    codes, scales, y = K.run(plan, X, y_debug=True)
    K.check_plan_against_oracle(inp, plan, codes, scales, y)
    s = K.np_scales(scales)
    cn = codes.cpu().numpy()
    if case == "clip_zero":
        assert np.all(s == 0) and np.all(cn == 0)
    if case == "zero_token":
        assert np.all(s[[0, 517, T - 1]] == 0) and np.all(cn[[0, 517, T - 1]] == 0)
    e = torch.empty((0, inp.wl.n), dtype=torch.bfloat16, device=gpu)
    c0, s0 = plan(e)
    assert c0.shape == (0, inp.wl.n * bits // 8) and s0.shape == (0,)


# Reading R9 on every kernel family: with fp32 steps, a token whose absmax is 2^-126 has
# the step fp32(2^-126 / 7) < 2^-128, whose reciprocal overflows fp32; that step counts as
# an underflow (stored 0, codes 0). Identity factors keep Y = X exactly (normal numbers,
# entries 0 / 1), so the tiny tokens reach the quantizer unchanged.
TINY_STEP_CASES = [
    ("hidden_n8192", 1100, 0, "fused_mfma_bf16_stream_64x128"),
    ("hidden_n8192", 37, 0, "fused_mfma_bf16_pair_64x128"),
    ("down_proj_n14336", 301, 0, "fused_mfma_bf16_cols_112x128_c"),
    ("attn_n4096", 1100, 0, "fused_mfma_bf16_stream_64x64_c"),
    ("hidden_n8192", 203, B.KQ_FLAG_FORCE_GENERIC, "generic_fp32_fma"),
    ("tiny_fp32_n64", 16, 0, "generic_fp32_fma"),
]


@pytest.mark.parametrize("name,T,flags,kernel", TINY_STEP_CASES)
def test_fp32_step_with_overflowing_reciprocal_is_an_underflow(gpu, name, T, flags, kernel):
    import torch
    wl = S.WORKLOADS[name]
    inp = S.make(wl, T=T)
    x = (S.bf16_bits_to_f32(inp.X) if wl.dtype == "bf16" else inp.X).astype(np.float32)
    tiny = [0, T // 2, T - 1]
    x[tiny] = 0
    x[tiny, 5] = np.float32(2.0 ** -126)      # step fp32(2^-126 / 7) < 2^-128: underflow
    x[tiny, 9] = -np.float32(2.0 ** -127)
    x[1] = 0
    x[1, 3] = np.float32(2.0 ** -122)         # step ~ 2^-125 > 2^-128: quantized normally
    x[1, 4] = -np.float32(2.0 ** -124)
    inp.X = S.to_bf16_bits(x.astype(np.float64)) if wl.dtype == "bf16" else x
    c = None
    if inp.c is not None:
        c = torch.ones(wl.n, dtype=torch.float32, device=gpu)
    dP1 = _factor_tensor(np.eye(wl.n1), wl.dtype, gpu)
    dP2 = _factor_tensor(np.eye(wl.n2), wl.dtype, gpu)
    plan, X = K.make_plan(inp, P1=dP1, P2=dP2, c=c, scale_dtype="fp32", flags=flags)
    assert plan.kernel_for(T) == kernel, plan.kernel_for(T)
    codes, scales, y = K.run(plan, X)
    yc = y.cpu().numpy()
    special = tiny + [1]                           # powers of two: exact on every kernel
    assert np.array_equal(yc[special], x[special])
    # identity factors: the other tokens are exact too, except on the fp16-operand kernels
    # (the with-c stream and column kernels) for values below fp16's 2^-17, which round to
    # its subnormal grid (half-step 2^-25)
    assert np.max(np.abs(yc.astype(np.float64) - x)) <= 2.0 ** -25
    K.assert_quant_bit_exact(codes.cpu().numpy(), K.np_scales(scales), yc, plan.clip, "fp32")
    s = K.np_scales(scales)
    cn = codes.cpu().numpy()
    assert np.all(s[tiny] == 0) and np.all(cn[tiny] == 0)
    assert s[1] > 0 and np.any(cn[1] != 0)


# The with-c stream and column kernels carry Z to stage 2 in fp16 after a per-token
# power-of-two scale chosen from the token's largest |Z|; tokens far outside fp16's range
# (times 2^40 or 2^-60) take the scaled path, ordinary ones the unscaled one. Every token
# must still match the oracle, and both kernels of a plan give the same codes.
@pytest.mark.parametrize("name,T,kernel", [
    ("attn_n4096", 1100, "fused_mfma_bf16_stream_64x64_c"),
    ("attn_n4096", 300, "fused_mfma_bf16_rsplit_64x64_c"),
    ("down_proj_n14336", 301, "fused_mfma_bf16_cols_112x128_c"),
    ("ffn_n11008", 203, "fused_mfma_bf16_cols_86x128_c")])
def test_with_c_kernels_scale_z_into_fp16_range(gpu, name, T, kernel):
    import torch
    inp = S.make(name, T=T)
    x = O.bf16_bits_to_f64(inp.X)
    for i, k in enumerate((40, -60, 20, -30)):
        x[i::7] *= 2.0 ** k        # tokens 0, 7, 14, ... times 2^40; 1, 8, ... times 2^-60
    inp.X = S.to_bf16_bits(x)
    plan, X = K.make_plan(inp)
    assert plan.kernel_for(T) == kernel, plan.kernel_for(T)
    codes, scales, y = K.run(plan, X)
    K.check_plan_against_oracle(inp, plan, codes, scales, y)
    if name == "attn_n4096" and T > 1024:   # the small-batch split writes the same codes
        c2, s2 = K.run(plan, X[:1000], y_debug=False)
        assert plan.kernel_for(1000) == "fused_mfma_bf16_rsplit_64x64_c"
        assert torch.equal(c2, codes[:1000]) and torch.equal(s2, scales[:1000])


@pytest.mark.parametrize("name", ["hidden_n8192", "attn_n4096", "hidden_n7168", "kv_h8_d128"])
def test_codes_do_not_depend_on_the_batch_size(gpu, name):
    """A default plan may run another work split for small batches (include/kq.h,
    kq_plan_kernel_name_for: both compute the same Y and codes). The same tokens in a
    small and a large call give bit-identical Y, codes and steps."""
    import torch
    small, big = 300, 2200
    inp = S.make(name, T=big)
    X, P1, P2, c = K.device_inputs(inp)
    if inp.wl.per_row:
        plan = B.Plan(None, P2, None, inp.alpha, inp.wl.scale_dtype, n1=inp.wl.n1)
    else:
        plan = B.Plan(P1, P2, c, inp.alpha, inp.wl.scale_dtype)
    print(f"[batch] {name}: T={small} {plan.kernel_for(small)}, T={big} {plan.kernel_for(big)}", flush=True)
    a = K.run(plan, X[:small].contiguous(), y_debug=True)
    b = K.run(plan, X, y_debug=True)
    assert torch.equal(a[0], b[0][:small]) and torch.equal(a[1], b[1][: a[1].shape[0]])
    assert torch.equal(a[2], b[2][:small])


# The column kernel with c holds each thread's c values in registers as fp16 when every
# nonzero |c| lies in fp16's normal range [2^-14, 2^15), and re-reads c (fp32) from L2
# otherwise. Channel scales far below or above that range (all of c times 2^-20, or times
# 2^17) must take the second path: as fp16 they would be subnormal (a few significant bits)
# or infinite. Both paths match the oracle; a c that straddles the edge (one channel at
# 2^15) does too.
@pytest.mark.parametrize("name,T,kernel", [
    ("down_proj_n14336", 301, "fused_mfma_bf16_cols_112x128_c"),
    ("ffn_n11008", 203, "fused_mfma_bf16_cols_86x128_c")])
@pytest.mark.parametrize("cscale", ["in_range", "tiny", "huge", "edge"])
def test_column_kernel_channel_scales_outside_fp16(gpu, name, T, kernel, cscale):
    import torch
    inp = S.make(name, T=T)
    c = inp.c.astype(np.float64)
    if cscale == "tiny":
        c = c * 2.0 ** -20
    elif cscale == "huge":
        c = c * 2.0 ** 17
    elif cscale == "edge":
        c = c.copy()
        c[5] = 2.0 ** 15
    inp.c = c.astype(np.float32)
    plan, X = K.make_plan(inp)
    assert plan.kernel_for(T) == kernel, plan.kernel_for(T)
    codes, scales, y = K.run(plan, X)
    rel = K.check_plan_against_oracle(inp, plan, codes, scales, y)
    assert rel < 1e-3, rel


# Tokens whose two halves of rows would need different fp16 scales of x^ (rows 32-63 times
# 2^20, or rows 0-31 times 2^-30): the stream kernel with c scales by the whole token's
# bound, and the timed and debug launches agree bit for bit and match the oracle.
def test_stream_with_c_uneven_token_halves(gpu):
    import torch
    name, T = "attn_n4096", 1100
    inp = S.make(name, T=T)
    wl = inp.wl
    x = O.bf16_bits_to_f64(inp.X).reshape(T, wl.n1, wl.n2)
    x[0::3, 32:, :] *= 2.0 ** 20
    x[1::3, :32, :] *= 2.0 ** -30
    inp.X = S.to_bf16_bits(x.reshape(T, -1))
    plan, X = K.make_plan(inp)
    assert plan.kernel_for(T) == "fused_mfma_bf16_stream_64x64_c", plan.kernel_for(T)
    codes, scales, y = K.run(plan, X)
    K.check_plan_against_oracle(inp, plan, codes, scales, y)
    c2, s2 = K.run(plan, X, y_debug=False)
    assert torch.equal(c2, codes) and torch.equal(s2, scales)
