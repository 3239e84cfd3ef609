"""GPU parity of the two designs for factors too large for one CU's on-chip memory
("FlatQuant: Fast Learnable Affine Quantization", Deep Dive: The fused kernel, Figure 8(b)
and 8(c); Where It Breaks: on-chip memory overflow): Figure 8(c) passes Z through a
device workspace between a stage-1 and a stage-2 + quantizer kernel, Figure 8(b) applies
P1 one tile of its output dimension at a time and quantizes in a second kernel. Both are
checked against the oracle like every other kernel: Y within the bf16 tolerance of the
fp64 transform, codes and steps bit-exact against the oracle quantizer on the GPU's Y,
and the launch without the debug output writing the same codes."""
from dataclasses import replace

import numpy as np
import pytest

import kqtest as K
from kronecker_factored_transforms_amd import binding as B
from kronecker_factored_transforms_amd import synth as S

pytestmark = pytest.mark.gpu

SPLITS = {"twostage": B.KQ_FLAG_SPLIT_TWOSTAGE, "ptile": B.KQ_FLAG_SPLIT_PTILE}
# (n1, n2, with_c, splits built)
LARGE = [(160, 160, False, "both"), (160, 160, True, "both"), (144, 192, False, "both"),
         (144, 192, True, "both"), (168, 176, False, "both"), (168, 176, True, "both"),
         (208, 256, False, "both"), (208, 256, True, "twostage"), (256, 256, False, "both"),
         (256, 256, True, "twostage"), (128, 160, True, "both"), (128, 192, True, "both"),
         (128, 224, True, "both"), (128, 256, True, "both"), (128, 224, False, "both")]


def _workload(n1, n2, with_c):
    base = S.WORKLOADS["down_proj_n14336"] if with_c else S.WORKLOADS["hidden_n8192"]
    return replace(base, n1=n1, n2=n2, n_outliers=4, pivot_channels=0)


def _run_checked(inp, plan, X):
    import torch
    codes, scales, y = K.run(plan, X, y_debug=True)
    codes2, scales2 = K.run(plan, X, y_debug=False)
    assert torch.equal(codes, codes2) and torch.equal(scales, scales2)
    return codes, scales, y


@pytest.mark.parametrize("n1,n2,with_c,built", LARGE)
@pytest.mark.parametrize("split", ["twostage", "ptile"])
def test_large_factor_parity(gpu, n1, n2, with_c, built, split):
    inp = S.make(_workload(n1, n2, with_c), T=37)
    if built not in ("both", split):
        with pytest.raises(B.KqError) as e:
            K.make_plan(inp, flags=SPLITS[split])
        assert e.value.status == B.KQ_ERR_UNSUPPORTED
        return
    plan, X = K.make_plan(inp, flags=SPLITS[split])
    suffix = "_c" if with_c else ""
    assert plan.kernel == f"{split}_mfma_bf16_{n1}x{n2}{suffix}", plan.kernel
    assert plan.workspace_bytes(37) > 0
    print(f"[large] {plan.kernel} T=37 workspace {plan.workspace_bytes(37)} B", flush=True)
    codes, scales, y = _run_checked(inp, plan, X)
    rel = K.check_against_oracle(inp, codes.cpu().numpy(), K.np_scales(scales), y.cpu().numpy(),
                                 plan.clip)
    print(f"[large] {plan.kernel} rel-L2 {rel:.3e}", flush=True)


# Hidden sizes whose factors (kq_choose_factors: n1 <= n2, n1 + n2 smallest) had no MFMA
# kernel: every one now gets one, never the generic fp32 kernel.
HIDDEN = [(2560, False), (5632, False), (6144, False), (8960, False), (25600, False),
          (27648, False), (28672, True), (29568, False), (53248, False), (65536, False),
          (2560, True), (8960, True), (25600, True), (65536, True)]


@pytest.mark.parametrize("n,with_c", HIDDEN)
def test_every_hidden_size_has_an_mfma_kernel(gpu, n, with_c):
    n1, n2 = B.kq_choose_factors(n)
    inp = S.make(_workload(n1, n2, with_c), T=29)
    plan, X = K.make_plan(inp)
    print(f"[hidden] n={n} -> {n1}x{n2} kernel={plan.kernel}", flush=True)
    assert "mfma" in plan.kernel and "generic" not in plan.kernel
    codes, scales, y = _run_checked(inp, plan, X)
    K.check_against_oracle(inp, codes.cpu().numpy(), K.np_scales(scales), y.cpu().numpy(), plan.clip)


@pytest.mark.parametrize("n1,n2,with_c", [(256, 256, False), (160, 160, True), (144, 192, False)])
@pytest.mark.parametrize("split", ["twostage", "ptile"])
def test_large_factor_many_tokens_per_workgroup_strided(gpu, n1, n2, with_c, split):
    """More tokens than the persistent grids hold (every workgroup of both kernels runs
    several tokens, the next token's loads in flight), every token against the oracle; the
    same codes from a row stride larger than the row."""
    import torch
    T = 611
    inp = S.make(_workload(n1, n2, with_c), T=T)
    plan, X = K.make_plan(inp, flags=SPLITS[split])
    codes, scales, y = _run_checked(inp, plan, X)
    K.check_all_tokens_chunked(inp, plan, codes, scales, y, chunk=256)
    n = n1 * n2
    wide = torch.zeros((T, n + 64), dtype=torch.bfloat16, device=gpu)
    wide[:, 32:32 + n] = X
    c2, s2 = plan(wide[:, 32:32 + n])
    assert torch.equal(c2, codes) and torch.equal(s2, scales)


@pytest.mark.parametrize("split", ["twostage", "ptile"])
def test_large_factor_workspace_errors(gpu, split):
    """The two-kernel designs refuse a call without a workspace, or with one that is too
    small or misaligned, before anything is enqueued; one larger than needed is fine."""
    import torch
    T = 5
    inp = S.make(_workload(160, 160, False), T=T)
    plan, X = K.make_plan(inp, flags=SPLITS[split])
    need = plan.workspace_bytes(T)
    assert need > 0 and plan.workspace_bytes(0) == 0
    codes = torch.empty((T, 160 * 160 // 2), dtype=torch.uint8, device=gpu)
    scales = torch.empty((T,), dtype=torch.float16, device=gpu)
    with pytest.raises(B.KqError) as e:
        B.kq_transform_quant(plan.handle, X, T, X.stride(0), codes, scales)
    assert e.value.status == B.KQ_ERR_WORKSPACE
    ws = torch.empty((need + 512,), dtype=torch.uint8, device=gpu)
    with pytest.raises(B.KqError) as e:
        B.kq_transform_quant_ws(plan.handle, X, T, X.stride(0), codes, scales, None, ws, need - 1)
    assert e.value.status == B.KQ_ERR_WORKSPACE
    with pytest.raises(B.KqError) as e:
        B.kq_transform_quant_ws(plan.handle, X, T, X.stride(0), codes, scales, None,
                                ws.data_ptr() + 16, need)
    assert e.value.status == B.KQ_ERR_ALIGNMENT
    B.kq_transform_quant_ws(plan.handle, X, T, X.stride(0), codes, scales, None, ws, need + 512)
    torch.cuda.synchronize()
    ref_c, ref_s = plan(X)
    assert torch.equal(codes, ref_c) and torch.equal(scales, ref_s)


@pytest.mark.parametrize("case", ["fp32_scales", "clip_zero", "zero_token", "item_scales"])
@pytest.mark.parametrize("split", ["twostage", "ptile"])
def test_large_factor_edge_cases(gpu, case, split):
    """item_scales: within a token, one 32-row block of X is scaled by 2^60 and another by
    2^-60 (exact in bf16), so that Figure 8(c)'s per-item fp16 scale of x c takes both
    signs in one token and is undone on Z; a wrong exponent would be off by 2^120."""
    import math
    wl = _workload(168, 176, True)
    if case == "clip_zero":
        wl = replace(wl, alpha=-math.inf)
    T = 40
    inp = S.make(wl, T=T)
    if case == "zero_token":
        X0 = inp.X.copy()
        X0[[0, 17, T - 1]] = 0
        inp.X = X0
    if case == "item_scales":
        f = S.bf16_bits_to_f32(inp.X).reshape(T, 168, 176).astype(np.float64)
        f[::3, 32:64] *= 2.0 ** 60
        f[1::3, 96:128] *= 2.0 ** -60
        f[2::3, 0:32] *= 2.0 ** 60
        f[2::3, 128:160] *= 2.0 ** -60
        inp.X = S.to_bf16_bits(f.reshape(T, -1))
    # (the 2^60 blocks take steps beyond fp16's range: fp32 steps keep the codes nonzero)
    sd = "fp32" if case in ("fp32_scales", "item_scales") else inp.wl.scale_dtype
    plan, X = K.make_plan(inp, scale_dtype=sd, flags=SPLITS[split])
    codes, scales, y = _run_checked(inp, plan, X)
    K.check_plan_against_oracle(inp, plan, codes, scales, y)
    s = K.np_scales(scales)
    cn = codes.cpu().numpy()
    if case == "clip_zero":
        assert np.all(s == 0) and np.all(cn == 0)
    if case == "zero_token":
        assert np.all(s[[0, 17, T - 1]] == 0) and np.all(cn[[0, 17, T - 1]] == 0)
    if case == "item_scales":
        # (a 2^60 block sets its token's step; the token's other rows then quantize to 0)
        assert np.all(np.isfinite(s)) and np.all(cn.any(axis=1))
        assert np.all(s[0::3] > 1e15) and np.all(s[2::3] > 1e15) and np.all(s[1::3] < 1e3)
