"""GPU parity of the fp32 path on the matrix cores (fp32 X, P1, P2 carried as bf16 hi/lo
pairs, three MFMA products per product, Z kept in fp32): Y within rel-L2 1e-5 of the fp64
oracle (the fp32 tolerance), codes and steps bit-exact against the oracle quantizer on
the GPU's own Y, and the launch without the debug output writing the same codes."""
from dataclasses import replace

import numpy as np
import pytest

import kqtest as K
from kronecker_factored_transforms_amd import binding as B
from kronecker_factored_transforms_amd import synth as S

pytestmark = pytest.mark.gpu


def _run(inp, plan, X):
    import torch
    codes, scales, y = K.run(plan, X, y_debug=True)
    codes2, scales2 = K.run(plan, X, y_debug=False)
    assert torch.equal(codes, codes2) and torch.equal(scales, scales2)
    return codes, scales, y


@pytest.mark.parametrize("n1", [16, 32, 48, 64])
@pytest.mark.parametrize("T", [1, 203, 3 * 2048 + 77])
def test_fp32_kernel_parity(gpu, n1, T):
    """T = 6221 runs several tokens per wave (next-token DMA and deferred code stores)."""
    wl = replace(S.WORKLOADS["fp32_n4096"], n1=n1)
    inp = S.make(wl, T=T)
    plan, X = K.make_plan(inp)
    assert plan.kernel == f"fused_mfma_f32x3_stream_{n1}x64", plan.kernel
    codes, scales, y = _run(inp, plan, X)
    rel, worst = K.check_all_tokens_chunked(inp, plan, codes, scales, y)
    print(f"[fp32] {n1}x64 T={T} rel-L2 {rel:.3e} worst token {worst:.3e}", flush=True)


@pytest.mark.parametrize("scale_dtype", ["fp16", "fp32"])
def test_fp32_kernel_full_workload_and_strided(gpu, scale_dtype):
    import torch
    inp = S.make("fp32_n4096")
    plan, X = K.make_plan(inp, scale_dtype=scale_dtype)
    codes, scales, y = _run(inp, plan, X)
    K.check_all_tokens_chunked(inp, plan, codes, scales, y)
    T, n = X.shape
    wide = torch.zeros((T, n + 32), dtype=torch.float32, device=gpu)
    wide[:, 16:16 + n] = X
    c2, s2 = plan(wide[:, 16:16 + n])
    assert torch.equal(c2, codes) and torch.equal(s2, scales)


def test_fp32_edge_cases_and_fallbacks(gpu):
    """Zero tokens and clip 0 on the fp32 kernel; fp32 with a per-channel scale, and fp32
    shapes beyond its n2 = 64 tiles, run the generic fp32 kernel."""
    import math
    import torch
    wl = replace(S.WORKLOADS["fp32_n4096"], alpha=-math.inf)
    inp = S.make(wl, T=77)
    X0 = inp.X.copy()
    X0[[0, 40]] = 0
    inp.X = X0
    plan, X = K.make_plan(inp)
    codes, scales, y = _run(inp, plan, X)
    K.check_plan_against_oracle(inp, plan, codes, scales, y)
    assert np.all(K.np_scales(scales) == 0) and np.all(codes.cpu().numpy() == 0)
    inp = S.make("fp32_n4096", T=40)
    c = torch.from_numpy(np.linspace(0.5, 2.0, 4096).astype(np.float32)).to(gpu)
    plan, X = K.make_plan(inp, c=c)
    assert plan.kernel == "generic_fp32_fma"
    for n1, n2 in [(32, 128), (8, 8)]:
        inp = S.make(replace(S.WORKLOADS["fp32_n4096"], n1=n1, n2=n2), T=21)
        plan, X = K.make_plan(inp)
        assert plan.kernel == "generic_fp32_fma", plan.kernel
        codes, scales, y = _run(inp, plan, X)
        K.check_plan_against_oracle(inp, plan, codes, scales, y)
