"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Gate ("FlatQuant: Fast Learnable Affine Quantization" workloads, synthetic): the fp32
transformed tensor Y within rel-L2 2e-3 of the fp64 oracle for bf16 inputs (1e-5 for
fp32), and the INT4 codes and scales bit-exact against the oracle quantizer applied to
the GPU's own Y. Every case also checks that the launch without the debug output (the
configuration the benchmark times) writes the same codes and scales.
"""
import numpy as np
import pytest

import kqtest as K
from kronecker_factored_transforms_amd import synth as S

pytestmark = pytest.mark.gpu


def _run_and_check(inp, plan, X, token_ids=None):
    import torch
    codes, scales, y = K.run(plan, X, y_debug=True)
    codes2, scales2 = K.run(plan, X, y_debug=False)
    assert torch.equal(codes, codes2) and torch.equal(scales, scales2)
    return codes, scales, y


# sizes the oracle finishes in seconds; ragged T spans several workgroups and a tail
SMALL = [
    ("tiny_fp32_n64", 16),
    ("attn_n4096", 2048),
    ("attn_n4096", 333),
    ("hidden_n8192", 1001),
    ("down_proj_n14336", 301),
    ("decode_n8192_t64", 64),
    ("prefill_n8192_t65536", 777),
    ("down_proj_n28672", 203),
    ("ffn_n11008", 301),
    ("hidden_n7168", 333),
    ("ffn_n18432", 277),
]


@pytest.mark.parametrize("name,T", SMALL)
def test_parity_against_full_oracle(gpu, name, T):
    inp = S.make(name, T=T)
    plan, X = K.make_plan(inp)
    print(f"[parity] {name} T={T} kernel={plan.kernel}", flush=True)
    codes, scales, y = _run_and_check(inp, plan, X)
    rel = K.check_against_oracle(inp, codes.cpu().numpy(), K.np_scales(scales), y.cpu().numpy(),
                                 plan.clip)
    print(f"[parity] {name} T={T} rel-L2 {rel:.3e}", flush=True)
    if inp.wl.dtype == "bf16":
        assert plan.kernel.startswith("fused_mfma_bf16")


FULL = ["attn_n4096", "hidden_n8192", "down_proj_n14336", "decode_n8192_t64",
        "prefill_n8192_t65536", "down_proj_n28672", "ffn_n11008", "hidden_n7168", "ffn_n18432"]


@pytest.mark.parametrize("name", FULL)
def test_parity_full_size_sampled_tokens(gpu, name):
    """Full workload size, same launch as the benchmark; the oracle checks a sample of
    tokens one by one (first, last, and random ones)."""
    import torch
    inp = S.make(name)
    plan, X = K.make_plan(inp)
    T = inp.T
    print(f"[parity-full] {name} T={T} kernel={plan.kernel}", flush=True)
    codes, scales, y = _run_and_check(inp, plan, X)
    rng = np.random.default_rng(1234)
    ids = np.unique(np.concatenate([[0, 1, T - 1], rng.choice(T, min(T, 384), replace=False)]))
    idx = torch.from_numpy(ids).to(X.device)
    rel = K.check_against_oracle(inp, codes[idx].cpu().numpy(), K.np_scales(scales[idx]),
                                 y[idx].cpu().numpy(), plan.clip, token_ids=ids)
    print(f"[parity-full] {name} sampled {ids.size} tokens rel-L2 {rel:.3e}", flush=True)
