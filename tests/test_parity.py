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
from kronecker_factored_transforms_amd import binding as B
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
def test_parity_full_size_every_token(gpu, name):
    """Full workload size, the benchmark's launch: every token against the oracle (Y within
    the tolerance over the whole tensor, codes and steps bit-exact), a chunk at a time."""
    inp = S.make(name)
    plan, X = K.make_plan(inp)
    T = inp.T
    print(f"[parity-full] {name} T={T} kernel={plan.kernel_for(T)}", flush=True)
    codes, scales, y = _run_and_check(inp, plan, X)
    rel, worst = K.check_all_tokens_chunked(inp, plan, codes, scales, y)
    print(f"[parity-full] {name} all {T} tokens: rel-L2 {rel:.3e}, worst token {worst:.3e}",
          flush=True)


# Enough tokens that every wave of a persistent grid runs several tokens (the next-token
# DMA and the deferred code stores of the loop), with a ragged tail, for each default
# split: the stream kernel, the pair kernel (forced: it is the small-batch split), the
# column kernel and the rows kernel.
LOOP_T = 3 * 2048 + 77
LOOP_CASES = [("hidden_n8192", 0, "fused_mfma_bf16_stream_64x128"),
              ("hidden_n8192", B.KQ_FLAG_SPLIT_PAIR, "fused_mfma_bf16_pair_64x128"),
              ("attn_n4096", 0, "fused_mfma_bf16_stream_64x64_c"),
              ("hidden_n7168", 0, "fused_mfma_bf16_stream_64x112"),
              ("down_proj_n14336", 0, "fused_mfma_bf16_cols_112x128_c")]


@pytest.mark.parametrize("name,flags,kernel", LOOP_CASES)
def test_parity_multi_token_loop_every_token(gpu, name, flags, kernel):
    inp = S.make(name, T=LOOP_T)
    plan, X = K.make_plan(inp, flags=flags)
    assert plan.kernel_for(LOOP_T) == kernel, plan.kernel_for(LOOP_T)
    print(f"[parity-loop] {name} T={LOOP_T} kernel={kernel}", flush=True)
    codes, scales, y = _run_and_check(inp, plan, X)
    rel, worst = K.check_all_tokens_chunked(inp, plan, codes, scales, y)
    print(f"[parity-loop] {name} rel-L2 {rel:.3e}, worst token {worst:.3e}", flush=True)


def test_parity_rows_multi_tile_loop_every_token(gpu):
    """Per-row plan (KV heads): enough rows that every wave cycles through its 4-slot tile
    ring several times."""
    T = 5 * 8192 + 77  # 5129 16-row tiles: about 10 per wave of the persistent grid
    inp = S.make("kv_h8_d128", T=T)
    _, _, P2, _ = K.device_inputs(inp)
    plan = B.Plan(None, P2, None, inp.alpha, inp.wl.scale_dtype, n1=inp.wl.n1)
    X = K.torch_from(inp.X, "bf16").to("cuda:0")
    codes, scales, y = _run_and_check(inp, plan, X)
    K.check_plan_against_oracle(inp, plan, codes, scales, y)
