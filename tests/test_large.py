"""Inputs larger than 4 GiB, for every kernel: token, code and scale offsets must be
computed in 64 bits (a 32-bit byte or element offset wraps long before this size).

Each case draws BLOCK seeded tokens, checks their outputs against the oracle, then builds
on the GPU an input of more than 4.25 GiB made of R copies of the block followed by its
first TAIL tokens, optionally with a row stride larger than the row. Tokens are
independent, so token t of the large call must give exactly the codes and steps of token
t mod BLOCK of the small call: a property that holds at any size, so the oracle never
has to see the large input."""
from dataclasses import replace

import pytest

import kqtest as K
from kronecker_factored_transforms_amd import binding as B
from kronecker_factored_transforms_amd import synth as S

pytestmark = pytest.mark.gpu

BLOCK = 1024
TAIL = 77
MIN_BYTES = 17 * 2 ** 28  # 4.25 GiB of input rows

W = S.WORKLOADS
CASES = {
    # name: (workload, split flags, bits, per-row, extra elements per row)
    "stream": (W["hidden_n8192"], 0, 4, False, 0),
    "stream_strided": (W["hidden_n8192"], 0, 4, False, 64),
    "reg1": (W["hidden_n8192"], B.KQ_FLAG_SPLIT_REG1, 4, False, 64),
    "reg2": (W["hidden_n8192"], B.KQ_FLAG_SPLIT_REG2, 4, False, 64),
    "deep": (W["hidden_n8192"], B.KQ_FLAG_SPLIT_DEEP, 4, False, 64),
    "cols": (W["hidden_n8192"], B.KQ_FLAG_SPLIT_COLS, 4, False, 64),
    "pair": (W["hidden_n8192"], B.KQ_FLAG_SPLIT_PAIR, 4, False, 64),
    "stream_int8": (W["hidden_n8192"], 0, 8, False, 0),
    "stream_c_64x64": (W["attn_n4096"], 0, 4, False, 0),
    "cols_c_112x128": (W["down_proj_n14336"], 0, 4, False, 0),
    "cols_c_86x128": (W["ffn_n11008"], 0, 4, False, 64),
    "cols_128x224": (W["down_proj_n28672"], 0, 4, False, 0),
    "stream_64x112_padded_n2": (W["hidden_n7168"], 0, 4, False, 64),
    "cols_64x112_padded_n2": (W["hidden_n7168"], B.KQ_FLAG_SPLIT_COLS, 4, False, 0),
    "cols_128x144_padded_n2": (W["ffn_n18432"], 0, 4, False, 0),
    "cols_c_112x128_int8": (W["down_proj_n14336"], 0, 8, False, 64),
    "cols_128x224_int8": (W["down_proj_n28672"], 0, 8, False, 0),
    "cols_128x256": (replace(W["down_proj_n28672"], n2=256), 0, 4, False, 64),
    "rows": (W["kv_h8_d128"], 0, 4, True, 0),
    "rows_strided": (W["kv_h8_d128"], 0, 4, True, 64),
    "rows_int8": (W["kv_h8_d128"], 0, 8, True, 0),
    "generic_fp32": (replace(W["tiny_fp32_n64"], n1=64, n2=64), B.KQ_FLAG_FORCE_GENERIC, 4, False, 0),
    "f32x3_64x64": (replace(W["tiny_fp32_n64"], n1=64, n2=64), 0, 4, False, 64),
}


def _plan(inp, flags, bits, per_row):
    X, P1, P2, c = K.device_inputs(inp)
    if per_row:
        return B.Plan(None, P2, None, inp.alpha, inp.wl.scale_dtype, n1=inp.wl.n1, bits=bits), X
    return B.Plan(P1, P2, c, inp.alpha, inp.wl.scale_dtype, flags=flags, bits=bits), X


def _tiled(X, pad):
    """R copies of X then its first TAIL rows, as a [T, n] view of rows n + pad long."""
    import torch
    T0, n = X.shape
    R = -(-MIN_BYTES // (T0 * (n + pad) * X.element_size()))
    buf = torch.empty((R * T0 + TAIL, n + pad), dtype=X.dtype, device=X.device)
    Xb = buf[:, :n]
    Xb[:R * T0].unflatten(0, (R, T0)).copy_(X.unsqueeze(0).expand(R, T0, n))
    Xb[R * T0:].copy_(X[:TAIL])
    return Xb, R


def _same_as_block(big, small, R):
    import torch
    T0 = small.shape[0]
    head = big[:R * T0].unflatten(0, (R, T0))
    assert torch.equal(head, small.unsqueeze(0).expand_as(head))
    assert torch.equal(big[R * T0:], small[:TAIL])


@pytest.mark.parametrize("case", sorted(CASES))
def test_inputs_past_4_gib(gpu, case):
    import torch
    wl, flags, bits, per_row, pad = CASES[case]
    inp = S.make(wl, T=BLOCK)
    plan, X = _plan(inp, flags, bits, per_row)
    codes, scales, y = K.run(plan, X, y_debug=True)
    K.check_plan_against_oracle(inp, plan, codes, scales, y)
    del y
    Xb, R = _tiled(X, pad)
    assert Xb.shape[0] * Xb.stride(0) * Xb.element_size() > 2 ** 32
    print(f"[large] {case}: kernel {plan.kernel_for(Xb.shape[0])}, T = {Xb.shape[0]}, "
          f"ldx = {Xb.stride(0)}", flush=True)
    cb, sb = K.run(plan, Xb, y_debug=False)
    _same_as_block(cb, codes, R)
    _same_as_block(sb, scales, R)
    del Xb, cb, sb
    torch.cuda.empty_cache()
