"""HIP graph capture of the library's entry points.

kq_transform_quant and kq_int4_gemm allocate nothing, copy nothing and never
synchronize, so a call can be captured once and replayed. Each case captures one call on
torch's capture stream, then replays it several times with new inputs copied in eagerly
(and a synchronization) between replays, and checks every replay bit for bit against an
eager call on the same inputs.
"""
import numpy as np
import pytest

import kqtest as K
from kronecker_factored_transforms_amd import binding as B
from kronecker_factored_transforms_amd import synth as S

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _inputs(name, T, n_sets, gpu):
    """n_sets seeded token batches of a workload (different token ranges)."""
    inp = S.make(name, T=T * n_sets)
    X = K.torch_from(inp.X, "bf16").to(gpu)
    return inp, [X[i * T:(i + 1) * T].contiguous() for i in range(n_sets)]


def _capture(fn):
    import torch
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("name,T,per_row,bits", [("hidden_n8192", 300, False, 4),
                                                 ("hidden_n8192", 2000, False, 4),
                                                 ("hidden_n8192", 1500, False, 8),
                                                 ("attn_n4096", 700, False, 4),
                                                 ("kv_h8_d128", 900, True, 4),
                                                 ("kv_h8_d128", 900, True, 8)])
def test_transform_quant_replays(gpu, name, T, per_row, bits):
    import torch
    inp, sets = _inputs(name, T, REPLAYS, gpu)
    Xd, P1, P2, c = K.device_inputs(inp, gpu)
    plan = (B.Plan(None, P2, None, inp.alpha, inp.wl.scale_dtype, n1=inp.wl.n1, bits=bits)
            if per_row else B.Plan(P1, P2, c, inp.alpha, inp.wl.scale_dtype, bits=bits))
    ref = [plan(X) for X in sets]
    torch.cuda.synchronize()

    X_in = torch.empty_like(sets[0])
    X_in.copy_(sets[0])
    codes, scales = plan(X_in)  # output buffers the graph writes
    torch.cuda.synchronize()
    g = _capture(lambda: plan(X_in, out=(codes, scales)))
    for i in range(REPLAYS):
        X_in.copy_(sets[i])           # eager work between replays
        codes.fill_(0xA5)
        scales.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(codes, ref[i][0]), f"replay {i}: codes differ"
        assert torch.equal(scales, ref[i][1]), f"replay {i}: scales differ"


def test_int4_gemm_replays(gpu):
    import torch
    rng = np.random.default_rng(11)
    T, N, Kc = 300, 520, 1024
    dev = gpu

    def batch():
        xq = torch.from_numpy(rng.integers(0, 256, (T, Kc // 2), dtype=np.uint8)).to(dev)
        sx = torch.from_numpy(rng.uniform(0.01, 1, T).astype(np.float32)).to(dev)
        return xq, sx

    wq = torch.from_numpy(rng.integers(0, 256, (N, Kc // 2), dtype=np.uint8)).to(dev)
    sw = torch.from_numpy(rng.uniform(0.01, 1, N).astype(np.float32)).to(dev)
    sets = [batch() for _ in range(REPLAYS)]
    ref = [B.int4_gemm(xq, sx, wq, sw, "bf16") for xq, sx in sets]
    torch.cuda.synchronize()

    xq_in, sx_in = sets[0][0].clone(), sets[0][1].clone()
    out = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    g = _capture(lambda: B.int4_gemm(xq_in, sx_in, wq, sw, "bf16", out=out))
    for i in range(REPLAYS):
        xq_in.copy_(sets[i][0])
        sx_in.copy_(sets[i][1])
        out.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[i]), f"replay {i}: outputs differ"
