"""The entry point for callers that cannot allocate (kq_transform_quant_noalloc): its
workspace is the library's per-GPU scratch array. Through the C ABI, it must write the
same codes, steps and Y as kq_transform_quant_ws with a caller workspace, on two calls in
a row (the second smaller, so stale scratch contents from the first are present), for
both two-kernel designs; a single-kernel plan needs no scratch at any size, and a call
needing more scratch than the library holds is refused before anything is enqueued."""
from dataclasses import replace

import pytest

import kqtest as K
from kronecker_factored_transforms_amd import binding as B
from kronecker_factored_transforms_amd import synth as S

pytestmark = pytest.mark.gpu


def _outputs(torch, plan, T, dev):
    return (torch.full((T, plan.n // 2), 0xA5, dtype=torch.uint8, device=dev),
            torch.full((T,), 7.0, dtype=plan.scale_dtype, device=dev),
            torch.full((T, plan.n), float("nan"), dtype=torch.float32, device=dev))


@pytest.mark.parametrize("n1,n2,with_c,flags", [
    (160, 160, True, B.KQ_FLAG_SPLIT_TWOSTAGE), (168, 176, False, B.KQ_FLAG_SPLIT_PTILE),
    (256, 256, False, 0)])
def test_noalloc_matches_workspace_entry_point(gpu, n1, n2, with_c, flags):
    import torch
    base = S.WORKLOADS["down_proj_n14336"] if with_c else S.WORKLOADS["hidden_n8192"]
    wl = replace(base, n1=n1, n2=n2, n_outliers=4, pivot_channels=0)
    inp = S.make(wl, T=211)
    plan, X = K.make_plan(inp, flags=flags)
    for T in (211, 53):  # the second call is smaller: the scratch holds the first's data
        assert 0 < plan.workspace_bytes(T) <= B.KQ_NOALLOC_SCRATCH_BYTES
        Xt = X[:T]
        c1, s1, y1 = _outputs(torch, plan, T, gpu)
        B.kq_transform_quant_noalloc(plan.handle, Xt, T, Xt.stride(0), c1, s1, y1)
        c1b, s1b, _ = _outputs(torch, plan, T, gpu)
        B.kq_transform_quant_noalloc(plan.handle, Xt, T, Xt.stride(0), c1b, s1b, None)
        ws = torch.empty((plan.workspace_bytes(T),), dtype=torch.uint8, device=gpu)
        c2, s2, y2 = _outputs(torch, plan, T, gpu)
        B.kq_transform_quant_ws(plan.handle, Xt, T, Xt.stride(0), c2, s2, y2, ws, ws.numel())
        torch.cuda.synchronize()
        assert torch.equal(c1, c2) and torch.equal(s1, s2) and torch.equal(y1, y2)
        assert torch.equal(c1b, c2) and torch.equal(s1b, s2)
    sub = S.make(wl, T=53)
    K.check_against_oracle(sub, c1.cpu().numpy(), K.np_scales(s1), y1.cpu().numpy(), plan.clip)


def test_noalloc_limits(gpu):
    import torch
    # a two-kernel plan: a call needing more than the scratch holds is refused
    wl = replace(S.WORKLOADS["hidden_n8192"], n1=256, n2=256, n_outliers=4)
    inp = S.make(wl, T=4)
    plan, X = K.make_plan(inp)
    per_tok = plan.workspace_bytes(1)
    T_big = B.KQ_NOALLOC_SCRATCH_BYTES // per_tok + 1
    assert plan.workspace_bytes(T_big) > B.KQ_NOALLOC_SCRATCH_BYTES
    Xb = torch.zeros((T_big, plan.n), dtype=torch.bfloat16, device=gpu)
    cb = torch.empty((T_big, plan.n // 2), dtype=torch.uint8, device=gpu)
    sb = torch.empty((T_big,), dtype=torch.float16, device=gpu)
    with pytest.raises(B.KqError) as e:
        B.kq_transform_quant_noalloc(plan.handle, Xb, T_big, plan.n, cb, sb)
    assert e.value.status == B.KQ_ERR_WORKSPACE
    # a single-kernel plan needs no scratch at any size
    inp = S.make("hidden_n8192", T=3000)
    plan, X = K.make_plan(inp)
    assert plan.workspace_bytes(3000) == 0
    c1, s1 = torch.empty((3000, 4096), dtype=torch.uint8, device=gpu), torch.empty((3000,), dtype=torch.float16, device=gpu)
    B.kq_transform_quant_noalloc(plan.handle, X, 3000, X.stride(0), c1, s1)
    c2, s2 = plan(X)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(s1, s2)
