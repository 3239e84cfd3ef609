"""Every fused work split (one or two waves per token with the token in registers, the
column kernel with the token in LDS, the DMA-fed stream and pair kernels, the row split
with c) against the oracle, on shapes around the workloads:
square and non-square factors, with and without the per-channel scale, ragged T."""
from dataclasses import replace

import pytest

import kqtest as K
from kronecker_factored_transforms_amd import binding as B
from kronecker_factored_transforms_amd import synth as S

pytestmark = pytest.mark.gpu

SPLITS = {"reg1": B.KQ_FLAG_SPLIT_REG1, "reg2": B.KQ_FLAG_SPLIT_REG2, "cols": B.KQ_FLAG_SPLIT_COLS,
          "deep": B.KQ_FLAG_SPLIT_DEEP, "stream": B.KQ_FLAG_SPLIT_STREAM,
          "pair": B.KQ_FLAG_SPLIT_PAIR, "rsplit": B.KQ_FLAG_SPLIT_RSPLIT}
DEEP_SHAPES = {(64, 128, False), (64, 64, False), (64, 64, True)}
SHAPES = [(64, 128, False), (64, 128, True), (64, 64, False), (64, 64, True), (32, 128, False),
          (32, 64, True), (48, 64, True),
          (48, 128, True), (16, 64, True), (48, 64, False), (32, 32, True), (16, 32, False),
          (112, 128, False), (112, 128, True), (96, 128, False), (128, 128, True), (80, 128, False),
          (128, 160, False), (128, 224, False), (128, 256, False), (128, 224, True),
          (86, 128, False), (86, 128, True), (108, 128, False), (108, 128, True),
          (32, 48, False), (32, 48, True), (64, 80, False), (64, 80, True), (64, 112, False),
          (64, 112, True), (128, 144, False), (56, 64, False), (56, 64, True), (64, 104, False),
          (64, 104, True), (40, 64, False), (40, 64, True), (64, 88, False), (64, 88, True),
          (64, 96, False), (64, 96, True), (80, 112, False), (80, 112, True)]


def _available(n1, n2, split, with_c=False):
    if n2 > 128:  # only the column kernel, without c (P2 operands read from L2)
        return split == "cols" and not with_c
    if n1 % 16:  # n1 padded to whole row tiles: only the column kernel
        return split == "cols"
    if n2 % 32:  # n2 padded to a multiple of 32: the column kernel, and 64 x 112 rows in
        # the stream kernel's 128-column layout
        return split == "cols" or (split == "stream" and (n1, n2, with_c) == (64, 112, False))
    if n2 not in (32, 64, 128):  # e.g. 64 x 96: only the column kernel
        return split == "cols"
    if split == "rsplit":
        return with_c and n2 == 64
    if split == "deep":
        return (n1, n2, with_c) in DEEP_SHAPES
    if split == "stream":
        return n1 <= 64 and n2 >= 64 and (not with_c or n2 == 64)
    if split == "pair":
        return n1 <= 64 and n2 >= 64 and not with_c
    if split == "reg1":
        return n1 <= 64
    if split == "reg2":
        return n1 <= 64 and n2 >= 64
    return True


@pytest.mark.parametrize("n1,n2,with_c", SHAPES)
@pytest.mark.parametrize("split", sorted(SPLITS))
def test_split_parity(gpu, n1, n2, with_c, split):
    base = S.WORKLOADS["attn_n4096"] if with_c else S.WORKLOADS["hidden_n8192"]
    wl = replace(base, n1=n1, n2=n2, n_outliers=4, pivot_channels=0)
    inp = S.make(wl, T=203)
    if not _available(n1, n2, split, with_c):
        with pytest.raises(B.KqError) as e:
            K.make_plan(inp, flags=SPLITS[split])
        assert e.value.status == B.KQ_ERR_UNSUPPORTED
        return
    plan, X = K.make_plan(inp, flags=SPLITS[split])
    assert plan.kernel.startswith(f"fused_mfma_bf16_{split}_"), plan.kernel
    codes, scales, y = K.run(plan, X)
    codes2, scales2 = K.run(plan, X, y_debug=False)
    import torch
    assert torch.equal(codes, codes2) and torch.equal(scales, scales2)
    K.check_against_oracle(inp, codes.cpu().numpy(), K.np_scales(scales), y.cpu().numpy(), plan.clip)


@pytest.mark.parametrize("n2", [160, 224, 256])
def test_cols_large_n2_several_tokens_per_workgroup_strided(gpu, n2):
    """More tokens than workgroups, so each workgroup loads its next tile while it computes
    one (by DMA into a second LDS buffer for n2 <= 224), with a row stride larger than the
    row; the same codes as the contiguous call, and the oracle's."""
    import torch
    wl = replace(S.WORKLOADS["hidden_n8192"], n1=128, n2=n2, n_outliers=4, pivot_channels=0)
    T = 3 * 256 + 77
    inp = S.make(wl, T=T)
    plan, X = K.make_plan(inp)
    assert plan.kernel == f"fused_mfma_bf16_cols_128x{n2}", plan.kernel
    n = inp.wl.n
    wide = torch.zeros((T, n + 64), dtype=torch.bfloat16, device=gpu)
    wide[:, 32:32 + n] = X
    Xs = wide[:, 32:32 + n]
    assert Xs.stride(0) == n + 64
    codes, scales, y = K.run(plan, Xs)
    c2, s2 = K.run(plan, X, y_debug=False)
    assert torch.equal(codes, c2) and torch.equal(scales, s2)
    K.check_against_oracle(inp, codes.cpu().numpy(), K.np_scales(scales), y.cpu().numpy(), plan.clip)


@pytest.mark.parametrize("n1", [86, 108])
@pytest.mark.parametrize("T", [1, 3, 845])
def test_cols_padded_n1_with_c_strided(gpu, n1, T):
    """n1 not a multiple of 16: zero-padded row tiles, whose rows must neither reach the
    absmax nor be stored, at a single token, a few tokens and several tokens per
    workgroup, with a row stride larger than the row."""
    import torch
    wl = replace(S.WORKLOADS["ffn_n11008"], n1=n1)
    inp = S.make(wl, T=T)
    plan, X = K.make_plan(inp)
    assert plan.kernel == f"fused_mfma_bf16_cols_{n1}x128_c", plan.kernel
    n = inp.wl.n
    wide = torch.zeros((T, n + 64), dtype=torch.bfloat16, device=gpu)
    wide[:, 32:32 + n] = X
    Xs = wide[:, 32:32 + n]
    codes, scales, y = K.run(plan, Xs)
    c2, s2 = K.run(plan, X, y_debug=False)
    assert torch.equal(codes, c2) and torch.equal(scales, s2)
    K.check_against_oracle(inp, codes.cpu().numpy(), K.np_scales(scales), y.cpu().numpy(), plan.clip)


@pytest.mark.parametrize("n1,n2,with_c", [(64, 112, True), (64, 80, False), (128, 144, False),
                                          (64, 104, True), (56, 64, True)])
def test_cols_padded_n2_strided(gpu, n1, n2, with_c):
    """n2 an odd multiple of 16: zero-padded columns of the tile (in LDS, or filled by the
    tile DMA for n2 > 128) and of P2, whose columns of Y must neither reach the absmax nor
    be stored; several tokens per workgroup and a row stride larger than the row."""
    import torch
    base = S.WORKLOADS["down_proj_n14336"] if with_c else S.WORKLOADS["hidden_n8192"]
    wl = replace(base, n1=n1, n2=n2, n_outliers=4, pivot_channels=0)
    T = 3 * 256 + 77
    inp = S.make(wl, T=T)
    plan, X = K.make_plan(inp)
    assert plan.kernel == f"fused_mfma_bf16_cols_{n1}x{n2}{'_c' if with_c else ''}", plan.kernel
    n = inp.wl.n
    wide = torch.zeros((T, n + 64), dtype=torch.bfloat16, device=gpu)
    wide[:, 32:32 + n] = X
    codes, scales, y = K.run(plan, wide[:, 32:32 + n])
    c2, s2 = K.run(plan, X, y_debug=False)
    assert torch.equal(codes, c2) and torch.equal(scales, s2)
    K.check_against_oracle(inp, codes.cpu().numpy(), K.np_scales(scales), y.cpu().numpy(), plan.clip)


@pytest.mark.gpu
def test_stream_rows_of_112_values():
    """hidden 7168 = 64 x 112 runs on the stream kernel in its 128-column layout: the tile
    DMA fetches 14 real pieces per row (the 2 padding pieces re-read the first one and meet
    P2's zero rows), the codes of the padded columns are not stored. Several tokens per
    wave, a row stride larger than the row, and identity with the column kernel."""
    import torch
    gpu = "cuda:0"
    inp = S.make("hidden_n7168", T=5000)
    plan, X = K.make_plan(inp)
    assert plan.kernel == "fused_mfma_bf16_stream_64x112" and plan.kernel_for(5000) == plan.kernel
    assert plan.kernel_for(64) == "fused_mfma_bf16_cols_64x112"  # small batches
    n = inp.wl.n
    wide = torch.zeros((5000, n + 64), dtype=torch.bfloat16, device=gpu)
    wide[:, 32:32 + n] = X
    codes, scales, y = K.run(plan, wide[:, 32:32 + n])
    c2, s2 = K.run(plan, X, y_debug=False)
    assert torch.equal(codes, c2) and torch.equal(scales, s2)
    K.check_against_oracle(inp, codes.cpu().numpy(), K.np_scales(scales), y.cpu().numpy(), plan.clip)
    cols, _ = K.make_plan(inp, flags=B.KQ_FLAG_SPLIT_COLS)
    c3, s3 = K.run(cols, X, y_debug=False)
    assert torch.equal(codes, c3) and torch.equal(scales, s3)
