"""Fused Kronecker-factored activation transform + per-token INT4 quantization for
AMD Instinct MI355X (gfx950): a C-ABI HIP library (libkq) and its Python binding."""
from .binding import (  # noqa: F401
    KQ_BF16, KQ_FP16, KQ_FP32, KQ_FLAG_FORCE_GENERIC, KQ_FLAG_SPLIT_COLS,
    KQ_FLAG_SPLIT_REG1, KQ_FLAG_SPLIT_REG2, KqError, Plan, kq_choose_factors,
    kq_create, kq_destroy, kq_plan_clip_ratio, kq_plan_kernel_name, kq_status_string,
    kq_transform_quant, kq_version,
)
