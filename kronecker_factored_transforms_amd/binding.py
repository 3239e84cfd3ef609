"""ctypes binding of libkq: the C ABI of include/kq.h under the same names.

Argument marshalling only: tensors are turned into device pointers, sizes and the HIP
stream handle; every step of the transform and the quantizer runs in the HIP kernels.
There is no CPU fallback: if libkq.so is missing the first call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkq.so")

(KQ_OK, KQ_ERR_INVALID_ARG, KQ_ERR_UNSUPPORTED, KQ_ERR_ALIGNMENT, KQ_ERR_OUT_OF_MEMORY, KQ_ERR_HIP,
 KQ_ERR_WORKSPACE) = range(7)
KQ_BF16, KQ_FP32, KQ_FP16 = 0, 1, 2
KQ_FLAG_FORCE_GENERIC = 0x1
KQ_FLAG_SPLIT_REG1 = 0x10
KQ_FLAG_SPLIT_REG2 = 0x20
KQ_FLAG_SPLIT_COLS = 0x40
KQ_FLAG_SPLIT_DEEP = 0x80
KQ_FLAG_SPLIT_STREAM = 0x100
KQ_FLAG_SPLIT_PAIR = 0x200
KQ_FLAG_PER_ROW = 0x400
KQ_FLAG_INT8 = 0x800
KQ_FLAG_SPLIT_TWOSTAGE = 0x1000
KQ_FLAG_SPLIT_PTILE = 0x2000
KQ_FLAG_SPLIT_RSPLIT = 0x4000

# every symbol declared in include/kq.h
EXPORTS = (
    "kq_choose_factors", "kq_create", "kq_create_ex", "kq_transform_quant", "kq_destroy",
    "kq_plan_clip_ratio", "kq_plan_kernel_name", "kq_plan_kernel_name_for", "kq_status_string",
    "kq_version", "kq_int4_gemm", "kq_workspace_size", "kq_transform_quant_ws",
    "kq_transform_quant_noalloc", "kq_weight_factor",
)
KQ_NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None


class KqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {kq_status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """Load libkq.so (built in-tree by kronecker_factored_transforms_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m kronecker_factored_transforms_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint
    L.kq_choose_factors.argtypes = [i64, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    L.kq_choose_factors.restype = i32
    L.kq_create.argtypes = [ctypes.POINTER(vp), i32, i32, i32, i32, vp, vp, vp, ctypes.c_float, vp]
    L.kq_create.restype = i32
    L.kq_create_ex.argtypes = [ctypes.POINTER(vp), i32, i32, i32, i32, vp, vp, vp, ctypes.c_float, vp, u32]
    L.kq_create_ex.restype = i32
    L.kq_transform_quant.argtypes = [vp, vp, i64, i64, vp, vp, vp, vp]
    L.kq_transform_quant.restype = i32
    L.kq_transform_quant_ws.argtypes = [vp, vp, i64, i64, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.kq_transform_quant_ws.restype = i32
    L.kq_transform_quant_noalloc.argtypes = [vp, vp, i64, i64, vp, vp, vp, vp]
    L.kq_transform_quant_noalloc.restype = i32
    L.kq_workspace_size.argtypes = [vp, i64, ctypes.POINTER(ctypes.c_size_t)]
    L.kq_workspace_size.restype = i32
    L.kq_destroy.argtypes = [vp]
    L.kq_destroy.restype = i32
    L.kq_plan_clip_ratio.argtypes = [vp]
    L.kq_plan_clip_ratio.restype = ctypes.c_float
    L.kq_plan_kernel_name.argtypes = [vp]
    L.kq_plan_kernel_name.restype = ctypes.c_char_p
    L.kq_plan_kernel_name_for.argtypes = [vp, i64]
    L.kq_plan_kernel_name_for.restype = ctypes.c_char_p
    L.kq_status_string.argtypes = [i32]
    L.kq_status_string.restype = ctypes.c_char_p
    L.kq_int4_gemm.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, i64, i32, i32, vp, i64, vp]
    L.kq_int4_gemm.restype = i32
    L.kq_weight_factor.argtypes = [vp, i32, i32, vp, vp]
    L.kq_weight_factor.restype = i32
    L.kq_version.argtypes = []
    L.kq_version.restype = i32
    _lib = L
    return L


# ------------------------------------------------------------------------------------
def _ptr(x) -> int | None:
    """Device pointer of a GPU tensor, an int address, or None. A host tensor is refused:
    its address would reach the kernels as a device address."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not getattr(x, "is_cuda", False):
        raise ValueError("libkq takes device tensors; got one on " + str(getattr(x, "device", "?")))
    return int(x.data_ptr())


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream) or None
    if isinstance(stream, int):
        return stream or None
    return int(stream.cuda_stream) or None


def _dtype_code(d) -> int:
    if isinstance(d, int):
        return d
    s = str(d).replace("torch.", "")
    return {"bf16": KQ_BF16, "bfloat16": KQ_BF16, "fp32": KQ_FP32, "float32": KQ_FP32,
            "fp16": KQ_FP16, "float16": KQ_FP16}[s]


def _check(st: int, what: str):
    if st != KQ_OK:
        raise KqError(st, what)


def kq_status_string(status: int) -> str:
    return lib().kq_status_string(int(status)).decode()


def kq_version() -> int:
    return int(lib().kq_version())


def kq_choose_factors(n: int) -> tuple[int, int]:
    a, b = ctypes.c_int(0), ctypes.c_int(0)
    _check(lib().kq_choose_factors(int(n), ctypes.byref(a), ctypes.byref(b)), "kq_choose_factors")
    return a.value, b.value


def kq_create(n1, n2, x_dtype, scale_dtype, P1, P2, c=None, alpha=math.inf, stream=None, flags=0):
    """Returns an opaque plan handle (int). P1, P2, c are device tensors (or addresses)."""
    h = ctypes.c_void_p(0)
    st = lib().kq_create_ex(ctypes.byref(h), int(n1), int(n2), _dtype_code(x_dtype),
                            _dtype_code(scale_dtype), _ptr(P1), _ptr(P2), _ptr(c),
                            ctypes.c_float(alpha), _stream(stream), int(flags))
    _check(st, "kq_create")
    return h.value


def kq_transform_quant(plan, X, T, ldx, codes, scales, y_debug=None, stream=None) -> None:
    st = lib().kq_transform_quant(plan, _ptr(X), int(T), int(ldx), _ptr(codes), _ptr(scales),
                                  _ptr(y_debug), _stream(stream))
    _check(st, "kq_transform_quant")


def kq_transform_quant_ws(plan, X, T, ldx, codes, scales, y_debug, workspace, workspace_bytes,
                          stream=None) -> None:
    st = lib().kq_transform_quant_ws(plan, _ptr(X), int(T), int(ldx), _ptr(codes), _ptr(scales),
                                     _ptr(y_debug), _ptr(workspace), int(workspace_bytes),
                                     _stream(stream))
    _check(st, "kq_transform_quant_ws")


def kq_transform_quant_noalloc(plan, X, T, ldx, codes, scales, y_debug=None, stream=None) -> None:
    st = lib().kq_transform_quant_noalloc(plan, _ptr(X), int(T), int(ldx), _ptr(codes),
                                          _ptr(scales), _ptr(y_debug), _stream(stream))
    _check(st, "kq_transform_quant_noalloc")


def kq_workspace_size(plan, T: int) -> int:
    b = ctypes.c_size_t(0)
    _check(lib().kq_workspace_size(plan, int(T), ctypes.byref(b)), "kq_workspace_size")
    return int(b.value)


def kq_destroy(plan) -> None:
    _check(lib().kq_destroy(plan), "kq_destroy")


def kq_plan_clip_ratio(plan) -> float:
    return float(lib().kq_plan_clip_ratio(plan))


def kq_plan_kernel_name(plan) -> str:
    return lib().kq_plan_kernel_name(plan).decode()


def kq_plan_kernel_name_for(plan, T: int) -> str:
    return lib().kq_plan_kernel_name_for(plan, int(T)).decode()


def kq_int4_gemm(xq, ldxq, sx, T, wq, ldwq, sw, N, K, scale_dtype, out_dtype, out, ldo,
                 stream=None) -> None:
    st = lib().kq_int4_gemm(_ptr(xq), int(ldxq), _ptr(sx), int(T), _ptr(wq), int(ldwq), _ptr(sw),
                            int(N), int(K), _dtype_code(scale_dtype), _dtype_code(out_dtype),
                            _ptr(out), int(ldo), _stream(stream))
    _check(st, "kq_int4_gemm")


def kq_weight_factor(P, m, dtype, out, stream=None) -> None:
    _check(lib().kq_weight_factor(_ptr(P), int(m), _dtype_code(dtype), _ptr(out), _stream(stream)),
           "kq_weight_factor")


def weight_factor(P, out=None, stream=None):
    """(P^-1)^T of a square bf16 or fp32 factor on the GPU: the factor that the weight rows of
    a W4A4 layer are transformed with (see kq_weight_factor in include/kq.h)."""
    import torch
    if P.dim() != 2 or P.shape[0] != P.shape[1] or not P.is_contiguous():
        raise ValueError("P must be a contiguous square matrix")
    if P.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("P must be bf16 or fp32")
    if out is None:
        out = torch.empty_like(P)
    elif out.shape != P.shape or out.dtype != P.dtype or not out.is_contiguous() or out.device != P.device:
        raise ValueError("out must be a contiguous tensor of P's shape, dtype and device")
    kq_weight_factor(P, P.shape[0], P.dtype, out, stream)
    return out


def int4_gemm(xq, sx, wq, sw, out_dtype="fp32", out=None, stream=None):
    """Tensor convenience wrapper of kq_int4_gemm: xq [T, K/2] uint8 codes with sx [T],
    wq [N, K/2] with sw [N] (same scale dtype) -> out [T, N] (allocated with torch)."""
    import torch
    T, N, K = int(xq.shape[0]), int(wq.shape[0]), int(xq.shape[1]) * 2
    if int(wq.shape[1]) * 2 != K or sx.dtype != sw.dtype:
        raise ValueError("xq/wq widths or scale dtypes differ")
    odt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[out_dtype]
    if out is None:
        out = torch.empty((T, N), dtype=odt, device=xq.device)
    kq_int4_gemm(xq, xq.stride(0), sx, T, wq, wq.stride(0), sw, N, K, sx.dtype, out_dtype, out,
                 out.stride(0), stream)
    return out


# ------------------------------------------------------------------------------------
class Plan:
    """Convenience wrapper: Plan(P1, P2, c, alpha)(X) -> (codes, scales[, y]).

    X is a [T, n] cuda tensor (bfloat16 or float32, last dim contiguous); P1/P2 have X's
    dtype; c is float32 [n] or None. Outputs are allocated with torch on X's device.
    """

    def __init__(self, P1, P2, c=None, alpha=math.inf, scale_dtype="fp16", stream=None, flags=0,
                 n1=None, bits=4):
        """P1 = None means an identity left factor of size n1 (given) and one step per row
        of V (KQ_FLAG_PER_ROW): scales then have shape [T, n1]."""
        import torch
        if bits not in (4, 8):
            raise ValueError("bits must be 4 or 8")
        if bits == 8:
            flags |= KQ_FLAG_INT8
        self.bits = bits
        if P1 is None:
            if n1 is None:
                raise ValueError("n1 is required with an identity left factor (P1=None)")
            flags |= KQ_FLAG_PER_ROW
        elif P1.dtype != P2.dtype:
            raise TypeError("P1 and P2 must have the same dtype")
        if P2.dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("factors must be bfloat16 or float32")
        if not P2.is_cuda or (P1 is not None and not P1.is_cuda) or (c is not None and not c.is_cuda):
            raise ValueError("factors must live on the GPU")
        P1 = None if P1 is None else P1.contiguous()
        P2 = P2.contiguous()
        if c is not None:
            if c.dtype != torch.float32:
                raise TypeError("c must be float32")
            c = c.contiguous()
        self.per_row = P1 is None
        self.n1, self.n2 = (int(n1) if P1 is None else int(P1.shape[0])), int(P2.shape[0])
        self.n = self.n1 * self.n2
        self.x_dtype = P2.dtype
        self.scale_dtype = torch.float16 if _dtype_code(scale_dtype) == KQ_FP16 else torch.float32
        self.handle = kq_create(self.n1, self.n2, P2.dtype, self.scale_dtype, P1, P2, c, alpha,
                                stream, flags)
        self.clip = kq_plan_clip_ratio(self.handle)
        self.kernel = kq_plan_kernel_name(self.handle)

    def workspace_bytes(self, T: int) -> int:
        """Device workspace a call of T tokens needs (0 for the single-kernel designs)."""
        return kq_workspace_size(self.handle, T)

    def __call__(self, X, y_debug=False, out=None, stream=None, workspace=None):
        """workspace: a uint8 device tensor of at least workspace_bytes(T) bytes for the
        two-kernel designs; allocated here with torch when not given."""
        import torch
        if X.dtype != self.x_dtype or X.dim() != 2 or X.shape[1] != self.n or X.stride(1) != 1:
            raise ValueError("X must be [T, n] of the plan's dtype with unit column stride")
        T = X.shape[0]
        code_shape = (T, self.n * self.bits // 8)
        scale_shape = (T, self.n1) if self.per_row else (T,)
        if out is None:
            codes = torch.empty(code_shape, dtype=torch.uint8, device=X.device)
            scales = torch.empty(scale_shape, dtype=self.scale_dtype, device=X.device)
        else:
            codes, scales = out
            # the C ABI cannot see buffer sizes: a short buffer here would be written past
            # its end by the kernels
            if (codes.dtype != torch.uint8 or tuple(codes.shape) != code_shape
                    or not codes.is_contiguous() or codes.device != X.device):
                raise ValueError(f"codes must be a contiguous uint8 tensor of shape {code_shape} "
                                 f"on {X.device}")
            if (scales.dtype != self.scale_dtype or tuple(scales.shape) != scale_shape
                    or not scales.is_contiguous() or scales.device != X.device):
                raise ValueError(f"scales must be a contiguous {self.scale_dtype} tensor of shape "
                                 f"{scale_shape} on {X.device}")
        y = torch.empty((T, self.n), dtype=torch.float32, device=X.device) if y_debug else None
        need = self.workspace_bytes(T) if T else 0
        if need and workspace is None:
            workspace = torch.empty((need,), dtype=torch.uint8, device=X.device)
        if workspace is not None and (workspace.dtype != torch.uint8 or workspace.numel() < need
                                      or workspace.device != X.device):
            raise ValueError(f"workspace must be a uint8 tensor of at least {need} bytes on {X.device}")
        kq_transform_quant_ws(self.handle, X, T, X.stride(0) if T else self.n, codes, scales, y,
                              workspace, workspace.numel() if workspace is not None else 0, stream)
        return (codes, scales, y) if y_debug else (codes, scales)

    def kernel_for(self, T: int) -> str:
        """Name of the kernel a call with T tokens runs."""
        return kq_plan_kernel_name_for(self.handle, T)

    def close(self):
        if getattr(self, "handle", None):
            kq_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
