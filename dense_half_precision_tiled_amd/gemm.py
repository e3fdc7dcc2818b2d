"""Python binding of libdhpt_gemm.so (argument marshalling only).

The functions mirror include/gemm.h one to one (``gemm_run``, ``gemm_run_ex``,
``gemm_run_ws``, ``gemm_run_noalloc``, ``gemm_run_splitk``, ``gemm_workspace_size``,
``gemm_splitk_workspace_size``, ``gemm_strerror``,
``gemm_select_instance``, ``gemm_select_instance_ex``,
``gemm_select_instance_ws``, ``gemm_num_instances``, ``gemm_instance_name``,
``gemm_run_instance``, ``gemm_run_instance_ex``, ``gemm_run_instance_ws``,
``gemm_tile_order``) and take raw device pointers as Python ints.  ``gemm(A, B, out_dtype)`` is the
convenience form on torch tensors: it allocates C with ``torch.empty`` and
passes ``data_ptr()``, the strides and the current HIP stream (gemm_run for a
row-major B, gemm_run_ex with GEMM_B_COL_MAJOR for a column-major B).

There is no fallback: if the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdhpt_gemm.so")

GEMM_F16_F32, GEMM_F16_F16, GEMM_BF16_F32, GEMM_BF16_BF16 = 0, 1, 2, 3
GEMM_E4M3_F32, GEMM_E4M3_F16, GEMM_E4M3_BF16 = 4, 5, 6
GEMM_E5M2_F32, GEMM_E5M2_F16, GEMM_E5M2_BF16 = 7, 8, 9
GEMM_OK = 0
GEMM_ERR_DIM, GEMM_ERR_LD, GEMM_ERR_NULL, GEMM_ERR_DTYPE = -1, -2, -3, -4
GEMM_ERR_ALIAS, GEMM_ERR_RANGE, GEMM_ERR_LAUNCH, GEMM_ERR_ALIGN = -5, -6, -7, -8
GEMM_ERR_INSTANCE, GEMM_ERR_LAYOUT, GEMM_ERR_WORKSPACE = -9, -10, -11
GEMM_B_ROW_MAJOR, GEMM_B_COL_MAJOR = 0, 1

EXPORTED = ["gemm_run", "gemm_run_ex", "gemm_strerror", "gemm_select_instance",
            "gemm_select_instance_ex", "gemm_num_instances", "gemm_instance_name",
            "gemm_run_instance", "gemm_run_instance_ex", "gemm_tile_order",
            "gemm_workspace_size", "gemm_run_ws", "gemm_run_instance_ws", "gemm_select_instance_ws",
            "gemm_run_noalloc", "gemm_splitk_workspace_size", "gemm_run_splitk"]

_lib = None


class GemmError(RuntimeError):
    def __init__(self, status: int):
        super().__init__("gemm failed: %d (%s)" % (status, gemm_strerror(status)))
        self.status = status


def load(lib_path: str | None = None) -> ctypes.CDLL:
    """Load the library once (``lib_path``: another build of it, e.g. the
    timeline-recording profiling variant; only the first call's path counts)."""
    global _lib
    if _lib is None:
        path = lib_path or LIB_PATH
        if not os.path.exists(path):
            raise RuntimeError("%s is not built (run __graft_entry__.build() or "
                               "python -m dense_half_precision_tiled_amd.build)" % os.path.basename(path))
        lib = ctypes.CDLL(path)
        i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.gemm_run.argtypes = [i64, i64, i64, i32, vp, i64, vp, i64, vp, i64, vp]
        lib.gemm_run.restype = i32
        lib.gemm_run_instance.argtypes = [i32, i64, i64, i64, i32, vp, i64, vp, i64, vp, i64, vp]
        lib.gemm_run_instance.restype = i32
        f32 = ctypes.c_float
        lib.gemm_run_ex.argtypes = [i64, i64, i64, i32, i32, vp, i64, vp, i64, vp, i64, f32, f32, vp,
                                    i32, vp]
        lib.gemm_run_ex.restype = i32
        lib.gemm_run_instance_ex.argtypes = [i32] + lib.gemm_run_ex.argtypes
        lib.gemm_run_instance_ex.restype = i32
        lib.gemm_select_instance_ex.argtypes = [i64, i64, i64, i32, i32, vp, i64, vp, i64, vp, i64,
                                                f32, f32, vp, i32]
        lib.gemm_select_instance_ex.restype = i32
        lib.gemm_select_instance.argtypes = [i64, i64, i64, i32, vp, i64, vp, i64, vp, i64]
        lib.gemm_select_instance.restype = i32
        lib.gemm_strerror.argtypes = [i32]
        lib.gemm_strerror.restype = ctypes.c_char_p
        lib.gemm_num_instances.argtypes = []
        lib.gemm_num_instances.restype = i32
        lib.gemm_instance_name.argtypes = [i32]
        lib.gemm_instance_name.restype = ctypes.c_char_p
        lib.gemm_tile_order.argtypes = [i32, i64, i64, ctypes.POINTER(ctypes.c_int32),
                                        ctypes.POINTER(ctypes.c_int32), i64]
        lib.gemm_tile_order.restype = i64
        lib.gemm_workspace_size.argtypes = []
        lib.gemm_workspace_size.restype = i64
        lib.gemm_run_ws.argtypes = lib.gemm_run_ex.argtypes[:-1] + [vp, i64, vp]
        lib.gemm_run_ws.restype = i32
        lib.gemm_run_instance_ws.argtypes = [i32] + lib.gemm_run_ws.argtypes
        lib.gemm_run_instance_ws.restype = i32
        lib.gemm_select_instance_ws.argtypes = lib.gemm_select_instance_ex.argtypes + [vp, i64]
        lib.gemm_select_instance_ws.restype = i32
        lib.gemm_run_noalloc.argtypes = lib.gemm_run_ex.argtypes
        lib.gemm_run_noalloc.restype = i32
        lib.gemm_splitk_workspace_size.argtypes = [i64, i64, i64, i32]
        lib.gemm_splitk_workspace_size.restype = i64
        lib.gemm_run_splitk.argtypes = lib.gemm_run_ex.argtypes[:-1] + [i32, vp, i64, vp]
        lib.gemm_run_splitk.restype = i32
        _lib = lib
    return _lib


def gemm_run(M, N, K, dtype, A, lda, B, ldb, C, ldc, stream=None) -> int:
    return load().gemm_run(M, N, K, dtype, A, lda, B, ldb, C, ldc, stream)


def gemm_run_instance(instance, M, N, K, dtype, A, lda, B, ldb, C, ldc, stream=None) -> int:
    return load().gemm_run_instance(instance, M, N, K, dtype, A, lda, B, ldb, C, ldc, stream)


def gemm_select_instance(M, N, K, dtype, A, lda, B, ldb, C, ldc) -> int:
    return load().gemm_select_instance(M, N, K, dtype, A, lda, B, ldb, C, ldc)


def gemm_run_ex(M, N, K, dtype, b_layout, A, lda, B, ldb, C, ldc, alpha=1.0, beta=0.0, bias=None,
                relu=0, stream=None) -> int:
    return load().gemm_run_ex(M, N, K, dtype, b_layout, A, lda, B, ldb, C, ldc, alpha, beta, bias,
                              relu, stream)


def gemm_run_instance_ex(instance, M, N, K, dtype, b_layout, A, lda, B, ldb, C, ldc, alpha=1.0,
                         beta=0.0, bias=None, relu=0, stream=None) -> int:
    return load().gemm_run_instance_ex(instance, M, N, K, dtype, b_layout, A, lda, B, ldb, C, ldc,
                                       alpha, beta, bias, relu, stream)


def gemm_select_instance_ex(M, N, K, dtype, b_layout, A, lda, B, ldb, C, ldc, alpha=1.0, beta=0.0,
                            bias=None, relu=0) -> int:
    return load().gemm_select_instance_ex(M, N, K, dtype, b_layout, A, lda, B, ldb, C, ldc, alpha,
                                          beta, bias, relu)


def gemm_workspace_size() -> int:
    return load().gemm_workspace_size()


def gemm_run_ws(M, N, K, dtype, b_layout, A, lda, B, ldb, C, ldc, alpha, beta, bias, relu, workspace,
                workspace_bytes, stream=None) -> int:
    return load().gemm_run_ws(M, N, K, dtype, b_layout, A, lda, B, ldb, C, ldc, alpha, beta, bias, relu,
                              workspace, workspace_bytes, stream)


def gemm_run_instance_ws(instance, M, N, K, dtype, b_layout, A, lda, B, ldb, C, ldc, alpha, beta, bias,
                         relu, workspace, workspace_bytes, stream=None) -> int:
    return load().gemm_run_instance_ws(instance, M, N, K, dtype, b_layout, A, lda, B, ldb, C, ldc, alpha,
                                       beta, bias, relu, workspace, workspace_bytes, stream)


def gemm_select_instance_ws(M, N, K, dtype, b_layout, A, lda, B, ldb, C, ldc, alpha, beta, bias, relu,
                            workspace, workspace_bytes) -> int:
    return load().gemm_select_instance_ws(M, N, K, dtype, b_layout, A, lda, B, ldb, C, ldc, alpha, beta,
                                          bias, relu, workspace, workspace_bytes)


def gemm_run_noalloc(M, N, K, dtype, b_layout, A, lda, B, ldb, C, ldc, alpha=1.0, beta=0.0, bias=None,
                     relu=0, stream=None) -> int:
    return load().gemm_run_noalloc(M, N, K, dtype, b_layout, A, lda, B, ldb, C, ldc, alpha, beta, bias, relu,
                                   stream)


def gemm_splitk_workspace_size(M, N, K, splits) -> int:
    return load().gemm_splitk_workspace_size(M, N, K, splits)


def gemm_run_splitk(M, N, K, dtype, b_layout, A, lda, B, ldb, C, ldc, alpha, beta, bias, relu, splits,
                    workspace, workspace_bytes, stream=None) -> int:
    return load().gemm_run_splitk(M, N, K, dtype, b_layout, A, lda, B, ldb, C, ldc, alpha, beta, bias, relu,
                                  splits, workspace, workspace_bytes, stream)


def gemm_strerror(status: int) -> str:
    return load().gemm_strerror(status).decode()


def gemm_num_instances() -> int:
    return load().gemm_num_instances()


def gemm_instance_name(instance: int) -> str:
    return load().gemm_instance_name(instance).decode()


def gemm_tile_order(instance: int, M: int, N: int):
    """(tm, tn) int32 arrays over the launch's workgroup ids."""
    lib = load()
    T = lib.gemm_tile_order(instance, M, N, None, None, 0)
    if T < 0:
        raise GemmError(int(T))
    tm = np.zeros(T, dtype=np.int32)
    tn = np.zeros(T, dtype=np.int32)
    lib.gemm_tile_order(instance, M, N, tm.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                        tn.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), T)
    return tm, tn


# ------------------------------------------------------------------ torch form
def _dtype_code(in_dtype, out_dtype) -> int:
    import torch
    table = {(torch.float16, torch.float32): GEMM_F16_F32,
             (torch.float16, torch.float16): GEMM_F16_F16,
             (torch.bfloat16, torch.float32): GEMM_BF16_F32,
             (torch.bfloat16, torch.bfloat16): GEMM_BF16_BF16,
             (torch.float8_e4m3fn, torch.float32): GEMM_E4M3_F32,
             (torch.float8_e4m3fn, torch.float16): GEMM_E4M3_F16,
             (torch.float8_e4m3fn, torch.bfloat16): GEMM_E4M3_BF16,
             (torch.float8_e5m2, torch.float32): GEMM_E5M2_F32,
             (torch.float8_e5m2, torch.float16): GEMM_E5M2_F16,
             (torch.float8_e5m2, torch.bfloat16): GEMM_E5M2_BF16}
    try:
        return table[(in_dtype, out_dtype)]
    except KeyError:
        raise TypeError("unsupported dtype pair %s -> %s" % (in_dtype, out_dtype)) from None


def _row_major_ld(t, name):
    if t.dim() != 2:
        raise ValueError("%s must be 2-D" % name)
    if t.stride(1) != 1 and t.shape[1] > 1:
        raise ValueError("%s must be row-major (unit column stride)" % name)
    return max(t.stride(0), t.shape[1]) if t.shape[0] <= 1 else t.stride(0)


def _is_col_major(t) -> bool:
    return t.dim() == 2 and t.shape[0] > 1 and t.stride(0) == 1 and t.stride(1) >= t.shape[0]


def gemm(A, B, out_dtype=None, out=None, instance: int | None = None, stream=None):
    """C = A @ B on the GPU through gemm_run / gemm_run_ex (or their forced-
    instance forms).

    A: [M, K] row-major CUDA tensor of fp16, bf16, float8_e4m3fn or
    float8_e5m2 (row strides may exceed the row length).  B: [K, N] of the
    same dtype, row-major, or column-major (the transpose of a row-major
    [N, K] tensor, e.g. ``Bt.t()``).
    out_dtype defaults to the input dtype for 16-bit inputs and to bfloat16
    for 8-bit ones.  ``out`` may be a preallocated row-major [M, N] tensor (its
    row stride is ldc).
    """
    import torch
    if A.dtype != B.dtype:
        raise TypeError("A and B must share a dtype")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    in8 = A.dtype in (torch.float8_e4m3fn, torch.float8_e5m2)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or (torch.bfloat16 if in8 else A.dtype), device=A.device)
    elif out_dtype is not None and out.dtype != out_dtype:
        raise TypeError("out has dtype %s" % out.dtype)
    code = _dtype_code(A.dtype, out.dtype)
    lda, ldc = _row_major_ld(A, "A"), _row_major_ld(out, "C")
    col = _is_col_major(B)
    ldb = B.stride(1) if col else _row_major_ld(B, "B")
    if stream is None:
        stream = torch.cuda.current_stream(A.device).cuda_stream
    if col:
        args = (M, N, K, code, GEMM_B_COL_MAJOR, A.data_ptr(), lda, B.data_ptr(), ldb, out.data_ptr(), ldc,
                1.0, 0.0, None, 0, stream)
        st = gemm_run_ex(*args) if instance is None else gemm_run_instance_ex(instance, *args)
    else:
        args = (M, N, K, code, A.data_ptr(), lda, B.data_ptr(), ldb, out.data_ptr(), ldc, stream)
        st = gemm_run(*args) if instance is None else gemm_run_instance(instance, *args)
    if st != GEMM_OK:
        raise GemmError(st)
    return out
