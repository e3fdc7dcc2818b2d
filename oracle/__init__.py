"""TEST INFRASTRUCTURE ONLY: the CPU fp64 oracle for C = A.B.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never imports, links or
calls it, and this package imports nothing from the GPU library.

The arithmetic lives in ``oracle.c`` (plain C, built with gcc into
``liboracle.so`` next to this file).  This module is argument marshalling plus
the comparison rule that decides parity:

* ``gemm_f64`` / ``gemm_rows_f64``: C[i][j] = sum_k A[i][k]*B[k][j] in fp64, k
  ascending, on exactly decoded fp16/bf16 inputs (the "arithmetic correctness
  reference" of "GEMM From Naive CUDA to Tensor Cores", section "The
  two-reference testing protocol"), or on 8-bit float inputs in the OCP OFP8
  E4M3 / E5M2 formats (uint8 bit patterns; the 8-bit float the Ada
  tensor-core GEMM write-up leaves untested).
* ``round_to`` / ``ulp``: IEEE round-to-nearest-even to fp32/fp16/bf16 and the
  spacing of those formats (same page, section "What FP32 accumulation
  preserves, and what it can't recover").
* ``bound``: the acceptance bound for a GPU result y against the fp64 result r:
  |y - r| <= K * 2^-20 for fp32 output, and ulp_fmt(r) + K * 2^-20 for fp16 or
  bf16 output.  Bit-exact fixtures instead require y == round_to(fmt, r).
* ``flops``: the 2MNK count (same page, "Compute one output before launching a
  warp": one multiply and one add per inner step).
* ``align_bound8``: the extra error gfx950's 8-bit MFMA adds for 8-bit float
  inputs, for which the pages give no tolerance.  The probe tests pin its
  arithmetic: each group of 8 consecutive k is aligned to the largest of its
  8 products, and every other product of the group keeps only the bits down
  to 13 binades below that largest one (the rest truncated toward zero); the
  incoming accumulator is added at fp32 precision.  So a group loses less
  than 7 * 2^(e - 13), 2^e <= its largest |a*b| <= max|a| * max|b| over the
  group, and the output loses at most 7 * 2^-13 * sum over groups of
  max_g|A[i,k]| * max_g|B[k,j]| -- a matmul of the group maxima.  The 8-bit
  bound is bound() plus this term (``compare(..., extra=...)``).
  PARITY UNPINNED: the group size and the 13 kept binades are device-derived
  (probes of the GPU under test); neither the pages nor the 8-bit float
  specification fixes them, and the CPU pin checks the formula only against
  an emulation of that same model.  It is the envelope for 8-bit results on
  random data and nothing more; the sharp 8-bit checks are the exact
  0.25-grid fixtures (every product a multiple of 1/16 no larger than 4, so
  the 13-binade cut drops no bit and every partial sum is exact in fp32),
  compared bit for bit up to 8192^3, and random data with magnitudes in
  [0.5, 2] (every product in [2^-2, 2^2] with its lowest bit at 2^-8 or
  above, inside any 13-binade window), held to bound() alone.
* ``gemm_ex_f64`` / ``bound_ex`` / ``compare_ex``: the general form
  act(alpha*A.B + beta*C_old + bias) with B row-major or column-major, for the
  fused-epilogue entry point (alpha/beta: the general GEMM the same page opens
  with; bias + ReLU: the fused epilogue of the Ada tensor-core GEMM write-up;
  column-major B: that write-up's "TN" layout).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

IN_F16, IN_BF16, IN_E4M3, IN_E5M2 = 0, 1, 2, 3
OUT_F32, OUT_F16, OUT_BF16 = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc into liboracle.so (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC",
                               "-shared", _SRC, "-o", tmp, "-lm", "-lpthread"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        _lib = _declare(ctypes.CDLL(build()))
    return _lib


def _declare(lib):
    """Set the argument and result types of the oracle's exported functions."""
    i64, u16p, f64p, i64p = (ctypes.c_int64, ctypes.c_void_p,
                             ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64))
    lib.oracle_gemm_f64.argtypes = [i64, i64, i64, ctypes.c_int, u16p, i64, u16p, i64,
                                    f64p, i64, ctypes.c_int]
    lib.oracle_gemm_f64.restype = ctypes.c_int
    lib.oracle_gemm_rows_f64.argtypes = [i64, i64p, i64, i64, ctypes.c_int, u16p, i64,
                                         u16p, i64, f64p, i64, ctypes.c_int]
    lib.oracle_gemm_rows_f64.restype = ctypes.c_int
    lib.oracle_gemm_ex_f64.argtypes = [i64, i64p, i64, i64, ctypes.c_int, ctypes.c_int, u16p,
                                       i64, u16p, i64, ctypes.c_double, ctypes.c_double, f64p,
                                       i64, f64p, ctypes.c_int, f64p, i64, ctypes.c_int]
    lib.oracle_gemm_ex_f64.restype = ctypes.c_int
    lib.oracle_round_to_array.argtypes = [ctypes.c_int, f64p, f64p, i64]
    lib.oracle_round_to_array.restype = None
    lib.oracle_ulp_array.argtypes = [ctypes.c_int, f64p, f64p, i64]
    lib.oracle_ulp_array.restype = None
    lib.oracle_decode_array.argtypes = [ctypes.c_int, u16p, f64p, i64]
    lib.oracle_decode_array.restype = None
    lib.oracle_round_to.argtypes = [ctypes.c_int, ctypes.c_double]
    lib.oracle_round_to.restype = ctypes.c_double
    lib.oracle_ulp.argtypes = [ctypes.c_int, ctypes.c_double]
    lib.oracle_ulp.restype = ctypes.c_double
    lib.oracle_decode_f16.argtypes = [ctypes.c_uint16]
    lib.oracle_decode_f16.restype = ctypes.c_double
    lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
    lib.oracle_decode_bf16.restype = ctypes.c_double
    lib.oracle_decode_e4m3.argtypes = [ctypes.c_uint8]
    lib.oracle_decode_e4m3.restype = ctypes.c_double
    lib.oracle_decode_e5m2.argtypes = [ctypes.c_uint8]
    lib.oracle_decode_e5m2.restype = ctypes.c_double
    return lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _vptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _fmt_in(in_fmt) -> int:
    if in_fmt in ("f16", "fp16", "float16", IN_F16):
        return IN_F16
    if in_fmt in ("bf16", "bfloat16", IN_BF16):
        return IN_BF16
    if in_fmt in ("e4m3", IN_E4M3):
        return IN_E4M3
    if in_fmt in ("e5m2", IN_E5M2):
        return IN_E5M2
    raise ValueError("unknown input format %r" % (in_fmt,))


def _bits_dtype(in_fmt):
    """Storage of one input bit pattern: uint8 for the 8-bit formats."""
    return np.uint8 if _fmt_in(in_fmt) in (IN_E4M3, IN_E5M2) else np.uint16


def _fmt_out(out_fmt) -> int:
    if out_fmt in ("f32", "fp32", "float32", OUT_F32):
        return OUT_F32
    if out_fmt in ("f16", "fp16", "float16", OUT_F16):
        return OUT_F16
    if out_fmt in ("bf16", "bfloat16", OUT_BF16):
        return OUT_BF16
    raise ValueError("unknown output format %r" % (out_fmt,))


def _as_bits_2d(x: np.ndarray, in_fmt) -> np.ndarray:
    x = np.asarray(x)
    want = _bits_dtype(in_fmt)
    if x.dtype != want:
        raise TypeError("%s inputs are %s bit patterns, got %s" % (in_fmt, np.dtype(want).name, x.dtype))
    if x.ndim != 2:
        raise ValueError("oracle inputs are 2-D")
    if x.strides[1] != x.itemsize:
        x = np.ascontiguousarray(x)
    return x


def _ld(x: np.ndarray) -> int:
    """Row stride of a 2-D bit array in elements."""
    return x.strides[0] // x.itemsize


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def gemm_f64(A_bits, B_bits, in_fmt, threads: int | None = None) -> np.ndarray:
    """Full C = A.B in fp64 from input bit patterns (row-major, any row stride)."""
    A = _as_bits_2d(A_bits, in_fmt)
    B = _as_bits_2d(B_bits, in_fmt)
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
    C = np.zeros((M, N), dtype=np.float64)
    rc = _load().oracle_gemm_f64(M, N, K, _fmt_in(in_fmt), _vptr(A), _ld(A), _vptr(B), _ld(B),
                                 _ptr(C, ctypes.c_double), N, threads or default_threads())
    if rc != 0:
        raise MemoryError("oracle allocation failed")
    return C


def gemm_rows_f64(A_bits, B_bits, rows, in_fmt, threads: int | None = None) -> np.ndarray:
    """Rows ``rows`` of C = A.B in fp64 (len(rows) x N)."""
    A = _as_bits_2d(A_bits, in_fmt)
    B = _as_bits_2d(B_bits, in_fmt)
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if r.size and (r.min() < 0 or r.max() >= M):
        raise IndexError("row index out of range")
    C = np.zeros((r.size, N), dtype=np.float64)
    rc = _load().oracle_gemm_rows_f64(r.size, _ptr(r, ctypes.c_int64), N, K, _fmt_in(in_fmt),
                                      _vptr(A), _ld(A), _vptr(B), _ld(B),
                                      _ptr(C, ctypes.c_double), N, threads or default_threads())
    if rc != 0:
        raise MemoryError("oracle allocation failed")
    return C


def decode(bits, in_fmt) -> np.ndarray:
    """Input bit patterns -> exact float64 values (oracle's own decoder)."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=_bits_dtype(in_fmt)))
    out = np.empty(b.shape, dtype=np.float64)
    _load().oracle_decode_array(_fmt_in(in_fmt), _vptr(b), _ptr(out, ctypes.c_double), b.size)
    return out


def round_to(x, out_fmt) -> np.ndarray:
    """IEEE round-to-nearest-even of float64 values to fp32/fp16/bf16 (as float64)."""
    f = _fmt_out(out_fmt)
    shape = np.shape(x)
    xs = np.ascontiguousarray(np.asarray(x, dtype=np.float64)).reshape(-1)
    out = np.empty(xs.shape, dtype=np.float64)
    _load().oracle_round_to_array(f, _ptr(xs, ctypes.c_double), _ptr(out, ctypes.c_double), xs.size)
    return out.reshape(shape)


def ulp(r, out_fmt) -> np.ndarray:
    """Spacing of the output format at r (smallest subnormal at r == 0)."""
    f = _fmt_out(out_fmt)
    shape = np.shape(r)
    rs = np.ascontiguousarray(np.asarray(r, dtype=np.float64)).reshape(-1)
    out = np.empty(rs.shape, dtype=np.float64)
    _load().oracle_ulp_array(f, _ptr(rs, ctypes.c_double), _ptr(out, ctypes.c_double), rs.size)
    return out.reshape(shape)


def flops(M: int, N: int, K: int) -> int:
    """2MNK: one multiply and one add per inner-loop step."""
    return 2 * int(M) * int(N) * int(K)


def bound(K: int, out_fmt, r, extra=None) -> np.ndarray:
    """Acceptance bound on |y - r| for a GPU output y against oracle value r
    (plus ``extra``, e.g. align_bound8, where given)."""
    f = _fmt_out(out_fmt)
    acc = float(K) * 2.0 ** -20
    r = np.asarray(r, dtype=np.float64)
    b = np.full(r.shape, acc) if f == OUT_F32 else ulp(r, f) + acc
    if extra is not None:
        b = b + np.asarray(extra, dtype=np.float64)
    return b


ALIGN8_GROUP = 8       # consecutive k aligned together by the 8-bit MFMA
ALIGN8_BITS = 13       # binades kept below a group's largest product


def align_bound8(A_bits, B_bits, in_fmt, b_layout="row", rows=None) -> np.ndarray:
    """7 * 2^-13 * sum_g max_{k in g}|A[i,k]| * max_{k in g}|B[k,j]| over the
    groups g = [8m, 8m+8) of k: the most the 8-bit MFMA's alignment can lose
    on output (i, j).  B_bits is K x N ("row") or N x K ("col"); ``rows``
    selects output rows."""
    A = np.abs(decode(_as_bits_2d(A_bits, in_fmt), in_fmt))
    B = np.abs(decode(_as_bits_2d(B_bits, in_fmt), in_fmt))
    if _layout(b_layout) == B_COL_MAJOR:
        B = B.T
    if rows is not None:
        A = A[np.asarray(rows, dtype=np.int64)]
    M, K = A.shape
    N = B.shape[1]
    G = -(-K // ALIGN8_GROUP)
    Ap = np.zeros((M, G * ALIGN8_GROUP))
    Ap[:, :K] = A
    Bp = np.zeros((G * ALIGN8_GROUP, N))
    Bp[:K] = B
    maxA = Ap.reshape(M, G, ALIGN8_GROUP).max(axis=2)
    maxB = Bp.reshape(G, ALIGN8_GROUP, N).max(axis=1)
    return (ALIGN8_GROUP - 1) * 2.0 ** -ALIGN8_BITS * (maxA @ maxB)


def compare(y, r, K: int, out_fmt, extra=None) -> dict:
    """Check a GPU result y (float64 array of decoded outputs) against oracle r.

    Returns max_abs, max_rel (over |r| > 0), the worst excess over the bound,
    the number of elements outside the bound, and ``ok``.
    """
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if y.shape != r.shape:
        raise ValueError("shape mismatch %s vs %s" % (y.shape, r.shape))
    if y.size == 0:
        return {"ok": True, "max_abs": 0.0, "max_rel": 0.0, "n_bad": 0, "worst_ratio": 0.0}
    err = np.abs(y - r)
    err = np.where(np.isnan(err), np.inf, err)
    b = bound(K, out_fmt, r, extra)
    nz = np.abs(r) > 0
    max_rel = float(np.max(err[nz] / np.abs(r[nz]))) if nz.any() else 0.0
    n_bad = int(np.count_nonzero(err > b))
    return {"ok": n_bad == 0, "max_abs": float(err.max()), "max_rel": max_rel,
            "n_bad": n_bad, "worst_ratio": float(np.max(err / b))}


B_ROW_MAJOR, B_COL_MAJOR = 0, 1


def _layout(b_layout) -> int:
    if b_layout in ("row", "nn", B_ROW_MAJOR):
        return B_ROW_MAJOR
    if b_layout in ("col", "tn", B_COL_MAJOR):
        return B_COL_MAJOR
    raise ValueError("unknown B layout %r" % (b_layout,))


def gemm_ex_f64(A_bits, B_bits, in_fmt, b_layout="row", alpha=1.0, beta=0.0, C_old=None,
                bias=None, relu=False, rows=None, threads: int | None = None) -> np.ndarray:
    """act(alpha * A.B + beta * C_old + bias) in fp64.

    B_bits is K x N (b_layout "row") or its N x K transpose (b_layout "col").
    C_old: float64 values of the old output (the selected rows when ``rows``
    is given); ignored when beta == 0.  bias: N float64 values or None.
    relu: apply max(x, 0) last.  rows: output rows to compute (None = all).
    """
    A = _as_bits_2d(A_bits, in_fmt)
    B = _as_bits_2d(B_bits, in_fmt)
    lay = _layout(b_layout)
    M, K = A.shape
    K2, N = B.shape if lay == B_ROW_MAJOR else B.shape[::-1]
    if K != K2:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
    if rows is None:
        r = np.arange(M, dtype=np.int64)
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        if r.size and (r.min() < 0 or r.max() >= M):
            raise IndexError("row index out of range")
    C = np.zeros((r.size, N), dtype=np.float64)
    cold_p, ldcold = None, 0
    if beta != 0.0:
        if C_old is None:
            raise ValueError("beta != 0 needs C_old")
        cold = np.ascontiguousarray(np.asarray(C_old, dtype=np.float64))
        if cold.shape != (r.size, N):
            raise ValueError("C_old must be %d x %d" % (r.size, N))
        cold_p, ldcold = _ptr(cold, ctypes.c_double), N
    bias_p = None
    if bias is not None:
        bz = np.ascontiguousarray(np.asarray(bias, dtype=np.float64))
        if bz.shape != (N,):
            raise ValueError("bias must have N = %d values" % N)
        bias_p = _ptr(bz, ctypes.c_double)
    rc = _load().oracle_gemm_ex_f64(r.size, _ptr(r, ctypes.c_int64), N, K, _fmt_in(in_fmt), lay,
                                    _vptr(A), _ld(A), _vptr(B), _ld(B),
                                    float(alpha), float(beta), cold_p, ldcold, bias_p,
                                    1 if relu else 0, _ptr(C, ctypes.c_double), N,
                                    threads or default_threads())
    if rc != 0:
        raise MemoryError("oracle allocation failed") if rc == -1 else ValueError("oracle rc %d" % rc)
    return C


def bound_ex(K: int, out_fmt, r, alpha=1.0, beta=0.0, C_old=None, bias=None, dot=None,
             extra=None) -> np.ndarray:
    """Acceptance bound for the general form.

    The fp32 accumulation contributes |alpha| * K * 2^-20 (the plain bound
    scaled by alpha); the fp32 epilogue (scale, add beta*C_old, add bias) and
    an fp32 output rounding contribute at most four roundings of 2^-24 each
    of the largest magnitude involved.  The accumulator itself may lie up to
    K * 2^-20 from the exact dot product, so the scaled accumulator is at most
    |alpha| * (|dot| + K * 2^-20) in magnitude, and the roundings are bounded
    by 2^-22 * (|alpha| * (|dot| + K * 2^-20) + |beta * C_old| + |bias|)
    (an exact-rational emulation of the epilogue found the bound without the
    K * 2^-20 inside exceeded when |dot| << K * 2^-20).  A half-precision
    output adds one ulp of its format at |r| + e32, e32 being the fp32 part of
    the bound: the fp32 value that is rounded lies within e32 of r, and half
    an ulp at that value can exceed an ulp at r when r is small and
    cancellation left the accumulation error in place (the same emulation).
    ReLU is 1-Lipschitz and adds nothing.  ``dot`` is the fp64 A.B (defaults to r, exact when alpha = 1,
    beta = 0, no bias and no ReLU clipping)."""
    f = _fmt_out(out_fmt)
    r = np.asarray(r, dtype=np.float64)
    d = r if dot is None else np.asarray(dot, dtype=np.float64)
    mag = abs(alpha) * (np.abs(d) + float(K) * 2.0 ** -20)
    if beta != 0.0:
        mag = mag + np.abs(beta * np.asarray(C_old, dtype=np.float64))
    if bias is not None:
        mag = mag + np.abs(np.asarray(bias, dtype=np.float64))[None, :]
    b = abs(alpha) * float(K) * 2.0 ** -20 + 2.0 ** -22 * mag
    if extra is not None:                  # a bound on the dot product's own error, scaled by alpha
        b = b + abs(alpha) * np.asarray(extra, dtype=np.float64)
    if f != OUT_F32:
        b = b + ulp(np.abs(r) + b, f)
    return b


def compare_ex(y, r, K: int, out_fmt, **kw) -> dict:
    """compare() with the bound of the general form (keyword args of bound_ex)."""
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if y.shape != r.shape:
        raise ValueError("shape mismatch %s vs %s" % (y.shape, r.shape))
    if y.size == 0:
        return {"ok": True, "max_abs": 0.0, "n_bad": 0, "worst_ratio": 0.0}
    err = np.abs(y - r)
    err = np.where(np.isnan(err), np.inf, err)
    b = bound_ex(K, out_fmt, r, **kw)
    n_bad = int(np.count_nonzero(err > b))
    return {"ok": n_bad == 0, "max_abs": float(err.max()), "n_bad": n_bad,
            "worst_ratio": float(np.max(err / b))}
