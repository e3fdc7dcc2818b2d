"""Planted mistakes in a copy of the oracle (CPU only).

Each mutant is oracle.c with one plausible slip (a dropped term, a wrong sign,
a transposed operand, an ignored stride, a wrong exponent bias, a wrong tie
rule).  It is compiled to a temporary library and run through a small battery
of the pins; every mutant must fail at least one of them, and the unmutated
copy must pass all of them.  This shows the pins have teeth.
"""
import ctypes
import json
import os
import shutil
import subprocess

import numpy as np
import pytest

from dense_half_precision_tiled_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "control": None,
    "dropped_last_k": ("for (int64_t k = 0; k < jb->K; ++k) {", "for (int64_t k = 0; k + 1 < jb->K; ++k) {"),
    "sign_dropped_f16": ("    return sign ? -v : v;\n}\n\n/* bfloat16", "    (void)sign; return v;\n}\n\n/* bfloat16"),
    "transposed_B": ("c[j] += a * b[j];", "c[j] += a * jb->Bd[(j % jb->K) * jb->N + (k % jb->N)]; (void)b;"),
    "ignores_lda": ("load_in(jb->in_fmt, jb->A, i * jb->lda + k)", "load_in(jb->in_fmt, jb->A, i * jb->K + k)"),
    "subnormal_scale": ("v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    "bf16_bias": ("v = ldexp((double)(128 + f), e - 134);", "v = ldexp((double)(128 + f), e - 133);"),
    "ties_away": ("return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "return fl + 1.0;"),
    "accumulate_in_float": ("c[j] += a * b[j];", "c[j] = (float)(c[j] + a * b[j]);"),
    "e4m3_bias": ("v = ldexp((double)(8 + f), e - 10);", "v = ldexp((double)(8 + f), e - 9);"),
    "e4m3_exp15_all_nan": ("if (e == 15 && f == 7)", "if (e == 15)"),
    "e4m3_sign_dropped": ("    return sign ? -v : v;\n}\n\n/* OFP8 E5M2", "    (void)sign; return v;\n}\n\n/* OFP8 E5M2"),
    "e5m2_subnormal_scale": ("v = ldexp((double)f, -16);", "v = ldexp((double)f, -17);"),
    "e5m2_hidden_bit": ("v = ldexp((double)(4 + f), e - 17);", "v = ldexp((double)(8 + f), e - 18);"),
    "byte_read_as_halfword": ("oracle_decode_e4m3(((const uint8_t*)base)[idx])",
                              "oracle_decode_e4m3((uint8_t)((const uint16_t*)base)[idx])"),
}


def _build(tmp_path, name, mutation):
    src = open(SRC).read()
    if mutation is not None:
        old, new = mutation
        assert src.count(old) >= 1, "mutation anchor not found: %s" % name
        src = src.replace(old, new, 1)
    c = tmp_path / ("%s.c" % name)
    so = tmp_path / ("lib%s.so" % name)
    c.write_text(src)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", str(c), "-o", str(so),
                           "-lm", "-lpthread"])
    lib = ctypes.CDLL(str(so))
    i64, u16p, f64p = ctypes.c_int64, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)
    lib.oracle_gemm_f64.argtypes = [i64, i64, i64, ctypes.c_int, u16p, i64, u16p, i64, f64p, i64,
                                    ctypes.c_int]
    lib.oracle_decode_array.argtypes = [ctypes.c_int, u16p, f64p, i64]
    lib.oracle_round_to.argtypes = [ctypes.c_int, ctypes.c_double]
    lib.oracle_round_to.restype = ctypes.c_double
    return lib


FMT_CODE = {"f16": 0, "bf16": 1, "e4m3": 2, "e5m2": 3}


def _gemm(lib, A, B, fmt):
    M, K = A.shape
    N = B.shape[1]
    C = np.zeros((M, N))
    lib.oracle_gemm_f64(M, N, K, FMT_CODE[fmt],
                        ctypes.c_void_p(A.ctypes.data), A.strides[0] // A.itemsize,
                        ctypes.c_void_p(B.ctypes.data), B.strides[0] // B.itemsize,
                        C.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), N, 2)
    return C


def _battery(lib):
    """Names of the pins this library fails."""
    failed = []
    with open(os.path.join(ROOT, "tests", "golden", "worked_example_2x3x2.json")) as f:
        g = json.load(f)
    for fmt in ("f16", "bf16"):
        C = _gemm(lib, inputs.from_values(g["A"], fmt), inputs.from_values(g["B"], fmt), fmt)
        if C.tolist() != g["C"]:
            failed.append("worked_example_" + fmt)
    # integer fixture with padded leading dimensions, against an int64 matmul
    A = inputs.padded(inputs.ints((19, 37), 5, "f16"), 48)[:, :37]
    B = inputs.padded(inputs.ints((37, 23), 6, "f16"), 32)[:, :23]
    exact = (A.view(np.float16).astype(np.int64) @ B.view(np.float16).astype(np.int64))
    if not np.array_equal(_gemm(lib, A, B, "f16"), exact.astype(np.float64)):
        failed.append("int_fixture_ld")
    # brute force against exact scaled-integer arithmetic on a random case
    A = inputs.uniform((9, 300), 7, "f16")
    B = inputs.uniform((300, 11), 8, "f16")
    Ai = (A.view(np.float16).astype(np.float64) * 2.0 ** 24).astype(np.int64)
    Bi = (B.view(np.float16).astype(np.float64) * 2.0 ** 24).astype(np.int64)
    exact = np.array([[float(int(v)) for v in r] for r in Ai @ Bi]) * 2.0 ** -48
    absdot = np.abs(Ai).astype(float) @ np.abs(Bi).astype(float) * 2.0 ** -48
    if not np.all(np.abs(_gemm(lib, A, B, "f16") - exact) <= 300 * 2.0 ** -52 * absdot):
        failed.append("exact_random")
    # decoders against numpy / float32 widening
    bits = np.arange(65536, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        bf16_ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for fmt, ref in (("f16", bits.view(np.float16).astype(np.float64)),
                     ("bf16", bf16_ref)):
        out = np.empty(65536)
        lib.oracle_decode_array(FMT_CODE[fmt], ctypes.c_void_p(bits.ctypes.data),
                                out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), 65536)
        fin = np.isfinite(ref)
        if not np.array_equal(out[fin], ref[fin]):
            failed.append("decode_" + fmt)
    # 8-bit decoders against torch's float8 types, specials included
    import torch
    codes = np.arange(256, dtype=np.uint8)
    for fmt, dt in (("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)):
        ref = torch.from_numpy(codes.copy()).view(dt).to(torch.float64).numpy()
        out = np.empty(256)
        lib.oracle_decode_array(FMT_CODE[fmt], ctypes.c_void_p(codes.ctypes.data),
                                out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), 256)
        if not (np.array_equal(np.isnan(out), np.isnan(ref)) and
                np.array_equal(out[~np.isnan(ref)], ref[~np.isnan(ref)])):
            failed.append("decode_" + fmt)
    # 8-bit integer fixture with padded (NaN-filled) leading dimensions
    for fmt in ("e4m3", "e5m2"):
        A = inputs.padded(inputs.ints((13, 41), 15, fmt), 56)[:, :41]
        B = inputs.padded(inputs.ints((41, 17), 16, fmt), 24)[:, :17]
        Av = torch.from_numpy(np.ascontiguousarray(A)).view(
            torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2).to(torch.float64).numpy()
        Bv = torch.from_numpy(np.ascontiguousarray(B)).view(
            torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2).to(torch.float64).numpy()
        exact = Av.astype(np.int64) @ Bv.astype(np.int64)
        if not np.array_equal(_gemm(lib, A, B, fmt), exact.astype(np.float64)):
            failed.append("int_fixture_" + fmt)
    # rounding ties against numpy's IEEE float16 cast
    ties = 1.0 + (np.arange(0, 1000) + 0.5) * 2.0 ** -10   # halfway between fp16 neighbours in [1, 2)
    got = np.array([lib.oracle_round_to(1, float(t)) for t in ties])
    if not np.array_equal(got, ties.astype(np.float16).astype(np.float64)):
        failed.append("round_ties_f16")
    return failed


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    lib = _build(tmp_path, name, MUTANTS[name])
    failed = _battery(lib)
    if name == "control":
        assert failed == []
    else:
        assert failed, "planted mistake %s passed every pin" % name


# ---------------------------------------------------------------------------
# The general form act(alpha*A.B + beta*C_old + bias) and column-major B.
# Mutants of that code run through the pins of tests/test_oracle_ex_pins.py,
# with the mutant library swapped in for the oracle's own.
EX_MUTANTS = {
    "ex_control": None,
    "relu_before_bias": ("            if (bias) v += bias[j];\n            if (relu && v < 0.0) v = 0.0;",
                         "            if (relu && v < 0.0) v = 0.0;\n            if (bias) v += bias[j];"),
    "bias_by_row": ("if (bias) v += bias[j];", "if (bias) v += bias[r % N];"),
    "beta_ignored": ("if (beta != 0.0) v += beta * Cold[r * ldcold + j];", "(void)Cold; (void)ldcold;"),
    "beta_sign": ("v += beta * Cold[r * ldcold + j];", "v -= beta * Cold[r * ldcold + j];"),
    "alpha_on_bias": ("if (bias) v += bias[j];", "if (bias) v += alpha * bias[j];"),
    "col_major_read_as_row": ("Bd[k * N + j] = load_in(in_fmt, B, j * ldb + k);",
                              "Bd[k * N + j] = load_in(in_fmt, B, (k * ldb + j) % (N * ldb));"),
    "col_major_ignores_ldb": ("Bd[k * N + j] = load_in(in_fmt, B, j * ldb + k);",
                              "Bd[k * N + j] = load_in(in_fmt, B, j * K + k);"),
    "relu_clips_to_abs": ("if (relu && v < 0.0) v = 0.0;", "if (relu && v < 0.0) v = -v;"),
}


def _ex_battery(lib, monkeypatch):
    import oracle
    from tests import test_oracle_ex_pins as P
    monkeypatch.setattr(oracle, "_lib", oracle._declare(lib))
    pins = [("exact_%d" % n, lambda c=c: P.test_general_form_against_exact_rationals(c))
            for n, c in enumerate(P.CASES)]
    pins += [
        ("int_tn_f16", lambda: P.test_column_major_B_integer_fixture_matches_int64_matmul("f16")),
        ("int_tn_padded", P.test_column_major_B_with_padded_leading_dimension),
        ("zero_A", P.test_zero_A_leaves_beta_C_plus_bias),
        ("alpha_zero", P.test_alpha_zero_ignores_the_product),
        ("pow2_alpha", P.test_power_of_two_alpha_scales_exactly),
        ("beta_zero_nan", P.test_beta_zero_never_reads_old_output),
        ("bias_then_relu", P.test_bias_is_per_column_and_added_before_relu),
        ("rows_mode", P.test_rows_mode_matches_full_general_form),
    ]
    failed = []
    for name, fn in pins:
        try:
            fn()
        except AssertionError:
            failed.append(name)
    return failed


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(EX_MUTANTS))
def test_general_form_mutant_is_caught(tmp_path, monkeypatch, name):
    lib = _build(tmp_path, name, EX_MUTANTS[name])
    failed = _ex_battery(lib, monkeypatch)
    if name == "ex_control":
        assert failed == []
    else:
        assert failed, "planted mistake %s passed every pin" % name
