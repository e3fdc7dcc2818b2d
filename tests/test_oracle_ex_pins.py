"""Pins for the oracle's general form act(alpha*A.B + beta*C_old + bias) and its
column-major-B ("TN") indexing (no GPU).

Each test checks the oracle against something other than itself: exact
rational arithmetic written out here with Python Fractions, integer matmuls,
and closed forms (zero operands, power-of-two scaling, ReLU of a dominated
bias, a NaN in the old output that beta = 0 must never read).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from dense_half_precision_tiled_amd import inputs


def _exact_ex(Ad, Bd_kn, alpha, beta, Cold, bias, relu):
    """Exact rational act(alpha*A.B + beta*C_old + bias), rounded once to double.

    Ad is M x K, Bd_kn is K x N (already in the logical orientation)."""
    M, K = Ad.shape
    N = Bd_kn.shape[1]
    out = np.empty((M, N))
    fa, fb = Fraction(alpha), Fraction(beta)
    for i in range(M):
        for j in range(N):
            s = sum((Fraction(Ad[i, k]) * Fraction(Bd_kn[k, j]) for k in range(K)), Fraction(0))
            v = fa * s
            if beta != 0:
                v += fb * Fraction(Cold[i, j])
            if bias is not None:
                v += Fraction(bias[j])
            if relu and v < 0:
                v = Fraction(0)
            out[i, j] = float(v)
    return out


def _scale(Ad, Bd_kn, alpha, beta, Cold, bias):
    mag = abs(alpha) * (np.abs(Ad) @ np.abs(Bd_kn))
    if beta != 0:
        mag = mag + abs(beta) * np.abs(Cold)
    if bias is not None:
        mag = mag + np.abs(bias)[None, :]
    return mag


CASES = [
    # (M, N, K, fmt, layout, alpha, beta, use_bias, relu)
    (3, 5, 7, "f16", "col", 1.0, 0.0, False, False),
    (4, 3, 9, "bf16", "col", 1.0, 0.0, False, False),
    (5, 4, 6, "f16", "row", 0.75, -1.5, True, False),
    (6, 7, 5, "bf16", "col", -2.0, 0.5, True, True),
    (2, 9, 11, "f16", "col", 0.3, 1.0, True, True),
    (7, 2, 3, "bf16", "row", 1.0, 0.0, True, True),
    (1, 1, 1, "f16", "col", 1.0, 1.0, False, True),
]


@pytest.mark.parametrize("case", CASES)
def test_general_form_against_exact_rationals(case):
    M, N, K, fmt, layout, alpha, beta, use_bias, relu = case
    seed = 1000 + M * 100 + N * 10 + K
    A = inputs.uniform((M, K), seed, fmt)
    Bkn = inputs.uniform((K, N), seed + 1, fmt)
    Bmem = np.ascontiguousarray(Bkn.T) if layout == "col" else Bkn
    rng = np.random.Generator(np.random.PCG64(seed + 2))
    Cold = rng.uniform(-2, 2, (M, N))
    bias = rng.uniform(-1, 1, N) if use_bias else None
    got = oracle.gemm_ex_f64(A, Bmem, fmt, b_layout=layout, alpha=alpha, beta=beta,
                             C_old=Cold, bias=bias, relu=relu)
    Ad, Bd = oracle.decode(A, fmt), oracle.decode(Bkn, fmt)
    want = _exact_ex(Ad, Bd, alpha, beta, Cold, bias, relu)
    tol = (K + 4) * 2.0 ** -52 * _scale(Ad, Bd, alpha, beta, Cold, bias)
    assert np.all(np.abs(got - want) <= tol)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_column_major_B_integer_fixture_matches_int64_matmul(fmt):
    A = inputs.ints((13, 21), 31, fmt)
    Bt = inputs.ints((17, 21), 32, fmt)          # N x K in memory: the TN operand
    Ai = oracle.decode(A, fmt).astype(np.int64)
    Bti = oracle.decode(Bt, fmt).astype(np.int64)
    got = oracle.gemm_ex_f64(A, Bt, fmt, b_layout="col")
    assert np.array_equal(got, (Ai @ Bti.T).astype(np.float64))


def test_column_major_B_with_padded_leading_dimension():
    A = inputs.ints((9, 14), 41, "f16")
    Bt = inputs.padded(inputs.ints((11, 14), 42, "f16"), 40)[:, :14]   # ldb = 40 > K
    assert Bt.strides[0] == 80
    Ai = oracle.decode(A, "f16").astype(np.int64)
    Bti = oracle.decode(np.ascontiguousarray(Bt), "f16").astype(np.int64)
    got = oracle.gemm_ex_f64(A, Bt, "f16", b_layout="col")
    assert np.array_equal(got, (Ai @ Bti.T).astype(np.float64))


def test_zero_A_leaves_beta_C_plus_bias():
    A = np.zeros((4, 6), dtype=np.uint16)
    B = inputs.uniform((6, 5), 51, "bf16")
    Cold = np.arange(20, dtype=np.float64).reshape(4, 5) - 7.0
    bias = np.array([0.5, -0.25, 1.0, 0.0, -3.0])
    got = oracle.gemm_ex_f64(A, B, "bf16", alpha=1.0, beta=2.0, C_old=Cold, bias=bias)
    assert np.array_equal(got, 2.0 * Cold + bias[None, :])
    got = oracle.gemm_ex_f64(A, B, "bf16", alpha=1.0, beta=2.0, C_old=Cold, bias=bias, relu=True)
    assert np.array_equal(got, np.maximum(2.0 * Cold + bias[None, :], 0.0))


def test_alpha_zero_ignores_the_product():
    A = inputs.uniform((3, 8), 52, "f16")
    B = inputs.uniform((8, 4), 53, "f16")
    Cold = np.full((3, 4), 1.25)
    got = oracle.gemm_ex_f64(A, B, "f16", alpha=0.0, beta=-1.0, C_old=Cold)
    assert np.array_equal(got, -Cold)


def test_power_of_two_alpha_scales_exactly():
    A = inputs.uniform((6, 40), 54, "f16")
    B = inputs.uniform((40, 7), 55, "f16")
    plain = oracle.gemm_f64(A, B, "f16")
    for alpha in (2.0, -0.5, 0.125):
        assert np.array_equal(oracle.gemm_ex_f64(A, B, "f16", alpha=alpha), alpha * plain)


def test_beta_zero_never_reads_old_output():
    A = inputs.uniform((3, 5), 56, "f16")
    B = inputs.uniform((5, 4), 57, "f16")
    Cold = np.full((3, 4), np.nan)
    got = oracle.gemm_ex_f64(A, B, "f16", alpha=1.0, beta=0.0, C_old=Cold)
    assert np.array_equal(got, oracle.gemm_f64(A, B, "f16"))


def test_bias_is_per_column_and_added_before_relu():
    A = inputs.ints((5, 8), 58, "f16")
    B = inputs.ints((8, 6), 59, "f16")
    plain = oracle.gemm_f64(A, B, "f16")
    bias = np.array([100.0, -100.0, 0.5, -0.5, 3.0, -1000.0])
    got = oracle.gemm_ex_f64(A, B, "f16", bias=bias)
    assert np.array_equal(got - plain, np.broadcast_to(bias, plain.shape))
    got = oracle.gemm_ex_f64(A, B, "f16", bias=bias, relu=True)
    assert np.array_equal(got, np.maximum(plain + bias[None, :], 0.0))
    # |plain| <= 8 * 4 = 32 here, so a bias of -1000 clips the whole column and
    # a bias of +100 makes it positive: ReLU must act after the bias
    assert np.all(got[:, 5] == 0.0) and np.all(got[:, 0] > 0.0)


def test_rows_mode_matches_full_general_form():
    A = inputs.uniform((12, 30), 60, "bf16")
    Bt = inputs.uniform((9, 30), 61, "bf16")
    rng = np.random.Generator(np.random.PCG64(62))
    Cold = rng.normal(size=(12, 9))
    bias = rng.normal(size=9)
    full = oracle.gemm_ex_f64(A, Bt, "bf16", b_layout="col", alpha=1.5, beta=-0.25, C_old=Cold,
                              bias=bias, relu=True)
    rows = np.array([11, 0, 5, 5])
    part = oracle.gemm_ex_f64(A, Bt, "bf16", b_layout="col", alpha=1.5, beta=-0.25,
                              C_old=Cold[rows], bias=bias, relu=True, rows=rows)
    assert np.array_equal(part, full[rows])


def test_bound_ex_reduces_to_plain_bound_terms():
    r = np.array([[1.0, -3.0]])
    # alpha = 1, beta = 0, no bias: K*2^-20 plus the epilogue rounding allowance
    acc = 64 * 2.0 ** -20
    b = oracle.bound_ex(64, "f32", r)
    assert np.array_equal(b, acc + 2.0 ** -22 * (np.abs(r) + acc))
    b16 = oracle.bound_ex(64, "f16", r)
    assert np.array_equal(b16 - b, oracle.ulp(np.abs(r) + b, "f16"))
    assert np.allclose(oracle.bound_ex(64, "f32", r, alpha=-4.0, dot=r / -4.0),
                       4 * acc + 2.0 ** -22 * (np.abs(r) + 4 * acc), rtol=0, atol=1e-18)
