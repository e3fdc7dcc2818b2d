"""Pins for the CPU oracle (no GPU).  Each test checks the oracle against
something other than itself: values printed on the pages, exact rational
arithmetic, closed forms, or an independent library routine."""
import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from dense_half_precision_tiled_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bits(values, fmt):
    return inputs.from_values(values, fmt)


# ---------------------------------------------------------------- decoders
def test_decode_f16_all_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.decode(bits, "f16")
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got), np.isinf(ref))


def test_decode_bf16_all_patterns_match_float32_widening():
    bits = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        ref = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    got = oracle.decode(bits.astype(np.uint16), "bf16")
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


# ---------------------------------------------------------------- rounding
def test_round_fp16_page_table():
    g = _golden("fp16_rounding.json")
    for x, want in g["fp16"]:
        assert oracle.round_to(x, "f16") == want
    for x, want in g["fp32"]:
        assert oracle.round_to(x, "f32") == want
    # the page's struct demo is IEEE binary16/binary32 storage
    for x, want in g["fp16"]:
        assert struct.unpack("e", struct.pack("e", x))[0] == want
    assert oracle.ulp(1.0, "f16") == g["fp16_epsilon"]
    assert oracle.ulp(1.0, "f32") == g["fp32_epsilon"]
    assert oracle.round_to(65504.0, "f16") == g["fp16_max_finite"]
    assert oracle.round_to(65519.99, "f16") == 65504.0
    assert math.isinf(oracle.round_to(65520.0, "f16"))


def test_round_fp16_matches_numpy_on_random_doubles():
    rng = np.random.Generator(np.random.PCG64(7))
    x = np.concatenate([
        rng.uniform(-70000, 70000, 4000),
        rng.standard_normal(4000) * 1e-5,          # subnormal range
        rng.standard_normal(4000),
        # exact ties between neighbouring fp16 values
        (np.arange(-2000, 2000) + 0.5) * 2.0 ** -10,
        (np.arange(1, 3000) + 0.5) * 2.0 ** -24,
    ])
    got = oracle.round_to(x, "f16")
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(got, ref)


def test_round_fp32_matches_numpy_on_random_doubles():
    rng = np.random.Generator(np.random.PCG64(8))
    x = np.concatenate([
        rng.standard_normal(5000) * 1e3,
        rng.standard_normal(2000) * 1e-40,         # fp32 subnormals
        (np.arange(-3000, 3000) + 0.5) * 2.0 ** -23 + 1.0,   # ties near 1
    ])
    got = oracle.round_to(x, "f32")
    ref = x.astype(np.float32).astype(np.float64)
    assert np.array_equal(got, ref)


def test_round_bf16_matches_torch_on_random_doubles():
    torch = pytest.importorskip("torch")
    rng = np.random.Generator(np.random.PCG64(9))
    # values exactly representable in fp32, so a single rounding to bf16
    x = np.concatenate([
        rng.standard_normal(5000).astype(np.float32),
        ((np.arange(-3000, 3000) + 0.5) * 2.0 ** -7 + 0.0).astype(np.float32),
    ]).astype(np.float64)
    got = oracle.round_to(x, "bf16")
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, ref)


def test_ulp_values():
    assert oracle.ulp(1024.0, "f16") == 1.0
    assert oracle.ulp(1023.0, "f16") == 0.5
    assert oracle.ulp(0.0, "f16") == 2.0 ** -24
    assert oracle.ulp(1.0, "bf16") == 2.0 ** -7
    assert oracle.ulp(100.0, "bf16") == 0.5
    assert oracle.ulp(-3.0, "f32") == 2.0 ** -22


# ---------------------------------------------------------------- worked example
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_worked_example(fmt):
    g = _golden("worked_example_2x3x2.json")
    A = _bits(g["A"], fmt)
    B = _bits(g["B"], fmt)
    C = oracle.gemm_f64(A, B, fmt)
    assert C.tolist() == g["C"]
    M, K = A.shape
    N = B.shape[1]
    assert oracle.flops(M, N, K) == g["flops"]
    # the page's two traffic models (fp32 words) for the same product
    scalar_bytes = 4 * M * N * (2 * K + 1)
    unique_bytes = 4 * (M * K + K * N + M * N)
    assert round(oracle.flops(M, N, K) / scalar_bytes, 3) == g["scalar_load_model_flop_per_byte"]
    assert round(oracle.flops(M, N, K) / unique_bytes, 3) == g["perfect_reuse_bound_flop_per_byte"]
    n = 4096
    assert round(oracle.flops(n, n, n) / (4 * 3 * n * n), 1) == g["fp32_ideal_intensity_n4096_flop_per_byte"]


def test_flop_counts():
    g = _golden("flop_counts.json")
    for c in g["cases"]:
        assert oracle.flops(c["M"], c["N"], c["K"]) == c["logical"]
        if "padded" in c:
            pm, pn, pk = c["padded_shape"]
            assert oracle.flops(pm, pn, pk) == c["padded"]
            for d, p in zip((c["M"], c["N"], c["K"]), c["padded_shape"]):
                assert p == -(-d // 16) * 16
        if "extra_percent" in c:
            assert round(100 * (c["padded"] / c["logical"] - 1), 1) == c["extra_percent"]


def test_two_reference_example():
    """Rounded-input reference is 0, original-input reference is ~1.0002e-4."""
    g = _golden("fp16_rounding.json")["two_reference"]
    A_orig = np.array([g["A"]])
    B_orig = np.array([g["B"]]).T
    A = inputs.from_values(A_orig, "f16")
    B = inputs.from_values(B_orig, "f16")
    ref1 = oracle.gemm_f64(A, B, "f16")[0, 0]
    a32 = np.array(g["A"], dtype=np.float32).astype(np.float64)
    ref2 = float(np.dot(a32, np.array(g["B"])))
    assert ref1 == g["rounded_input_ref"]
    assert round(ref2, 8) == g["original_input_ref_8dp"]
    assert abs(ref1 - ref2) / abs(ref2) == g["original_input_relative_error"]


# ---------------------------------------------------------------- exact rationals
def _exact_gemm(Ad, Bd):
    """Exact rational product, independent of the oracle's code."""
    M, K = Ad.shape
    N = Bd.shape[1]
    Af = [[Fraction(float(v)) for v in row] for row in Ad]
    Bf = [[Fraction(float(v)) for v in row] for row in Bd]
    return [[sum((Af[i][k] * Bf[k][j] for k in range(K)), Fraction(0)) for j in range(N)]
            for i in range(M)]


def _check_against_exact(A, B, fmt):
    Ad = A.view(np.float16).astype(np.float64) if fmt == "f16" else \
        (A.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    Bd = B.view(np.float16).astype(np.float64) if fmt == "f16" else \
        (B.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    C = oracle.gemm_f64(A, B, fmt, threads=2)
    E = _exact_gemm(Ad, Bd)
    K = A.shape[1]
    absdot = np.abs(Ad) @ np.abs(Bd)
    for i in range(C.shape[0]):
        for j in range(C.shape[1]):
            exact = E[i][j]
            tol = Fraction(max(K - 1, 0)) * Fraction(2) ** -53 * Fraction(float(absdot[i, j]))
            # absdot is rounded; pad the bound by one more relative ulp of it
            tol += Fraction(2) ** -50 * Fraction(float(absdot[i, j]))
            assert abs(Fraction(C[i, j]) - exact) <= tol, (i, j)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_brute_force_tiny_shapes(fmt):
    rng = np.random.Generator(np.random.PCG64(11))
    for M in range(1, 9):
        for N in (1, 3, 8):
            for K in (1, 2, 5, 8):
                seed = int(rng.integers(1 << 30))
                law = inputs.uniform if fmt == "f16" else inputs.normal
                A = law((M, K), seed, fmt)
                B = law((K, N), seed + 1, fmt)
                _check_against_exact(A, B, fmt)


@pytest.mark.parametrize("shape", [(17, 65, 19), (31, 29, 37)])
def test_brute_force_odd_shapes(shape):
    M, N, K = shape
    A = inputs.uniform((M, K), 21, "f16")
    B = inputs.uniform((K, N), 22, "f16")
    _check_against_exact(A, B, "f16")


@pytest.mark.parametrize("shape", [(73, 61, 67), (257, 263, 251)])
def test_exact_integer_scaled_odd_shapes(shape):
    """fp16 values in U[-1,1) are integers times 2^-24: the exact product is an
    int64 matmul of the scaled integers (no float anywhere), then one rounding."""
    M, N, K = shape
    A = inputs.uniform((M, K), 31, "f16")
    B = inputs.uniform((K, N), 32, "f16")
    Ai = (A.view(np.float16).astype(np.float64) * 2.0 ** 24).astype(np.int64)
    Bi = (B.view(np.float16).astype(np.float64) * 2.0 ** 24).astype(np.int64)
    assert np.array_equal(Ai.astype(np.float64) * 2.0 ** -24, A.view(np.float16).astype(np.float64))
    S = Ai @ Bi                                  # |S| < 2^48 * K < 2^63
    exact = np.array([[float(int(v)) for v in row] for row in S]) * 2.0 ** -48
    C = oracle.gemm_f64(A, B, "f16")
    absdot = np.abs(Ai).astype(np.float64) @ np.abs(Bi).astype(np.float64) * 2.0 ** -48
    assert np.all(np.abs(C - exact) <= K * 2.0 ** -52 * absdot + 1e-300)


# ---------------------------------------------------------------- closed forms
def test_all_ones_gives_K():
    for (M, N, K) in [(5, 7, 9), (1, 1, 1), (33, 17, 129)]:
        A = inputs.from_values(np.ones((M, K)), "bf16")
        B = inputs.from_values(np.ones((K, N)), "bf16")
        assert np.all(oracle.gemm_f64(A, B, "bf16") == K)


def test_identity_and_permutation():
    n = 24
    B = inputs.uniform((n, n), 41, "f16")
    Bd = B.view(np.float16).astype(np.float64)
    I = inputs.from_values(np.eye(n), "f16")
    assert np.array_equal(oracle.gemm_f64(I, B, "f16"), Bd)
    perm = np.random.Generator(np.random.PCG64(42)).permutation(n)
    P = inputs.from_values(np.eye(n)[perm], "f16")
    assert np.array_equal(oracle.gemm_f64(P, B, "f16"), Bd[perm])
    # right identity: A . I = A
    A = inputs.uniform((9, n), 43, "f16")
    assert np.array_equal(oracle.gemm_f64(A, I, "f16"), A.view(np.float16).astype(np.float64))


def test_rank_one_outer_product():
    M, N, K = 6, 5, 7
    u = inputs.ints((M, 1), 51, "f16", -3, 3).view(np.float16).astype(np.float64)[:, 0]
    v = inputs.ints((1, N), 52, "f16", -3, 3).view(np.float16).astype(np.float64)[0]
    Ad = np.zeros((M, K))
    Ad[:, 4] = u
    Bd = np.zeros((K, N))
    Bd[4, :] = v
    C = oracle.gemm_f64(inputs.from_values(Ad, "f16"), inputs.from_values(Bd, "f16"), "f16")
    assert np.array_equal(C, np.outer(u, v))


def test_integer_fixture_is_exact_and_rows_mode_agrees():
    A = inputs.ints((64, 256), 111, "f16")
    B = inputs.ints((256, 48), 112, "f16")
    Ai = A.view(np.float16).astype(np.int64)
    Bi = B.view(np.float16).astype(np.int64)
    C = oracle.gemm_f64(A, B, "f16", threads=3)
    assert np.array_equal(C, (Ai @ Bi).astype(np.float64))
    rows = [0, 5, 63, 17]
    Cr = oracle.gemm_rows_f64(A, B, rows, "f16", threads=2)
    assert np.array_equal(Cr, C[rows])


def test_leading_dimensions_and_threads_do_not_change_result():
    A = inputs.uniform((37, 41), 61, "f16")
    B = inputs.uniform((41, 29), 62, "f16")
    C1 = oracle.gemm_f64(A, B, "f16", threads=1)
    Ap = inputs.padded(A, 48)[:, :41]     # strided view, NaN in the padding
    Bp = inputs.padded(B, 40)[:, :29]
    C2 = oracle.gemm_f64(Ap, Bp, "f16", threads=5)
    assert np.array_equal(C1, C2)


def test_zero_K_gives_zero_matrix():
    A = np.zeros((3, 0), dtype=np.uint16)
    B = np.zeros((0, 4), dtype=np.uint16)
    C = oracle.gemm_f64(A, B, "f16")
    assert C.shape == (3, 4) and np.all(C == 0)


# ---------------------------------------------------------------- comparison rule
def test_bound_rule():
    r = np.array([0.0, 1.0, 100.0, -3.0])
    b32 = oracle.bound(4096, "f32", r)
    assert np.all(b32 == 4096 * 2.0 ** -20)
    b16 = oracle.bound(4096, "bf16", r)
    assert b16[2] == 0.5 + 4096 * 2.0 ** -20
    res = oracle.compare(r + 0.001, r, 4096, "f32")
    assert res["ok"] and res["n_bad"] == 0
    res = oracle.compare(r + 0.01, r, 4096, "f32")
    assert not res["ok"] and res["n_bad"] == 4
    nanres = oracle.compare(np.array([np.nan]), np.array([1.0]), 16, "f32")
    assert not nanres["ok"]
