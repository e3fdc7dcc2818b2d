"""Pins for the oracle's 8-bit float inputs (no GPU): the E4M3 and E5M2
formats of the OCP 8-bit floating point specification (OFP8), the 8-bit float
the Ada tensor-core GEMM write-up names as its untested next step.

Each test checks the oracle against something other than itself: torch's own
float8 types, the identity between E5M2 and the top byte of an IEEE binary16,
the limits the OFP8 specification tabulates, exact rational arithmetic and
int64 matmuls."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from dense_half_precision_tiled_amd import inputs

torch = pytest.importorskip("torch")

TORCH_DT = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def _torch_decode(bits, fmt):
    return torch.from_numpy(np.ascontiguousarray(bits)).view(TORCH_DT[fmt]).to(torch.float64).numpy()


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_decode_all_codes_match_torch(fmt):
    codes = np.arange(256, dtype=np.uint8)
    ref = _torch_decode(codes, fmt)
    got = oracle.decode(codes, fmt)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])          # infinities included (E5M2)
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))


def test_e5m2_is_the_top_byte_of_binary16():
    """E5M2 keeps binary16's sign and exponent fields and the top two
    fraction bits, so code b means the fp16 pattern b << 8 (numpy's decoder)."""
    codes = np.arange(256, dtype=np.uint8)
    ref = (codes.astype(np.uint16) << 8).view(np.float16).astype(np.float64)
    got = oracle.decode(codes, "e5m2")
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])


def test_ofp8_limits():
    """The limits the OFP8 specification tabulates for both formats."""
    d = lambda b, f: float(oracle.decode(np.array([b], dtype=np.uint8), f)[0])
    # E4M3: no infinities; S.1111.111 is NaN, so the largest normal is 1.75 * 2^8
    assert d(0x7E, "e4m3") == 448.0 and d(0xFE, "e4m3") == -448.0
    assert d(0x08, "e4m3") == 2.0 ** -6                     # smallest normal
    assert d(0x07, "e4m3") == 0.875 * 2.0 ** -6             # largest subnormal
    assert d(0x01, "e4m3") == 2.0 ** -9                     # smallest subnormal
    assert d(0x38, "e4m3") == 1.0
    assert np.isnan(d(0x7F, "e4m3")) and np.isnan(d(0xFF, "e4m3"))
    assert d(0x78, "e4m3") == 256.0                         # exponent 15 still holds normals
    # E5M2: IEEE-style specials
    assert d(0x7B, "e5m2") == 57344.0                       # 1.75 * 2^15
    assert d(0x04, "e5m2") == 2.0 ** -14
    assert d(0x01, "e5m2") == 2.0 ** -16
    assert d(0x3C, "e5m2") == 1.0
    assert d(0x7C, "e5m2") == float("inf") and d(0xFC, "e5m2") == float("-inf")
    assert all(np.isnan(d(b, "e5m2")) for b in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF))
    for f in ("e4m3", "e5m2"):
        z = oracle.decode(np.array([0x80], dtype=np.uint8), f)
        assert z[0] == 0.0 and np.signbit(z[0])


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_brute_force_against_exact_rationals(fmt):
    rng = np.random.Generator(np.random.PCG64(41))
    for (M, N, K) in [(1, 1, 1), (3, 5, 7), (8, 8, 16), (5, 3, 33), (7, 9, 64)]:
        seed = int(rng.integers(1 << 30))
        A = inputs.normal((M, K), seed, fmt)
        B = inputs.normal((K, N), seed + 1, fmt)
        Ad, Bd = _torch_decode(A, fmt), _torch_decode(B, fmt)
        C = oracle.gemm_f64(A, B, fmt, threads=2)
        for i in range(M):
            for j in range(N):
                exact = sum((Fraction(float(Ad[i, k])) * Fraction(float(Bd[k, j])) for k in range(K)),
                            Fraction(0))
                # products are exact in fp64 and partial sums carry few bits: exact
                assert Fraction(C[i, j]) == exact, (fmt, M, N, K, i, j)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_integer_fixture_with_padded_rows_matches_int64_matmul(fmt):
    A = inputs.padded(inputs.ints((37, 300), 51, fmt), 320)[:, :300]      # NaN padding
    B = inputs.padded(inputs.ints((300, 29), 52, fmt), 40)[:, :29]
    exact = _torch_decode(A, fmt).astype(np.int64) @ _torch_decode(B, fmt).astype(np.int64)
    assert np.array_equal(oracle.gemm_f64(A, B, fmt, threads=3), exact.astype(np.float64))
    rows = np.array([0, 17, 36])
    assert np.array_equal(oracle.gemm_rows_f64(A, B, rows, fmt, threads=2), exact[rows].astype(np.float64))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_column_major_B_and_general_form(fmt):
    A = inputs.ints((9, 70), 61, fmt)
    B = inputs.ints((70, 11), 62, fmt)
    Bt = np.ascontiguousarray(B.T)
    exact = (_torch_decode(A, fmt).astype(np.int64) @ _torch_decode(B, fmt).astype(np.int64)).astype(np.float64)
    bias = np.linspace(-3, 3, 11)
    got = oracle.gemm_ex_f64(A, Bt, fmt, b_layout="col", alpha=0.5, bias=bias, relu=True)
    assert np.array_equal(got, np.maximum(0.5 * exact + bias[None, :], 0.0))


def test_8bit_inputs_are_uint8():
    with pytest.raises(TypeError):
        oracle.gemm_f64(np.zeros((2, 2), np.uint16), np.zeros((2, 2), np.uint16), "e4m3")


# ------------------------------------------------ the 8-bit MFMA alignment bound
def _mfma8_model(Ad, Bd):
    """The 8-bit MFMA's summation as the probe tests pin it, written out by
    brute force: per group of 8 consecutive k, each product is cut toward zero
    to a multiple of 2^(e - 13), 2^e the largest product of the group."""
    M, K = Ad.shape
    N = Bd.shape[1]
    out = np.zeros((M, N))
    for i in range(M):
        for j in range(N):
            total = 0.0
            for g0 in range(0, K, 8):
                p = [Ad[i, k] * Bd[k, j] for k in range(g0, min(g0 + 8, K))]
                big = max(abs(v) for v in p)
                if big == 0.0:
                    continue
                q = 2.0 ** (int(np.floor(np.log2(big))) - 13)
                total += sum(float(np.trunc(v / q)) * q for v in p)
            out[i, j] = total
    return out


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_align_bound_covers_the_truncation_model(fmt):
    rng = np.random.Generator(np.random.PCG64(91))
    for (M, N, K) in [(3, 4, 8), (5, 6, 64), (4, 3, 130), (2, 2, 9)]:
        # wide exponent spread so that truncation happens often
        A = inputs.from_values(rng.choice([-1, 1], (M, K)) * 2.0 ** rng.integers(-8, 4, (M, K)), fmt)
        B = inputs.from_values(rng.choice([-1, 1], (K, N)) * 2.0 ** rng.integers(-8, 4, (K, N)) * 1.5, fmt)
        Ad, Bd = _torch_decode(A, fmt), _torch_decode(B, fmt)
        exact = oracle.gemm_f64(A, B, fmt, threads=1)
        model = _mfma8_model(Ad, Bd)
        b = oracle.align_bound8(A, B, fmt)
        assert np.all(np.abs(model - exact) <= b), (fmt, M, N, K)
        assert np.any(model != exact)           # the spread did exercise the truncation
        # column-major B and row selection give the same bound
        bt = oracle.align_bound8(A, np.ascontiguousarray(B.T), fmt, b_layout="col", rows=[0, M - 1])
        assert np.array_equal(bt, b[[0, M - 1]])


def test_align_bound_is_reached_by_a_worst_case():
    """A group with one product 1 * 8 = 2^3 and seven products
    2^-9 * 0.46875 = 0.9375 * 2^-10, just under the 2^(3-13) grid: the model
    drops all seven, 6.5625 * 2^-10, against a bound of 7 * 2^-13 * 1 * 8 =
    7 * 2^-10 -- the bound is not loose by more than the grid step."""
    A = inputs.from_values(np.array([[1.0] + [2.0 ** -9] * 7]), "e4m3")
    B = inputs.from_values(np.array([[8.0]] + [[0.46875]] * 7), "e4m3")
    Ad, Bd = _torch_decode(A, "e4m3"), _torch_decode(B, "e4m3")
    assert Ad[0, 1] == 2.0 ** -9 and Bd[1, 0] == 0.46875        # exact in E4M3
    model = _mfma8_model(Ad, Bd)
    assert model[0, 0] == 8.0
    bound = oracle.align_bound8(A, B, "e4m3")[0, 0]
    assert bound == 7 * 2.0 ** -10
    err = abs(model[0, 0] - float((Ad @ Bd)[0, 0]))
    assert err == 7 * 0.9375 * 2.0 ** -10 and err / bound == 0.9375
