"""GPU parity of the general entry point gemm_run_ex against the CPU oracle:
column-major B (the TN layout) and the fused epilogue
act(alpha*A.B + beta*C_old + bias).

Bars (written in each test):
* exact fixtures (integers, multiples of 0.25, power-of-two alpha/beta,
  integer bias): every element equals round_to(out_fmt, oracle), bit for bit;
* random inputs, plain epilogue: the plain bound |y - r| <= K*2^-20 (+ one
  ulp for fp16/bf16 output);
* random inputs, general epilogue: oracle.bound_ex, i.e. |alpha|*K*2^-20 plus
  four fp32 roundings of the largest term plus one ulp of a half output;
* column-major B gives the same bits as row-major B holding the same matrix
  (same MFMA operands in the same order);
* beta == 0 never reads C (NaN poison in C stays out of the result);
* memory outside the M x N region of C is never written.
"""
import numpy as np
import pytest

import oracle
from dense_half_precision_tiled_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from tests.gpu_helpers import DTYPES, assert_bound, assert_exact, encode_out, law_for, run  # noqa: E402


@pytest.fixture(scope="module")
def G():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from dense_half_precision_tiled_amd import gemm
    gemm.load()      # raises if the library is missing: no fallback
    return gemm


def _t(B):
    return np.ascontiguousarray(B.T)


def assert_bound_ex(y, r, K, out_fmt, what="", **kw):
    res = oracle.compare_ex(y, r, K, out_fmt, **kw)
    assert res["ok"], "%s: %d elements outside the bound; max_abs %.3g, worst/bound %.3g" % (
        what, res["n_bad"], res["max_abs"], res["worst_ratio"])
    return res


# ------------------------------------------------------------ column-major B
SMALL = [(1, 1, 1), (2, 2, 3), (3, 5, 7), (8, 8, 8), (1, 300, 17), (300, 1, 17), (17, 65, 19),
         (31, 29, 37), (73, 61, 67), (129, 131, 65), (64, 64, 1), (255, 257, 129), (256, 256, 64)]


@pytest.mark.parametrize("code", [0, 1, 2, 3])
def test_col_major_random_small_shapes(G, code):
    fmt, out = DTYPES[code]
    for i, (M, N, K) in enumerate(SMALL):
        A = law_for(fmt)((M, K), 3000 + i, fmt)
        B = law_for(fmt)((K, N), 4000 + i, fmt)
        y = run(G, A, _t(B), code, layout=G.GEMM_B_COL_MAJOR)
        assert_bound(y, oracle.gemm_ex_f64(A, _t(B), fmt, b_layout="col"), K, out,
                     "col-major %s" % ((M, N, K),))


@pytest.mark.parametrize("code", [0, 1, 2, 3])
@pytest.mark.parametrize("shape", [(512, 512, 512), (257, 263, 251), (1024, 768, 640), (64, 1000, 2048),
                                   (300, 7, 130)])
def test_col_major_quarter_grid_bit_exact(G, code, shape):
    M, N, K = shape
    fmt, out = DTYPES[code]
    A = inputs.quarter((M, K), 171, fmt)
    Bt = inputs.quarter((N, K), 172, fmt)
    y = run(G, A, Bt, code, layout=G.GEMM_B_COL_MAJOR)
    assert_exact(y, oracle.gemm_ex_f64(A, Bt, fmt, b_layout="col"), out, "col-major quarter %s" % (shape,))


@pytest.mark.parametrize("code", [0, 3])
@pytest.mark.parametrize("shape", [(512, 512, 512), (300, 264, 200), (129, 136, 67), (256, 256, 4096)])
def test_col_major_equals_row_major_bitwise(G, code, shape):
    """Row-major B and its column-major copy feed the MFMAs identical operands
    in the same k order: identical output bits."""
    M, N, K = shape
    fmt, out = DTYPES[code]
    A = law_for(fmt)((M, K), 181, fmt)
    B = law_for(fmt)((K, N), 182, fmt)
    y_nn = run(G, A, B, code)
    y_tn = run(G, A, _t(B), code, layout=G.GEMM_B_COL_MAJOR)
    assert np.array_equal(y_nn, y_tn)


def _fd2_instances(G):
    from tests.gpu_helpers import instances16
    return [i for i in instances16(G) if "_fd1" not in G.gemm_instance_name(i)]


RAGGED = [(129, 131, 67), (300, 260, 130), (1, 513, 65), (255, 8, 200), (8, 1031, 63),
          (257, 392, 1), (520, 512, 576), (300, 7, 130), (256, 250, 64)]


def test_col_major_every_instance_on_ragged_shapes(G):
    for (M, N, K) in RAGGED:
        A = inputs.uniform((M, K), M + N, "f16")
        Bt = inputs.uniform((N, K), M + K, "f16")
        r = oracle.gemm_ex_f64(A, Bt, "f16", b_layout="col")
        for i in _fd2_instances(G):
            name = G.gemm_instance_name(i)
            whole = M % 256 == 0 and N % 256 == 0 and K % 64 == 0 if "256x" in name else \
                M % 128 == 0 and N % 128 == 0 and K % 64 == 0
            whole_tile_instance = not name.endswith(("_clamp", "_masked"))
            expect = G.GEMM_ERR_INSTANCE if whole_tile_instance and not whole else 0
            print("col-major", name, (M, N, K), flush=True)
            y = run(G, A, Bt, 1, instance=i, expect=expect, layout=G.GEMM_B_COL_MAJOR)
            if expect == 0:
                assert_bound(y, r, K, "f16", "%s %s" % (name, (M, N, K)))


@pytest.mark.parametrize("code", [0, 3])
def test_col_major_misaligned_and_padded_strides(G, code):
    fmt, out = DTYPES[code]
    M, N, K = 300, 263, 200
    A = law_for(fmt)((M, K), 191, fmt)
    Bt = law_for(fmt)((N, K), 192, fmt)
    r = oracle.gemm_ex_f64(A, Bt, fmt, b_layout="col")
    y = run(G, A, Bt, code, layout=G.GEMM_B_COL_MAJOR)
    assert_bound(y, r, K, out, "col-major packed")
    y2 = run(G, A, Bt, code, lda=K + 1, ldb=K + 3, ldc=N + 5, a_off=1, layout=G.GEMM_B_COL_MAJOR)
    assert np.array_equal(y, y2)
    y3 = run(G, A, Bt, code, lda=K + 64, ldb=K + 8, ldc=N + 16, layout=G.GEMM_B_COL_MAJOR)
    assert np.array_equal(y, y3)


# ------------------------------------------------------------ fused epilogue
def _cold(M, N, out, seed):
    """Old output values representable in the output format, and their bits."""
    rng = np.random.Generator(np.random.PCG64(seed))
    v = rng.uniform(-4, 4, (M, N))
    bits = encode_out(v, out)
    from tests.gpu_helpers import decode_out
    return decode_out(bits, out), bits


EPI_CASES = [
    # alpha, beta, bias, relu
    (1.0, 0.0, True, False),
    (1.0, 0.0, True, True),
    (0.5, 1.0, False, False),
    (-1.25, 0.75, True, True),
    (2.0, -1.0, True, False),
    (1.0, 1.0, False, True),
]


@pytest.mark.parametrize("code", [0, 1, 2, 3])
@pytest.mark.parametrize("layout", ["row", "col"])
def test_epilogue_random(G, code, layout):
    fmt, out = DTYPES[code]
    lay = G.GEMM_B_COL_MAJOR if layout == "col" else G.GEMM_B_ROW_MAJOR
    for n, (M, N, K) in enumerate([(129, 136, 67), (256, 256, 256), (300, 264, 130), (7, 9, 5)]):
        A = law_for(fmt)((M, K), 500 + n, fmt)
        B = law_for(fmt)((K, N), 600 + n, fmt)
        Bs = _t(B) if layout == "col" else B
        dot = oracle.gemm_f64(A, B, fmt)
        for c, (alpha, beta, use_bias, relu) in enumerate(EPI_CASES):
            cold, cbits = _cold(M, N, out, 700 + 10 * n + c)
            bias = np.random.Generator(np.random.PCG64(800 + c)).uniform(-2, 2, N) if use_bias else None
            bias32 = None if bias is None else bias.astype(np.float32).astype(np.float64)
            y = run(G, A, Bs, code, layout=lay, alpha=alpha, beta=beta, bias=bias, relu=int(relu),
                    c_init=cbits)
            r = oracle.gemm_ex_f64(A, Bs, fmt, b_layout=layout, alpha=alpha, beta=beta, C_old=cold,
                                   bias=bias32, relu=relu)
            assert_bound_ex(y, r, K, out, "epi %s %s %s" % (layout, (M, N, K), EPI_CASES[c]),
                            alpha=alpha, beta=beta, C_old=cold, bias=bias32, dot=dot)


@pytest.mark.parametrize("code", [0, 1, 2, 3])
def test_epilogue_integer_fixture_bit_exact(G, code):
    """Integer A, B, C_old and bias with alpha = 2, beta = -1: every value,
    including the fp32 epilogue's intermediates, is an exact small integer."""
    fmt, out = DTYPES[code]
    M, N, K = 300, 264, 130
    A = inputs.ints((M, K), 901, fmt)
    B = inputs.ints((K, N), 902, fmt)
    rng = np.random.Generator(np.random.PCG64(903))
    cold = rng.integers(-50, 51, (M, N)).astype(np.float64)
    bias = rng.integers(-20, 21, N).astype(np.float64)
    for lay, Bs, name in ((G.GEMM_B_ROW_MAJOR, B, "row"), (G.GEMM_B_COL_MAJOR, _t(B), "col")):
        y = run(G, A, Bs, code, layout=lay, alpha=2.0, beta=-1.0, bias=bias, relu=1,
                c_init=encode_out(cold, out))
        r = oracle.gemm_ex_f64(A, Bs, fmt, b_layout=name, alpha=2.0, beta=-1.0, C_old=cold, bias=bias,
                               relu=True)
        assert_exact(y, r, out, "integer epilogue %s" % name)


def test_beta_zero_never_reads_C(G):
    """C starts as NaN poison; with beta == 0 the result is finite."""
    M, N, K = 256, 264, 128
    A = inputs.uniform((M, K), 911, "f16")
    B = inputs.uniform((K, N), 912, "f16")
    bias = np.linspace(-1, 1, N)
    for code in (0, 1):
        y = run(G, A, B, code, layout=G.GEMM_B_ROW_MAJOR, alpha=1.5, beta=0.0, bias=bias, relu=0)
        assert np.all(np.isfinite(y))
        r = oracle.gemm_ex_f64(A, B, "f16", alpha=1.5, bias=bias.astype(np.float32).astype(np.float64))
        assert_bound_ex(y, r, K, DTYPES[code][1], "beta 0", alpha=1.5,
                        bias=bias, dot=oracle.gemm_f64(A, B, "f16"))


def test_plain_form_through_ex_is_gemm_run_bitwise(G):
    for code, (M, N, K) in ((3, (512, 512, 512)), (1, (300, 264, 130)), (0, (100, 7, 33))):
        fmt, out = DTYPES[code]
        A = law_for(fmt)((M, K), 921, fmt)
        B = law_for(fmt)((K, N), 922, fmt)
        assert np.array_equal(run(G, A, B, code), run(G, A, B, code, layout=G.GEMM_B_ROW_MAJOR))


def test_zero_K_general_form(G):
    M, N = 5, 7
    A = np.zeros((M, 0), dtype=np.uint16)
    B = np.zeros((0, N), dtype=np.uint16)
    cold = np.arange(M * N, dtype=np.float64).reshape(M, N) - 17.0
    bias = np.arange(N, dtype=np.float64) - 3.0
    for code in (0, 1, 3):
        out = DTYPES[code][1]
        y = run(G, A, B, code, lda=1, ldc=9, layout=G.GEMM_B_ROW_MAJOR, alpha=3.0, beta=0.5, bias=bias,
                relu=1, c_init=encode_out(cold, out))
        assert np.array_equal(y, np.maximum(0.5 * cold + bias[None, :], 0.0))


def test_epilogue_every_instance(G):
    M, N, K = 256, 256, 192
    A = inputs.quarter((M, K), 931, "bf16")
    B = inputs.quarter((K, N), 932, "bf16")
    cold = np.random.Generator(np.random.PCG64(933)).integers(-8, 9, (M, N)).astype(np.float64)
    bias = np.arange(N, dtype=np.float64) * 0.25 - 30.0
    r = oracle.gemm_ex_f64(A, B, "bf16", alpha=0.5, beta=2.0, C_old=cold, bias=bias, relu=True)
    for i in _fd2_instances(G):
        print("epilogue", G.gemm_instance_name(i), flush=True)
        y = run(G, A, B, 2, instance=i, layout=G.GEMM_B_ROW_MAJOR, alpha=0.5, beta=2.0, bias=bias, relu=1,
                c_init=encode_out(cold, "f32"))
        assert_exact(y, r, "f32", G.gemm_instance_name(i))


# ------------------------------------------------------------ full size
def _rows(M, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.array(sorted({0, 1, 255, 256, M - 256, M - 1} | set(rng.integers(0, M, 10).tolist())))


@pytest.mark.parametrize("n", [4096, 8192])
def test_full_size_col_major_bf16(G, n):
    """The bf16 workloads with B stored column-major: sampled oracle rows and
    bitwise equality with the row-major call."""
    A = inputs.normal((n, n), 100 * (3 if n == 4096 else 4) + 1, "bf16")
    B = inputs.normal((n, n), 100 * (3 if n == 4096 else 4) + 2, "bf16")
    print("full-size col-major", n, flush=True)
    y_tn = run(G, A, _t(B), 3, layout=G.GEMM_B_COL_MAJOR)
    rows = _rows(n, 41)
    assert_bound(y_tn[rows], oracle.gemm_rows_f64(A, B, rows, "bf16"), n, "bf16", "col-major %d" % n)
    y_nn = run(G, A, B, 3)
    assert np.array_equal(y_tn, y_nn)


def test_full_size_epilogue_4096(G):
    n = 4096
    A = inputs.normal((n, n), 301, "bf16")
    B = inputs.normal((n, n), 302, "bf16")
    bias = np.random.Generator(np.random.PCG64(42)).normal(size=n)
    bias32 = bias.astype(np.float32).astype(np.float64)
    print("full-size epilogue", n, flush=True)
    y = run(G, A, _t(B), 3, layout=G.GEMM_B_COL_MAJOR, alpha=0.5, beta=0.0, bias=bias, relu=1)
    rows = _rows(n, 43)
    r = oracle.gemm_ex_f64(A, _t(B), "bf16", b_layout="col", alpha=0.5, bias=bias32, relu=True, rows=rows)
    dot = oracle.gemm_rows_f64(A, B, rows, "bf16")
    assert_bound_ex(y[rows], r, n, "bf16", "epilogue 4096", alpha=0.5, bias=bias32, dot=dot)
    assert np.all(y >= 0)
