"""GPU parity of the 8-bit float inputs (E4M3 and E5M2 of the OCP 8-bit
floating point specification; B row-major through gemm_run, or column-major
through gemm_run_ex), through the C ABI, against the CPU oracle.

Bars (as for the 16-bit inputs):
* exact fixtures (the page's worked example, small integers, multiples of
  0.25): every element equals round_to(out_fmt, oracle), bit for bit;
* random inputs with magnitudes in [0.5, 2] (random signs): every product
  lies in [2^-2, 2^2] and carries at most 8 significant bits, so no bit of
  any product falls below the 8-bit MFMA's alignment window (13 binades
  under the largest product of its group of 8 consecutive k) and the plain
  bound applies with no device-derived term: |y - r| <= K * 2^-20 (fp32
  output) or ulp_fmt(r) + K * 2^-20 (fp16/bf16 output), at every element,
  up to the full 8192^3 workload;
* random N(0, 1) inputs rounded to the 8-bit format: the same bound plus
  the alignment loss oracle.align_bound8, an envelope read off the device
  (test_mfma_f8_alignment_model), at every element;
* the 8-bit instances (three tile sizes; whole, clamped or masked edges)
  give identical bits where they apply, and so do the two B layouts;
* memory outside the M x N region of C is never written (checked by run()).
"""
import json
import os

import numpy as np
import pytest

import oracle
from dense_half_precision_tiled_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from tests.gpu_helpers import DTYPES, assert_bound, assert_exact, run  # noqa: E402

CODES8 = [4, 5, 6, 7, 8, 9]


@pytest.fixture(scope="module")
def G():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from dense_half_precision_tiled_amd import gemm
    gemm.load()      # raises if the library is missing: no fallback
    return gemm


def _run_tn(G, A, B, code, **kw):
    """A (M x K) and B (K x N) as bit patterns; B is passed column-major."""
    return run(G, A, np.ascontiguousarray(B.T), code, layout=G.GEMM_B_COL_MAJOR, **kw)


def _run_lay(G, A, B, code, lay, **kw):
    """B row-major through gemm_run ("row"), or column-major ("col")."""
    if lay == "col":
        return _run_tn(G, A, B, code, **kw)
    return run(G, A, B, code, **kw)


def _oracle(A, B, fmt):
    return oracle.gemm_ex_f64(A, np.ascontiguousarray(B.T), fmt, b_layout="col")


def _extra(A, B, fmt, rows=None):
    return oracle.align_bound8(A, B, fmt, rows=rows)


@pytest.mark.parametrize("lay", ["row", "col"])
@pytest.mark.parametrize("code", CODES8)
def test_worked_example(G, code, lay):
    with open(os.path.join(os.path.dirname(__file__), "golden", "worked_example_2x3x2.json")) as f:
        g = json.load(f)
    fmt, out = DTYPES[code]
    y = _run_lay(G, inputs.from_values(g["A"], fmt), inputs.from_values(g["B"], fmt), code, lay)
    assert y.tolist() == g["C"]


@pytest.mark.parametrize("lay", ["row", "col"])
@pytest.mark.parametrize("code", CODES8)
@pytest.mark.parametrize("shape", [(256, 256, 256), (512, 768, 1024), (257, 263, 251), (300, 520, 4099),
                                   (64, 1000, 2048), (1, 1, 1), (5, 3, 15), (33, 17, 129), (130, 48, 300)])
def test_integer_and_quarter_grid_bit_exact(G, code, shape, lay):
    """Integers in {-2..2} and multiples of 0.25 in [-2, 2] are exact in both
    8-bit formats; every partial sum is exact in fp32, so each output is the
    correctly rounded exact value."""
    M, N, K = shape
    fmt, out = DTYPES[code]
    for law, s in ((inputs.ints, 300), (inputs.quarter, 310)):
        A = law((M, K), s + code, fmt)
        B = law((K, N), s + 1 + code, fmt)
        print("8-bit exact", code, shape, lay, law.__name__, flush=True)
        assert_exact(_run_lay(G, A, B, code, lay), _oracle(A, B, fmt), out,
                     "%s %s %s %s" % (code, shape, lay, law.__name__))


@pytest.mark.parametrize("lay", ["row", "col"])
@pytest.mark.parametrize("code", CODES8)
@pytest.mark.parametrize("shape", [(1024, 1024, 1024), (4096, 2048, 512), (384, 640, 896),
                                   (1000, 1001, 777), (96, 50, 4160), (2, 300, 7), (700, 528, 333)])
def test_random_inputs_within_bound(G, code, shape, lay):
    M, N, K = shape
    fmt, out = DTYPES[code]
    A = inputs.normal((M, K), 400 + code, fmt)
    B = inputs.normal((K, N), 401 + code, fmt)
    print("8-bit random", code, shape, lay, flush=True)
    y = _run_lay(G, A, B, code, lay)
    res = assert_bound(y, _oracle(A, B, fmt), K, out, "%s %s" % (code, shape), extra=_extra(A, B, fmt))
    print("8-bit random", code, shape, "max_abs %.3g worst err/bound %.4f" % (res["max_abs"], res["worst_ratio"]),
          flush=True)


@pytest.mark.parametrize("lay", ["row", "col"])
@pytest.mark.parametrize("code", CODES8)
@pytest.mark.parametrize("shape", [(1024, 1024, 1024), (1000, 1001, 777), (96, 50, 4160), (300, 520, 4099)])
def test_narrow_range_meets_the_plain_bound(G, code, shape, lay):
    M, N, K = shape
    fmt, out = DTYPES[code]
    A = inputs.signed_magnitude((M, K), 450 + code, fmt)
    B = inputs.signed_magnitude((K, N), 451 + code, fmt)
    print("8-bit narrow range", code, shape, lay, flush=True)
    y = _run_lay(G, A, B, code, lay)
    res = assert_bound(y, _oracle(A, B, fmt), K, out, "%s %s" % (code, shape))
    print("8-bit narrow range", code, shape, "worst err/bound %.4f" % res["worst_ratio"], flush=True)


@pytest.mark.parametrize("name,fmt,code", [("e4m3_8192", "e4m3", 6), ("e5m2_8192", "e5m2", 7)])
def test_narrow_range_full_size(G, name, fmt, code):
    """The 8-bit workload's shape (8192^3, B column-major) on narrow-range
    data: every element within the plain bound."""
    n = 8192
    out = DTYPES[code][1]
    A = inputs.signed_magnitude((n, n), 460, fmt)
    B = inputs.signed_magnitude((n, n), 461, fmt)
    print("8-bit narrow range full size", name, code, flush=True)
    y = _run_tn(G, A, B, code)
    res = assert_bound(y, _oracle(A, B, fmt), n, out, name)
    print(name, "narrow range, full matrix, worst err/bound %.4f" % res["worst_ratio"], flush=True)


@pytest.mark.parametrize("lay", ["row", "col"])
@pytest.mark.parametrize("code", [4, 9])
def test_odd_leading_dimensions_and_offsets(G, code, lay):
    """1-byte elements: rows may start at any byte (odd lda, ldb, base)."""
    M, N, K = 333, 528, 1111
    fmt, out = DTYPES[code]
    A = inputs.normal((M, K), 500, fmt)
    B = inputs.normal((K, N), 501, fmt)
    r = _oracle(A, B, fmt)
    x = _extra(A, B, fmt)
    ys = []
    ldb0 = K if lay == "col" else N
    for lda, ldb, a_off in ((K + 1, ldb0 + 3, 1), (K + 5, ldb0, 3), (K, ldb0 + 7, 0), (K + 16, ldb0 + 16, 15)):
        print("8-bit strides", code, lay, lda, ldb, a_off, flush=True)
        y = _run_lay(G, A, B, code, lay, lda=lda, ldb=ldb, ldc=N + 5, a_off=a_off)
        assert_bound(y, r, K, out, "lda %d ldb %d off %d" % (lda, ldb, a_off), extra=x)
        ys.append(y)
    for y in ys[1:]:                     # strides and offsets move data only
        assert np.array_equal(y, ys[0], equal_nan=True)


def test_instances_agree_bitwise(G):
    """Tile size, edge handling and the B layout move data only: every 8-bit
    instance, with B row-major and column-major, gives identical bits on a
    shape they all run."""
    M, N, K = 512, 512, 1024
    ids = [i for i in range(G.gemm_num_instances()) if G.gemm_instance_name(i).startswith("dl8_")]
    assert len(ids) == 8
    for code in (4, 8):
        fmt, out = DTYPES[code]
        A = inputs.normal((M, K), 600, fmt)
        B = inputs.normal((K, N), 601, fmt)
        ys = []
        for i in ids:
            name = G.gemm_instance_name(i)
            for lay in ("row", "col"):
                print("8-bit instance", name, code, lay, flush=True)
                ys.append((name + " " + lay, _run_lay(G, A, B, code, lay, instance=i)))
        for name, y in ys[1:]:
            assert np.array_equal(y, ys[0][1], equal_nan=True), name
        assert_bound(ys[0][1], _oracle(A, B, fmt), K, out, extra=_extra(A, B, fmt))


@pytest.mark.parametrize("code", [4, 6, 8])
def test_general_form(G, code):
    M, N, K = 300, 264, 700
    fmt, out = DTYPES[code]
    A = inputs.normal((M, K), 700, fmt)
    B = inputs.normal((K, N), 701, fmt)
    Bs = np.ascontiguousarray(B.T)
    from tests.gpu_helpers import decode_out, encode_out
    cold = decode_out(encode_out(np.random.Generator(np.random.PCG64(702)).uniform(-4, 4, (M, N)), out), out)
    bias = np.random.Generator(np.random.PCG64(703)).uniform(-2, 2, N).astype(np.float32).astype(np.float64)
    for alpha, beta, b, relu in ((0.5, 0.0, None, 0), (-2.0, 1.0, bias, 1), (1.0, -0.5, bias, 0)):
        print("8-bit general", code, alpha, beta, b is not None, relu, flush=True)
        y = run(G, A, Bs, code, layout=G.GEMM_B_COL_MAJOR, alpha=alpha, beta=beta, bias=b, relu=relu,
                c_init=encode_out(cold, out))
        r = oracle.gemm_ex_f64(A, Bs, fmt, b_layout="col", alpha=alpha, beta=beta, C_old=cold, bias=b,
                               relu=bool(relu))
        dot = oracle.gemm_ex_f64(A, Bs, fmt, b_layout="col")
        res = oracle.compare_ex(y, r, K, out, alpha=alpha, beta=beta, C_old=cold, bias=b, dot=dot,
                                extra=_extra(A, B, fmt))
        assert res["ok"], res


def test_general_form_every_instance(G):
    """alpha, beta, bias and ReLU on every 8-bit instance and both B layouts
    (0.25-grid inputs: the result is exact), on whole tiles and on a ragged
    shape (N % 16 != 0: the row-major clamped kernels refuse it, the masked
    ones take it in both layouts)."""
    from tests.gpu_helpers import encode_out
    ids = [i for i in range(G.gemm_num_instances()) if G.gemm_instance_name(i).startswith("dl8_")]
    for (M, N, K) in ((512, 512, 1024), (300, 264, 700)):
        A = inputs.quarter((M, K), 901, "e5m2")
        B = inputs.quarter((K, N), 902, "e5m2")
        cold = np.random.Generator(np.random.PCG64(903)).integers(-8, 9, (M, N)).astype(np.float64)
        bias = np.arange(N, dtype=np.float64) * 0.25 - 30.0
        r = oracle.gemm_ex_f64(A, B, "e5m2", alpha=0.5, beta=2.0, C_old=cold, bias=bias, relu=True)
        for i in ids:
            name = G.gemm_instance_name(i)
            tile = int(name.split("_")[1].split("x")[0])
            for lay in ("row", "col"):
                if name.endswith("_masked"):
                    ok = True
                elif name.endswith("_clamp"):
                    ok = lay == "col" or N % 16 == 0
                else:
                    ok = M % tile == 0 and N % tile == 0 and K % 128 == 0
                print("8-bit epilogue", name, lay, (M, N, K), flush=True)
                Bs = np.ascontiguousarray(B.T) if lay == "col" else B
                y = run(G, A, Bs, 7, instance=i, layout=G.GEMM_B_COL_MAJOR if lay == "col" else G.GEMM_B_ROW_MAJOR,
                        alpha=0.5, beta=2.0, bias=bias, relu=1, c_init=encode_out(cold, "f32"),
                        expect=0 if ok else G.GEMM_ERR_INSTANCE)
                if ok:
                    assert_exact(y, r, "f32", "%s %s" % (name, lay))


def test_zero_K(G):
    """K == 0: the plain form writes zeros; the general form gives act(beta*C + bias)."""
    M, N = 70, 90
    A = np.zeros((M, 0), np.uint8)
    B = np.zeros((0, N), np.uint8)
    assert np.array_equal(_run_tn(G, A, B, 4), np.zeros((M, N)))
    from tests.gpu_helpers import encode_out
    y = run(G, A, np.zeros((N, 0), np.uint8), 4, layout=G.GEMM_B_COL_MAJOR, beta=2.0,
            c_init=encode_out(np.ones((M, N)), "f32"))
    assert np.array_equal(y, np.full((M, N), 2.0))


def test_torch_binding_with_float8_tensors(G):
    """gemm.gemm on torch float8 tensors with B as a transposed view."""
    M, N, K = 500, 384, 640
    A = inputs.normal((M, K), 800, "e4m3")
    B = inputs.normal((K, N), 801, "e4m3")
    tA = torch.from_numpy(A).cuda().view(torch.float8_e4m3fn)
    tBt = torch.from_numpy(np.ascontiguousarray(B.T)).cuda().view(torch.float8_e4m3fn)
    y = G.gemm(tA, tBt.t(), torch.float32)
    torch.cuda.synchronize()
    assert_bound(y.cpu().numpy().astype(np.float64), _oracle(A, B, "e4m3"), K, "f32",
                 extra=_extra(A, B, "e4m3"))
    y2 = G.gemm(tA, tBt.t().contiguous(), torch.float32)      # row-major B through gemm_run
    torch.cuda.synchronize()
    assert torch.equal(y, y2)


@pytest.mark.parametrize("name,lay", [("e4m3_8192", "col"), ("e5m2_8192", "col"), ("e4m3_8192", "row")])
def test_full_size_workloads(G, name, lay):
    """The 8-bit workloads at full size on N(0, 1) data: every element against
    the oracle, within the bound plus the alignment envelope."""
    A, B, w = inputs.workload_inputs(name)
    code = {("e4m3", "bf16"): 6, ("e5m2", "bf16"): 9}[(w["fmt"], w["out"])]
    print("full-size workload", name, lay, flush=True)
    y = _run_lay(G, A, B, code, lay)
    r = _oracle(A, B, w["fmt"])
    res = assert_bound(y, r, w["K"], w["out"], name, extra=_extra(A, B, w["fmt"]))
    print(name, lay, "full matrix, max_abs %.3g, worst err/bound %.4f" % (res["max_abs"], res["worst_ratio"]),
          flush=True)
