"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars (written in each test):
* exact fixtures (small integers, multiples of 0.25, unique-valued identity
  products): every element equals round_to(out_fmt, oracle), bit for bit
  (+0 and -0 compare equal);
* random inputs: |y - r| <= K * 2^-20 (fp32 output) or
  ulp_fmt(r) + K * 2^-20 (fp16/bf16 output) for every checked element;
* full-size shapes: every output of the full matrix against the oracle
  (random inputs at the bound; the exact 8192^3 fixtures of
  test_gpu_full_exact.py bit for bit);
* memory outside the M x N region of C (row padding and guard bands) is
  never written.
"""
import os

import numpy as np
import pytest

import oracle
from dense_half_precision_tiled_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from tests.gpu_helpers import DTYPES, assert_bound, assert_exact, family, instances16, law_for, run  # noqa: E402


@pytest.fixture(scope="module")
def G():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from dense_half_precision_tiled_amd import gemm
    gemm.load()      # raises if the library is missing: no fallback
    return gemm


# ------------------------------------------------------------ exact fixtures
@pytest.mark.parametrize("code", [0, 1, 2, 3])
def test_worked_example(G, code):
    import json
    with open(os.path.join(os.path.dirname(__file__), "golden", "worked_example_2x3x2.json")) as f:
        g = json.load(f)
    fmt, out = DTYPES[code]
    y = run(G, inputs.from_values(g["A"], fmt), inputs.from_values(g["B"], fmt), code)
    assert y.tolist() == g["C"]


def test_integer_fixture_256_bit_exact(G):
    """fp16 integers in {-2..2}, 256^3, fp32 output: |C| <= 1024, exact."""
    A, B, w = inputs.workload_inputs("f16_256_int")
    y = run(G, A, B, 0)
    r = oracle.gemm_f64(A, B, "f16")
    assert np.array_equal(y, r)


@pytest.mark.parametrize("code", [0, 1, 2, 3])
@pytest.mark.parametrize("shape", [(512, 512, 512), (257, 263, 251), (1024, 768, 640),
                                   (64, 1000, 2048)])
def test_quarter_grid_bit_exact(G, code, shape):
    M, N, K = shape
    fmt, out = DTYPES[code]
    A = inputs.quarter((M, K), 71, fmt)
    B = inputs.quarter((K, N), 72, fmt)
    y = run(G, A, B, code)
    assert_exact(y, oracle.gemm_f64(A, B, fmt), out, "quarter %s" % (shape,))


@pytest.mark.parametrize("code", [0, 3])
def test_unique_value_ownership(G, code):
    """Identity times a matrix of distinct integers returns that matrix: every
    output element lands where it belongs (fragment and accumulator maps)."""
    fmt, out = DTYPES[code]
    n = 256
    U = (np.arange(n * n) % 251 - 125).reshape(n, n).astype(np.float64)    # distinct per row
    U[:, ::7] += 0.5
    I = np.eye(n)
    y = run(G, inputs.from_values(I, fmt), inputs.from_values(U, fmt), code)
    assert np.array_equal(y, U)
    y = run(G, inputs.from_values(U, fmt), inputs.from_values(I, fmt), code)
    assert np.array_equal(y, U)
    P = np.eye(n)[np.random.Generator(np.random.PCG64(3)).permutation(n)]
    y = run(G, inputs.from_values(P, fmt), inputs.from_values(U, fmt), code)
    assert np.array_equal(y, P @ U)


# ------------------------------------------------------------ random, small
SMALL = [(1, 1, 1), (2, 2, 3), (3, 5, 7), (8, 8, 8), (1, 300, 17), (300, 1, 17), (17, 65, 19),
         (31, 29, 37), (73, 61, 67), (129, 131, 65), (64, 64, 1), (255, 257, 129)]


@pytest.mark.parametrize("code", [0, 1, 2, 3])
def test_random_small_shapes(G, code):
    fmt, out = DTYPES[code]
    for i, (M, N, K) in enumerate(SMALL):
        A = law_for(fmt)((M, K), 1000 + i, fmt)
        B = law_for(fmt)((K, N), 2000 + i, fmt)
        y = run(G, A, B, code)
        assert_bound(y, oracle.gemm_f64(A, B, fmt), K, out, "shape %s" % ((M, N, K),))


def test_config_256_uniform(G):
    A, B, w = inputs.workload_inputs("f16_256")
    y = run(G, A, B, 0)
    assert_bound(y, oracle.gemm_f64(A, B, "f16"), w["K"], "f32", "256^3")


@pytest.mark.parametrize("code", [0, 3])
def test_padded_leading_dimensions(G, code):
    fmt, out = DTYPES[code]
    M, N, K = 300, 260, 200
    A = law_for(fmt)((M, K), 81, fmt)
    B = law_for(fmt)((K, N), 82, fmt)
    r = oracle.gemm_f64(A, B, fmt)
    y = run(G, A, B, code, lda=K + 8, ldb=N + 24, ldc=N + 40)
    assert_bound(y, r, K, out, "padded ld")
    # 2-byte aligned rows and base pointer: unaligned 16-byte loads, same bits
    y2 = run(G, A, B, code, lda=K + 1, ldb=N + 3, ldc=N + 1, a_off=1)
    assert_bound(y2, r, K, out, "misaligned")
    assert np.array_equal(y, y2)


@pytest.mark.parametrize("code", [0, 3])
def test_aligned_tile_multiples_with_padding(G, code):
    """Tile-multiple shapes with 16-byte-aligned padded strides (vector path)."""
    fmt, out = DTYPES[code]
    M, N, K = 512, 256, 320
    A = law_for(fmt)((M, K), 91, fmt)
    B = law_for(fmt)((K, N), 92, fmt)
    r = oracle.gemm_f64(A, B, fmt)
    y = run(G, A, B, code, lda=K + 64, ldb=N + 8, ldc=N + 16)
    assert_bound(y, r, K, out, "aligned padded")


def test_zero_K_writes_zeros(G):
    for code in (0, 1, 3):
        A = np.zeros((5, 0), dtype=np.uint16)
        B = np.zeros((0, 7), dtype=np.uint16)
        y = run(G, A, B, code, lda=1, ldc=9)
        assert np.all(y == 0) and y.shape == (5, 7)


def test_empty_output_leaves_C_untouched(G):
    A = inputs.uniform((0, 5), 1, "f16")
    B = inputs.uniform((5, 4), 2, "f16")
    y = run(G, A, B, 0)
    assert y.shape == (0, 4)


def test_instances_agree_bitwise(G):
    """Instances of one kernel family that differ only in tile size, edge
    masking or visit order do the same per-element arithmetic in the same
    order: identical bits.  The two families (dl: waves split the tile; ks:
    waves split K and sum four partial tiles) add the k-steps in different
    orders, so across families only the bound applies."""
    for code in (0, 3):
        fmt, out = DTYPES[code]
        A = law_for(fmt)((512, 512), 101, fmt)
        B = law_for(fmt)((512, 512), 102, fmt)
        r = oracle.gemm_f64(A, B, fmt)
        first = {}
        for i in instances16(G):
            name = G.gemm_instance_name(i)
            print("instance", name, code, flush=True)
            y = run(G, A, B, code, instance=i)
            fam = family(name)
            if fam in first:
                assert np.array_equal(first[fam], y), name
            else:
                first[fam] = y
                assert_bound(y, r, 512, out, "instances " + name)
        assert set(first) == {"dl", "ks"}


def test_c_row_alignment_picks_the_store_form_not_the_result(G):
    """A whole-tile shape runs the whole-tile kernel (non-temporal stores of
    64-column row pieces) when C's rows start on 64-byte boundaries and the
    clamped kernel otherwise (a padded ldc, or C one element off): the same
    per-element arithmetic, so the same bits, and the padding and guard
    bands stay untouched (checked by run())."""
    # 2048 x 2048 runs 128x128 tiles, 4096 x 4096 the 256x256 tile: both pair
    # their 32-column blocks into row pieces
    for (M, N, K) in ((2048, 2048, 256), (4096, 4096, 128)):
        for code in (0, 1, 3):
            fmt, out = DTYPES[code]
            print("row alignment", (M, N, K), code, flush=True)
            A = law_for(fmt)((M, K), 111, fmt)
            B = law_for(fmt)((K, N), 112, fmt)
            y0 = run(G, A, B, code)                      # ldc = N: aligned rows
            y1 = run(G, A, B, code, ldc=N + 4)           # rows off 64-byte boundaries
            y2 = run(G, A, B, code, c_off=1)             # C itself 2 or 4 bytes off
            assert np.array_equal(y0, y1) and np.array_equal(y0, y2), (M, code)
            if M == 2048:
                assert_bound(y0, oracle.gemm_f64(A, B, fmt), K, out, "row alignment %d" % code)


def test_k_split_reduction_is_deterministic(G):
    """The four partial tiles are added in a fixed order: repeated calls give
    the same bits (whole tiles with an even slice count; clamped edges with an
    odd count and a partial slice)."""
    n = G.gemm_num_instances()
    ks = {G.gemm_instance_name(i): i for i in range(n) if G.gemm_instance_name(i).startswith("ks_")}
    for (M, N, K, name) in ((2048, 2048, 2048, "ks_128x128x64"), (640, 384, 64 * 9 + 17, "ks_128x128x64_clamp")):
        A = inputs.normal((M, K), 71, "bf16")
        B = inputs.normal((K, N), 72, "bf16")
        print("ks determinism", name, (M, N, K), flush=True)
        y1 = run(G, A, B, 3, instance=ks[name])
        y2 = run(G, A, B, 3, instance=ks[name])
        assert np.array_equal(y1, y2)
        assert_bound(y1, oracle.gemm_f64(A, B, "bf16"), K, "bf16", "%s %s" % (name, (M, N, K)))


RAGGED = [(129, 131, 67), (300, 260, 130), (1, 513, 65), (129, 136, 67), (300, 264, 130),
          (1, 520, 65), (255, 8, 200), (8, 1032, 63), (257, 392, 1), (520, 512, 576)]


def _edge_instances(G):
    return [i for i in instances16(G) if G.gemm_instance_name(i).endswith(("_clamp", "_masked"))]


def _expect_for(G, i, N):
    """Clamped-edge instances read row-major B in 8-column chunks: they take
    N % 8 == 0 only and refuse other shapes with GEMM_ERR_INSTANCE; the
    masked instances take any shape."""
    if G.gemm_instance_name(i).endswith("_clamp") and N % 8 != 0:
        return G.GEMM_ERR_INSTANCE
    return 0


def test_edge_instances_on_ragged_shapes(G):
    for (M, N, K) in RAGGED:
        A = inputs.uniform((M, K), M + N, "f16")
        B = inputs.uniform((K, N), M + K, "f16")
        r = oracle.gemm_f64(A, B, "f16")
        for i in _edge_instances(G):
            print("edge", G.gemm_instance_name(i), (M, N, K), flush=True)
            expect = _expect_for(G, i, N)
            y = run(G, A, B, 1, instance=i, expect=expect)
            if expect == 0:
                assert_bound(y, r, K, "f16", "%s %s" % (G.gemm_instance_name(i), (M, N, K)))


@pytest.mark.parametrize("code", [0, 3])
def test_edge_instances_misaligned_strides(G, code):
    """2-byte-aligned base pointer and leading dimensions on every edge
    instance: same bits as the packed, aligned call."""
    fmt, out = DTYPES[code]
    M, N, K = 300, 264, 200
    A = law_for(fmt)((M, K), 111, fmt)
    B = law_for(fmt)((K, N), 112, fmt)
    r = oracle.gemm_f64(A, B, fmt)
    for i in _edge_instances(G):
        print("misaligned", G.gemm_instance_name(i), flush=True)
        y = run(G, A, B, code, instance=i)
        y2 = run(G, A, B, code, lda=K + 1, ldb=N + 3, ldc=N + 1, a_off=1, instance=i)
        assert_bound(y2, r, K, out, "misaligned %s" % G.gemm_instance_name(i))
        assert np.array_equal(y, y2)


def test_non_edge_instance_rejects_ragged_shape(G):
    A = inputs.uniform((129, 64), 1, "f16")
    B = inputs.uniform((64, 128), 2, "f16")
    run(G, A, B, 0, instance=0, expect=G.GEMM_ERR_INSTANCE)


def test_runs_on_the_given_stream(G):
    s = torch.cuda.Stream()
    A = inputs.normal((384, 256), 5, "bf16")
    B = inputs.normal((256, 512), 6, "bf16")
    y = run(G, A, B, 3, stream=s)
    assert_bound(y, oracle.gemm_f64(A, B, "bf16"), 256, "bf16", "stream")


def test_torch_convenience_form(G):
    A = torch.randn(200, 96, dtype=torch.bfloat16, device="cuda")
    B = torch.randn(96, 150, dtype=torch.bfloat16, device="cuda")
    C = G.gemm(A, B, torch.float32)
    Ab = A.cpu().view(torch.int16).numpy().view(np.uint16)
    Bb = B.cpu().view(torch.int16).numpy().view(np.uint16)
    assert_bound(C.cpu().double().numpy(), oracle.gemm_f64(Ab, Bb, "bf16"), 96, "f32", "torch")


# ------------------------------------------------------------ full-size workloads
def _sample_rows(M, bm=256, n=24, seed=0):
    rng = np.random.Generator(np.random.PCG64(seed))
    last_tile = (M // bm) * bm if M % bm else M - bm
    rows = {0, 1, M - 1, min(bm, M - 1), min(bm - 1, M - 1), last_tile, min(last_tile + 1, M - 1)}
    rows |= set(rng.integers(0, M, n).tolist())
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("name", ["f16_256", "f16_2048", "bf16_4096", "bf16_8192", "f16_ragged"])
def test_full_size_workloads(G, name):
    """Every configuration at its full size, through gemm_run, against the
    oracle over all M x N outputs, element by element, at the acceptance
    bound (no sampling)."""
    A, B, w = inputs.workload_inputs(name)
    code = {("f16", "f32"): 0, ("f16", "f16"): 1, ("bf16", "f32"): 2,
            ("bf16", "bf16"): 3}[(w["fmt"], w["out"])]
    print("full-size workload", name, flush=True)
    y = run(G, A, B, code)
    r = oracle.gemm_f64(A, B, w["fmt"])
    res = assert_bound(y, r, w["K"], w["out"], name)
    print(name, "all %d outputs: n_bad %d max_abs %.3g max_rel %.3g worst/bound %.3g" % (
        y.size, res["n_bad"], res["max_abs"], res["max_rel"], res["worst_ratio"]), flush=True)
    assert res["n_bad"] == 0 and y.shape == (w["M"], w["N"])


def test_quarter_grid_full_size_bit_exact(G):
    """4096^3 bf16 -> fp32 on 0.25-grid inputs: every partial sum exact."""
    n = 4096
    A = inputs.quarter((n, n), 201, "bf16")
    B = inputs.quarter((n, n), 202, "bf16")
    y = run(G, A, B, 2)
    assert np.array_equal(y, oracle.gemm_f64(A, B, "bf16"))       # every output
    # exact Freivalds: all values are multiples of 1/16 below 2^24 in magnitude
    Ad = oracle.decode(A, "bf16")
    Bd = oracle.decode(B, "bf16")
    x = np.random.Generator(np.random.PCG64(7)).integers(-2, 3, n).astype(np.float64)
    assert np.array_equal(y @ x, Ad @ (Bd @ x))


@pytest.mark.parametrize("code", [0, 1])
def test_quarter_grid_ragged_bit_exact(G, code):
    """The ragged workload's shape and layout (3000 x 5000 x 4099, fp16 A with
    2-byte-aligned rows of 4099 elements, a partial last tile-row, tile-column
    and k-slice) on 0.25-grid inputs: every partial sum is a multiple of 1/16
    below 2^15, exact in fp32, so the fp32 output is the oracle's bit for bit
    and the fp16 output its correct rounding."""
    M, N, K = 3000, 5000, 4099
    fmt, out = DTYPES[code]
    A = inputs.quarter((M, K), 221, fmt)
    B = inputs.quarter((K, N), 222, fmt)
    print("quarter-grid ragged", code, flush=True)
    y = run(G, A, B, code)
    assert_exact(y, oracle.gemm_f64(A, B, fmt), out, "quarter ragged")


def test_quarter_grid_k_split_bit_exact(G):
    """2048^3 fp16 -> fp32 on 0.25-grid inputs through gemm_run (the k-split
    kernel: four partial tiles summed through LDS): every partial sum is a
    multiple of 1/16 below 2^14, exact in fp32, so the result is the oracle's
    bit for bit."""
    n = 2048
    A = inputs.quarter((n, n), 211, "f16")
    B = inputs.quarter((n, n), 212, "f16")
    inst = G.gemm_select_instance(n, n, n, 0, 1 << 32, n, 1 << 36, n, 1 << 40, n)
    assert G.gemm_instance_name(inst) == "ks_128x128x64"
    y = run(G, A, B, 0)
    assert np.array_equal(y, oracle.gemm_f64(A, B, "f16"))        # every output
    Ad = oracle.decode(A, "f16")
    Bd = oracle.decode(B, "f16")
    x = np.random.Generator(np.random.PCG64(8)).integers(-2, 3, n).astype(np.float64)
    assert np.array_equal(y @ x, Ad @ (Bd @ x))
