"""Whole-matrix bit-exact checks at 8192^3 (GPU).

Inputs are i.i.d. multiples of 0.25 in [-2, 2] (the exact fixtures of "mma.sync
and ldmatrix", section "Two probes and one matmul"): every value is exact in
bf16, E4M3 and E5M2; every product is a multiple of 1/16 of magnitude at most
4; every partial sum of K = 8192 of them is a multiple of 1/16 below
2^15 < 2^19, hence exact in fp32 whatever the summation order.  For the 8-bit
MFMA, which aligns each group of 8 products to the largest and keeps 13
binades below it, nothing is cut either: the largest product of a group is at
most 4 = 2^2, so the cut sits at or below 2^-11, under the 2^-4 grain of the
products.  So the fp32 output must equal the exact product, bit for bit, for
every one of the 67,108,864 outputs: the headline kernel (bf16, row-major B)
and the 8-bit kernels (E4M3 and E5M2, row- and column-major B).

The oracle runs once over the full matrix; the inputs of the five calls hold
the same values (checked by decoding each format's bit patterns), so the
same exact result serves all five.  An exact Freivalds check (integer x)
backs each comparison.
"""
import numpy as np
import pytest

import oracle
from dense_half_precision_tiled_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from tests.gpu_helpers import run  # noqa: E402

N = 8192
SEED_A, SEED_B = 401, 402


@pytest.fixture(scope="module")
def G():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from dense_half_precision_tiled_amd import gemm
    gemm.load()
    return gemm


@pytest.fixture(scope="module")
def exact():
    A = inputs.quarter((N, N), SEED_A, "bf16")
    B = inputs.quarter((N, N), SEED_B, "bf16")
    print("oracle 8192^3 on the 0.25 grid", flush=True)
    r = oracle.gemm_f64(A, B, "bf16")
    Ad = oracle.decode(A, "bf16")
    Bd = oracle.decode(B, "bf16")
    x = np.random.Generator(np.random.PCG64(17)).integers(-3, 4, N).astype(np.float64)
    return {"r": r, "Ad": Ad, "Bd": Bd, "x": x, "Bx": Bd @ x}


def _check(y, ex, what):
    bad = y != ex["r"]
    assert not bad.any(), "%s: %d of %d outputs differ, first at %s: %r vs %r" % (
        what, int(bad.sum()), y.size, np.argwhere(bad)[0], y[bad][0], ex["r"][bad][0])
    # exact Freivalds: integers times multiples of 1/16 below 2^15, sums below 2^53
    assert np.array_equal(y @ ex["x"], ex["Ad"] @ ex["Bx"]), what + ": Freivalds"
    print(what, "all %d outputs bit-exact" % y.size, flush=True)


def test_bf16_row_major_8192_fp32_bit_exact(G, exact):
    A = inputs.quarter((N, N), SEED_A, "bf16")
    B = inputs.quarter((N, N), SEED_B, "bf16")
    print("bf16 8192^3 -> f32, instance",
          G.gemm_instance_name(G.gemm_select_instance(N, N, N, 2, 1 << 32, N, 1 << 36, N, 1 << 40, N)),
          flush=True)
    _check(run(G, A, B, 2), exact, "bf16 8192^3")


@pytest.mark.parametrize("fmt,code", [("e4m3", 4), ("e5m2", 7)])
@pytest.mark.parametrize("lay", ["row", "col"])
def test_8bit_8192_fp32_bit_exact(G, exact, fmt, code, lay):
    A = inputs.quarter((N, N), SEED_A, fmt)
    B = inputs.quarter((N, N), SEED_B, fmt)
    # the same values as the bf16 fixture the oracle ran on
    assert np.array_equal(oracle.decode(A, fmt), exact["Ad"])
    assert np.array_equal(oracle.decode(B, fmt), exact["Bd"])
    print("%s 8192^3 -> f32, B %s-major" % (fmt, lay), flush=True)
    if lay == "row":
        y = run(G, A, B, code)
    else:
        y = run(G, A, np.ascontiguousarray(B.T), code, layout=G.GEMM_B_COL_MAJOR)
    _check(y, exact, "%s %s 8192^3" % (fmt, lay))
