"""The ping-pong kernel (8 waves in two groups taking turns between MFMAs
and data movement; instances pp_256x256x64 (half-slice phases) and
pp_256x256x64_ph4 (whole-slice phases), whole 256x256 tiles) on the GPU.

Each output element is accumulated over the same k-steps in the same order as
in the 256x256 direct-to-LDS kernel, so the two must agree bit for bit, on
every whole-tile shape, both B layouts and the general epilogue; one shape is
also checked against the oracle's bound, and the 4096^3 workload and a
0.25-grid 2048 x 2048 x 4096 product (exact) at full size.
"""
import numpy as np
import pytest

import oracle
from dense_half_precision_tiled_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from tests.gpu_helpers import DTYPES, assert_bound, law_for, run  # noqa: E402


@pytest.fixture(scope="module")
def G():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from dense_half_precision_tiled_amd import gemm
    gemm.load()
    return gemm


@pytest.fixture(scope="module")
def ids(G):
    return {G.gemm_instance_name(i): i for i in range(G.gemm_num_instances())}


SHAPES = [(256, 256, 64), (256, 512, 128), (768, 512, 64 * 7), (1024, 1024, 1024), (512, 2048, 320)]


PP = ["pp_256x256x64", "pp_256x256x64_ph4"]


@pytest.mark.parametrize("name", PP)
@pytest.mark.parametrize("code", [0, 1, 2, 3])
def test_equals_the_direct_to_lds_kernel(G, ids, code, name):
    fmt, out = DTYPES[code]
    for (M, N, K) in SHAPES:
        A = law_for(fmt)((M, K), M + K, fmt)
        B = law_for(fmt)((K, N), N + K, fmt)
        print(name, code, (M, N, K), flush=True)
        y = run(G, A, B, code, instance=ids[name])
        assert np.array_equal(y, run(G, A, B, code, instance=ids["dl_256x256x64_fd2"])), (M, N, K)


@pytest.mark.parametrize("name", PP)
def test_column_major_b_and_general_epilogue(G, ids, name):
    M, N, K = 512, 768, 256
    A = inputs.normal((M, K), 11, "bf16")
    Bt = inputs.normal((N, K), 12, "bf16")
    bias = np.linspace(-2, 2, N)
    c0 = inputs.normal((M, N), 13, "bf16")
    for kw in ({}, {"alpha": -0.5, "beta": 0.75, "bias": bias, "relu": 1, "c_init": c0}):
        for lay, Bs in ((G.GEMM_B_COL_MAJOR, Bt), (G.GEMM_B_ROW_MAJOR, np.ascontiguousarray(Bt.T))):
            print("pp layout", lay, sorted(kw), flush=True)
            y = run(G, A, Bs, 3, instance=ids[name], layout=lay, **kw)
            ref = run(G, A, Bs, 3, instance=ids["dl_256x256x64_fd2"], layout=lay, **kw)
            assert np.array_equal(y, ref)


@pytest.mark.parametrize("name", PP)
def test_against_the_oracle_and_refusals(G, ids, name):
    M, N, K = 512, 512, 576
    A = inputs.uniform((M, K), 21, "f16")
    B = inputs.uniform((K, N), 22, "f16")
    y = run(G, A, B, 0, instance=ids[name])
    assert_bound(y, oracle.gemm_f64(A, B, "f16"), K, "f32", name + " 512x512x576")
    # whole tiles only: other shapes are refused before any launch
    for (M, N, K) in ((300, 256, 64), (256, 264, 64), (256, 256, 100)):
        run(G, inputs.uniform((M, K), 1, "f16"), inputs.uniform((K, N), 2, "f16"), 0,
            instance=ids[name], expect=G.GEMM_ERR_INSTANCE)


@pytest.mark.parametrize("name", PP)
def test_full_size(G, ids, name):
    A, B, w = inputs.workload_inputs("bf16_4096")
    y = run(G, A, B, 3, instance=ids[name])
    assert np.array_equal(y, run(G, A, B, 3, instance=ids["dl_256x256x64_fd2"]))
    n = 2048
    A = inputs.quarter((n, 4096), 31, "f16")
    B = inputs.quarter((4096, n), 32, "f16")
    y = run(G, A, B, 0, instance=ids[name])
    assert np.array_equal(y, oracle.gemm_f64(A, B, "f16"))          # exact: every output
