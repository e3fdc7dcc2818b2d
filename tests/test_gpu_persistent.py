"""The persistent kernels (one workgroup per CU taking tiles from per-XCD
atomic queues in a caller-owned workspace; gemm_run_ws) on the GPU.

* Bit for bit the output of the one-workgroup-per-tile kernel of the same
  tile and edge mode, on shapes with fewer tiles than CUs, about one tile per
  CU, and several tiles per CU, both B layouts and the general epilogue:
  only the order in which tiles are taken differs.  Every output element of
  these calls is checked (poisoned C: a tile no workgroup took would stay
  NaN), and one shape against the oracle's bound directly.
* The scheduler words are left zeroed after every call (the next call can
  reuse the workspace), and repeated calls give identical bits.
* gemm_run_ws picks the persistent kernel with two or more 256x256 tiles per
  CU and gives the same bits as gemm_run everywhere.
* Two streams with two workspaces run concurrently and both results hold.
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


def new_ws(G):
    return torch.zeros(G.gemm_workspace_size() // 4, dtype=torch.int32, device="cuda")


SHAPES = [(256, 256, 64), (512, 768, 128), (2048, 2048, 256), (4096, 4096, 128), (8192, 4096, 128),
          (6144, 8192, 64)]


@pytest.mark.parametrize("code", [0, 1, 3])
def test_whole_tiles_equal_the_one_tile_kernel(G, ids, code):
    fmt, out = DTYPES[code]
    ws = new_ws(G)
    for (M, N, K) in SHAPES:
        A = law_for(fmt)((M, K), M + 7, fmt)
        B = law_for(fmt)((K, N), N + 9, fmt)
        print("pk vs dl", code, (M, N, K), flush=True)
        y = run(G, A, B, code, instance=ids["pk_256x256x64"], ws=ws)
        ref = run(G, A, B, code, instance=ids["dl_256x256x64_fd2"])
        assert np.array_equal(y, ref), (M, N, K)
        assert int(ws.abs().sum().item()) == 0, "scheduler words not reset"


def test_against_the_oracle(G, ids):
    M, N, K = 1536, 2560, 320
    A = inputs.normal((M, K), 31, "bf16")
    B = inputs.normal((K, N), 32, "bf16")
    y = run(G, A, B, 3, instance=ids["pk_256x256x64"], ws=new_ws(G))
    assert_bound(y, oracle.gemm_f64(A, B, "bf16"), K, "bf16", "pk 1536x2560x320")


@pytest.mark.parametrize("shape", [(3000, 5000, 4099), (257, 520, 67), (1000, 1032, 300), (8, 4104, 65)])
def test_clamped_edges_equal_the_one_tile_kernel(G, ids, shape):
    M, N, K = shape
    A = inputs.uniform((M, K), M, "f16")
    B = inputs.uniform((K, N), N, "f16")
    ws = new_ws(G)
    print("pk clamp", shape, flush=True)
    y = run(G, A, B, 1, instance=ids["pk_256x256x64_clamp"], ws=ws)
    ref = run(G, A, B, 1, instance=ids["dl_256x256x64_fd2_clamp"])
    assert np.array_equal(y, ref)
    # misaligned rows and base pointer, padded output rows
    y2 = run(G, A, B, 1, instance=ids["pk_256x256x64_clamp"], ws=ws, lda=K + 1, ldb=N + 8, ldc=N + 3, a_off=1)
    assert np.array_equal(y2, ref)
    assert int(ws.abs().sum().item()) == 0


def test_column_major_b_and_general_epilogue(G, ids):
    M, N, K = 2048, 1536, 192
    A = inputs.normal((M, K), 41, "bf16")
    Bt = inputs.normal((N, K), 42, "bf16")           # B stored column-major: its N x K transpose
    bias = np.random.Generator(np.random.PCG64(43)).standard_normal(N)
    c0 = inputs.normal((M, N), 44, "bf16")
    ws = new_ws(G)
    for kw in ({}, {"alpha": 0.5, "beta": -1.25, "bias": bias, "relu": 1, "c_init": c0}):
        for inst in ("pk_256x256x64", "pk_256x256x64_clamp"):
            print("pk col-major", inst, sorted(kw), flush=True)
            y = run(G, A, Bt, 3, instance=ids[inst], ws=ws, layout=G.GEMM_B_COL_MAJOR, **kw)
            ref = run(G, A, Bt, 3, instance=ids[inst.replace("pk_256x256x64", "dl_256x256x64_fd2")],
                      layout=G.GEMM_B_COL_MAJOR, **kw)
            assert np.array_equal(y, ref)


def test_repeated_calls_and_reuse_of_the_workspace(G, ids):
    M, N, K = 4096, 4096, 256
    A = inputs.normal((M, K), 51, "bf16")
    B = inputs.normal((K, N), 52, "bf16")
    ws = new_ws(G)
    first = run(G, A, B, 3, instance=ids["pk_256x256x64"], ws=ws)
    for _ in range(6):
        assert np.array_equal(run(G, A, B, 3, instance=ids["pk_256x256x64"], ws=ws), first)
    assert int(ws.abs().sum().item()) == 0


def test_selection_and_agreement_with_gemm_run(G, ids):
    ws = new_ws(G)
    wsb = G.gemm_workspace_size()
    sel = lambda M, N, K, code=3, lay=0: G.gemm_instance_name(G.gemm_select_instance_ws(
        M, N, K, code, lay, 1 << 32, K, 1 << 36, N if lay == 0 else K, 1 << 40, N, 1.0, 0.0, None, 0,
        ws.data_ptr(), wsb))
    assert sel(8192, 8192, 8192) == "pk_256x256x64"
    assert sel(8192, 8192, 8192, 3, 1) == "pk_256x256x64"
    assert sel(8000, 8000, 4099, 1) == "pk_256x256x64_clamp"
    assert sel(4096, 4096, 4096).startswith("dl_256")           # one tile per CU: nothing to rebalance
    assert sel(2048, 2048, 2048, 0).startswith("ks_")
    assert sel(8192, 8192, 8192, 6, 1).startswith("dl8_")        # 8-bit inputs: no persistent form
    for (M, N, K, code) in ((8192, 8192, 512, 3), (4096, 4096, 512, 3), (8000, 8008, 300, 1)):
        fmt = DTYPES[code][0]
        A = law_for(fmt)((M, K), K, fmt)
        B = law_for(fmt)((K, N), K + 1, fmt)
        print("gemm_run_ws vs gemm_run", (M, N, K, code), flush=True)
        assert np.array_equal(run(G, A, B, code, ws=ws), run(G, A, B, code))


def test_two_streams_two_workspaces(G, ids):
    M, N, K = 8192, 4096, 256
    A = inputs.normal((M, K), 61, "bf16")
    B = inputs.normal((K, N), 62, "bf16")
    ref = run(G, A, B, 3, instance=ids["dl_256x256x64_fd2"])
    tA = torch.from_numpy(A.view(np.int16)).cuda()
    tB = torch.from_numpy(B.view(np.int16)).cuda()
    outs = [torch.full((M, N), -1, dtype=torch.int16, device="cuda") for _ in range(2)]
    wss = [new_ws(G), new_ws(G)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for rep in range(3):
        for i in range(2):
            st = G.gemm_run_ws(M, N, K, 3, 0, tA.data_ptr(), K, tB.data_ptr(), N, outs[i].data_ptr(), N,
                               1.0, 0.0, None, 0, wss[i].data_ptr(), G.gemm_workspace_size(),
                               streams[i].cuda_stream)
            assert st == 0
    torch.cuda.synchronize()
    for i in range(2):
        raw = outs[i].cpu().numpy().view(np.uint16)
        y = (raw.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert np.array_equal(y, ref)
        assert int(wss[i].abs().sum().item()) == 0
