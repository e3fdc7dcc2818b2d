"""gemm_run_noalloc (scheduler words in the library's static device array)
against gemm_run_ws (the same words in a caller's workspace), through the C
ABI, on two calls in a row, the second on a smaller problem: both select the
persistent kernel, so both use the array; the outputs must be identical bit
for bit, and equal to gemm_run's.  Also: a shape that does not use the array,
a column-major B with the general epilogue, and the argument checks."""
import numpy as np
import pytest

from dense_half_precision_tiled_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from tests.gpu_helpers import DTYPES, law_for, run  # noqa: E402


@pytest.fixture(scope="module")
def G():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from dense_half_precision_tiled_amd import gemm
    gemm.load()
    return gemm


def _noalloc(G, A, B, code, layout=0, alpha=1.0, beta=0.0, bias=None, relu=0, c_init=None):
    """C through gemm_run_noalloc; returns decoded M x N values."""
    M, K = A.shape
    N = B.shape[1] if layout == 0 else B.shape[0]
    out = DTYPES[code][1]
    tA = torch.from_numpy(A.view(np.int16)).cuda()
    tB = torch.from_numpy(B.view(np.int16)).cuda()
    if c_init is not None:
        raw0 = np.asarray(c_init)
        tC = torch.from_numpy(raw0.view(np.int32 if out == "f32" else np.int16).copy()).cuda()
    else:
        tC = torch.full((M, N), -1, dtype=torch.int32 if out == "f32" else torch.int16, device="cuda")
    tb = torch.tensor(np.asarray(bias, dtype=np.float32), device="cuda") if bias is not None else None
    st = G.gemm_run_noalloc(M, N, K, code, layout, tA.data_ptr(), K, tB.data_ptr(), N if layout == 0 else K,
                            tC.data_ptr(), N, alpha, beta, tb.data_ptr() if tb is not None else None, relu,
                            torch.cuda.current_stream().cuda_stream)
    assert st == 0, G.gemm_strerror(st)
    torch.cuda.synchronize()
    raw = tC.cpu().numpy()
    if out == "f32":
        return raw.view(np.float32).astype(np.float64)
    if out == "f16":
        return raw.view(np.float16).astype(np.float64)
    return (raw.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _ws(G):
    return torch.zeros(G.gemm_workspace_size() // 4, dtype=torch.int32, device="cuda")


def test_two_calls_in_a_row_match_gemm_run_ws(G):
    ws = _ws(G)
    for (M, N, K) in ((8192, 8192, 256), (4096, 8192, 192)):     # 1024 then 512 tiles: persistent both times
        A = inputs.normal((M, K), M + K, "bf16")
        B = inputs.normal((K, N), N + K, "bf16")
        sel = G.gemm_instance_name(G.gemm_select_instance_ws(M, N, K, 3, 0, 1 << 32, K, 1 << 36, N, 1 << 40, N,
                                                             1.0, 0.0, None, 0, ws.data_ptr(),
                                                             G.gemm_workspace_size()))
        assert sel.startswith("pk_"), sel
        print("noalloc", (M, N, K), sel, flush=True)
        y = _noalloc(G, A, B, 3)
        ref = run(G, A, B, 3, ws=ws)
        assert np.array_equal(y, ref)
        assert np.array_equal(y, run(G, A, B, 3))


def test_shape_without_scratch_and_general_epilogue(G):
    # 4096^2 output: one tile per CU, the one-tile kernel, no scratch
    A = inputs.uniform((4096, 128), 3, "f16")
    B = inputs.uniform((128, 4096), 4, "f16")
    assert np.array_equal(_noalloc(G, A, B, 1), run(G, A, B, 1))
    # column-major B, alpha/beta/bias/ReLU, persistent kernel with clamped edges
    M, N, K = 8000, 8016, 100
    A = inputs.normal((M, K), 5, "bf16")
    Bt = inputs.normal((N, K), 6, "bf16")
    bias = np.linspace(-1, 1, N)
    c0 = inputs.normal((M, N), 7, "bf16")
    kw = dict(alpha=0.75, beta=-0.5, bias=bias, relu=1, c_init=c0)
    y = _noalloc(G, A, Bt, 3, layout=1, **kw)
    ref = run(G, A, Bt, 3, layout=G.GEMM_B_COL_MAJOR, ws=_ws(G), **kw)
    assert np.array_equal(y, ref)


def test_argument_errors(G):
    assert G.gemm_run_noalloc(-1, 4, 4, 0, 0, 1 << 32, 4, 1 << 36, 4, 1 << 40, 4, 1.0, 0.0, None, 0, None) \
        == G.GEMM_ERR_DIM
    assert G.gemm_run_noalloc(4, 4, 4, 0, 7, 1 << 32, 4, 1 << 36, 4, 1 << 40, 4, 1.0, 0.0, None, 0, None) \
        == G.GEMM_ERR_LAYOUT
    assert G.gemm_run_noalloc(0, 4, 4, 0, 0, 0, 4, 0, 4, 0, 4, 1.0, 0.0, None, 0, None) == 0
