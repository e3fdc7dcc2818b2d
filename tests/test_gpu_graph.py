"""HIP graph capture of the boundary calls.

gemm_run and gemm_run_ex enqueue kernels only: no allocation, no memset, no
host synchronisation, no state between calls.  So a call can be captured into
a HIP graph (torch.cuda.CUDAGraph drives hipStreamBeginCapture) and replayed.
Each replay is checked bit for bit against the eager call on the same inputs,
with eager work between the replays (new A written into the captured buffer,
C poisoned), and the eager results against the oracle.  Cases cover every
kernel geometry the selection uses (64x64, 128x128 split over waves or over
K, 256x256), the general epilogue with column-major B, and 8-bit inputs in
both B layouts; and the allocation-free entry point on the persistent kernel.
"""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from tests.gpu_helpers import DTYPES, assert_bound, decode_out, law_for  # noqa: E402


@pytest.fixture(scope="module")
def G():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from dense_half_precision_tiled_amd import gemm
    gemm.load()      # raises if the library is missing: no fallback
    return gemm


def _dev(bits):
    b = np.ascontiguousarray(bits)
    return torch.from_numpy(b.view(np.int16) if b.dtype == np.uint16 else b.view(np.int8)).cuda()


# (M, N, K, dtype code, B layout, expected kernel family prefix)
CASES = [
    (512, 384, 320, 0, "row", "dl_64x64"),          # small shape: 64x64 tiles
    (1024, 1024, 2048, 3, "row", "ks_"),            # 128x128, K split across the waves
    (1536, 1536, 1024, 3, "row", "dl_128x128"),     # 144 tiles of 128^2
    (2048, 4096, 512, 0, "row", "dl_256x256"),      # 128 tiles of 256^2
    (300, 264, 200, 1, "col", "dl_64x64"),          # general epilogue, column-major B, clamped edges
    (2048, 2048, 1024, 6, "row", "dl8_128x128"),    # 8-bit inputs (E4M3 -> bf16), row-major B
    (520, 392, 300, 7, "col", "dl8_64x64"),         # 8-bit inputs, general epilogue, column-major B
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%dx%dx%d_%d_%s" % c[:5])
def test_graph_replay_matches_eager(G, case):
    M, N, K, code, layout, family = case
    fmt, out = DTYPES[code]
    col = layout == "col"
    As = [law_for(fmt)((M, K), 300 + i, fmt) for i in range(2)]
    B = law_for(fmt)((K, N), 310, fmt)
    Bst = np.ascontiguousarray(B.T) if col else B
    tA, tB = _dev(As[0]), _dev(Bst)
    obits = np.uint32 if out == "f32" else np.uint16
    tC = torch.empty((M, N), dtype=torch.int32 if out == "f32" else torch.int16, device="cuda")
    ldb = K if col else N
    alpha, relu = (0.5, 1) if col else (1.0, 0)

    def enqueue(stream_handle):
        if col:
            return G.gemm_run_ex(M, N, K, code, G.GEMM_B_COL_MAJOR, tA.data_ptr(), K, tB.data_ptr(), ldb,
                                 tC.data_ptr(), N, alpha, 0.0, None, relu, stream_handle)
        return G.gemm_run(M, N, K, code, tA.data_ptr(), K, tB.data_ptr(), N, tC.data_ptr(), N, stream_handle)

    if col:
        inst = G.gemm_select_instance_ex(M, N, K, code, G.GEMM_B_COL_MAJOR, tA.data_ptr(), K, tB.data_ptr(),
                                         ldb, tC.data_ptr(), N, alpha, 0.0, None, relu)
    else:
        inst = G.gemm_select_instance(M, N, K, code, tA.data_ptr(), K, tB.data_ptr(), N, tC.data_ptr(), N)
    name = G.gemm_instance_name(inst)
    assert name.startswith(family), name
    print("graph case", case, name, flush=True)

    eager = []
    for A in As:
        tA.copy_(_dev(A))
        tC.fill_(-1)
        assert enqueue(torch.cuda.current_stream().cuda_stream) == 0
        torch.cuda.synchronize()
        eager.append(tC.cpu().numpy().view(obits).copy())

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        st = enqueue(torch.cuda.current_stream().cuda_stream)
    assert st == 0, G.gemm_strerror(st)
    torch.cuda.synchronize()

    for it in range(6):
        i = it % 2
        tA.copy_(_dev(As[i]))       # eager work between replays
        tC.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = tC.cpu().numpy().view(obits)
        assert np.array_equal(got, eager[i]), "replay %d differs from the eager call" % it

    for A, e in zip(As, eager):
        y = decode_out(e, out)
        extra = oracle.align_bound8(A, B, fmt) if fmt in ("e4m3", "e5m2") else None
        if col:
            r = oracle.gemm_ex_f64(A, Bst, fmt, b_layout="col", alpha=alpha, relu=bool(relu))
            res = oracle.compare_ex(y, r, K, out, alpha=alpha, dot=oracle.gemm_ex_f64(A, Bst, fmt, b_layout="col"),
                                    extra=extra)
            assert res["ok"], res
        else:
            assert_bound(y, oracle.gemm_f64(A, B, fmt), K, out, "eager %s" % name, extra=extra)


def test_noalloc_graph_replay_matches_gemm_run(G):
    """gemm_run_noalloc is for callers that cannot allocate, code under graph
    capture among them: on a shape that selects the persistent kernel (two
    256x256 tiles per compute unit), the captured call (the fill kernel that
    clears the library's scheduler array, then the persistent kernel) replays
    six times, with eager calls of the same entry point between the replays,
    each replay bit for bit equal to gemm_run's result on the same inputs."""
    M, N, K, code = 8192, 4096, 256, 3
    fmt, out = DTYPES[code]
    As = [law_for(fmt)((M, K), 330 + i, fmt) for i in range(2)]
    B = law_for(fmt)((K, N), 340, fmt)
    tA, tB = _dev(As[0]), _dev(B)
    tC = torch.empty((M, N), dtype=torch.int16, device="cuda")
    ws = torch.zeros(G.gemm_workspace_size() // 4, dtype=torch.int32, device="cuda")
    inst = G.gemm_select_instance_ws(M, N, K, code, G.GEMM_B_ROW_MAJOR, tA.data_ptr(), K, tB.data_ptr(), N,
                                     tC.data_ptr(), N, 1.0, 0.0, None, 0, ws.data_ptr(), ws.numel() * 4)
    assert G.gemm_instance_name(inst).startswith("pk_"), G.gemm_instance_name(inst)

    def noalloc(stream_handle):
        return G.gemm_run_noalloc(M, N, K, code, G.GEMM_B_ROW_MAJOR, tA.data_ptr(), K, tB.data_ptr(), N,
                                  tC.data_ptr(), N, 1.0, 0.0, None, 0, stream_handle)

    plain = []
    for A in As:
        tA.copy_(_dev(A))
        tC.fill_(-1)
        assert G.gemm_run(M, N, K, code, tA.data_ptr(), K, tB.data_ptr(), N, tC.data_ptr(), N,
                          torch.cuda.current_stream().cuda_stream) == 0
        torch.cuda.synchronize()
        plain.append(tC.cpu().numpy().view(np.uint16).copy())
        # an eager call first (as a caller would warm up): the library looks up
        # the array's device address once, outside any capture
        tC.fill_(-1)
        assert noalloc(torch.cuda.current_stream().cuda_stream) == 0
        torch.cuda.synchronize()
        assert np.array_equal(tC.cpu().numpy().view(np.uint16), plain[-1])

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        st = noalloc(torch.cuda.current_stream().cuda_stream)
    assert st == 0, G.gemm_strerror(st)
    torch.cuda.synchronize()

    for it in range(6):
        i = it % 2
        tA.copy_(_dev(As[1 - i]))
        tC.fill_(-1)
        assert noalloc(torch.cuda.current_stream().cuda_stream) == 0       # eager use of the same array
        torch.cuda.synchronize()
        assert np.array_equal(tC.cpu().numpy().view(np.uint16), plain[1 - i]), "eager call %d" % it
        tA.copy_(_dev(As[i]))
        tC.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(tC.cpu().numpy().view(np.uint16), plain[i]), "replay %d differs from gemm_run" % it
    assert_bound(decode_out(plain[0], out), oracle.gemm_f64(As[0], B, fmt), K, out, "persistent 8192x4096x256")
