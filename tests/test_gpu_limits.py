"""Limits and concurrency of the boundary on the GPU.

* Leading dimensions past 2^31 elements: a row offset i * ld no longer fits in
  32 bits, so every address the kernels form from it must be 64-bit.  The
  operands live in device buffers of several GiB of which only the used rows
  are written (device-side copies; nothing that size crosses from the host).
* Two streams: the library keeps no state and allocates nothing, so two
  different products enqueued on two streams at once both come out right.
* The copy-offset limit: the whole-tile kernels address their copies as byte
  offsets below 2^31 from a per-tile base.  At the largest leading dimension
  that fits, a full tile reaches offsets just under 2^31; the result must
  equal, bit for bit, the masked kernel's (same family, same k order), which
  the next leading dimension up is sent to.
"""
import numpy as np
import pytest

import oracle
from dense_half_precision_tiled_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from tests.gpu_helpers import DTYPES, assert_bound, decode_out  # noqa: E402

BIG = (1 << 31) + 64        # elements: row 1 starts past 2^31


@pytest.fixture(scope="module")
def G():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from dense_half_precision_tiled_amd import gemm
    gemm.load()      # raises if the library is missing: no fallback
    return gemm


def _rows_at(bits, ld, dtype):
    """A device buffer of (rows - 1) * ld + cols elements holding `bits` row by
    row at stride ld; the gaps are left unwritten."""
    rows, cols = bits.shape
    buf = torch.empty((rows - 1) * ld + cols, dtype=dtype, device="cuda")
    src = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16 if bits.dtype == np.uint16 else np.int8)).cuda()
    for r in range(rows):
        buf[r * ld:r * ld + cols].copy_(src[r])
    return buf


@pytest.mark.parametrize("code,fmt,out,layout", [(3, "bf16", "bf16", "row"), (0, "f16", "f32", "col"),
                                                  (4, "e4m3", "f32", "row"), (6, "e4m3", "bf16", "col")])
def test_leading_dimensions_past_2_pow_31(G, code, fmt, out, layout):
    col = layout == "col"
    M, N, K = 3, (2 if col else 256), 320       # column-major B holds N rows at stride ld: keep N small
    in8 = fmt in ("e4m3", "e5m2")
    idt = torch.int8 if in8 else torch.int16
    A = inputs.normal((M, K), 1201, fmt) if fmt != "f16" else inputs.uniform((M, K), 1201, fmt)
    B = inputs.normal((K, N), 1202, fmt) if fmt != "f16" else inputs.uniform((K, N), 1202, fmt)
    Bs = np.ascontiguousarray(B.T) if col else B
    tA = _rows_at(A, BIG, idt)
    tB = _rows_at(Bs, BIG, idt) if col else torch.from_numpy(B.view(np.int16 if not in8 else np.int8)).cuda()
    ldb = BIG if col else N
    tC = torch.full(((M - 1) * BIG + N,), -1, dtype=torch.int32 if out == "f32" else torch.int16, device="cuda")
    print("large ld", code, layout, flush=True)
    st = G.gemm_run_ex(M, N, K, code, G.GEMM_B_COL_MAJOR if col else G.GEMM_B_ROW_MAJOR, tA.data_ptr(), BIG,
                       tB.data_ptr(), ldb, tC.data_ptr(), BIG, 1.0, 0.0, None, 0,
                       torch.cuda.current_stream().cuda_stream)
    assert st == 0, G.gemm_strerror(st)
    torch.cuda.synchronize()
    rows = torch.stack([tC[r * BIG:r * BIG + N] for r in range(M)]).cpu().numpy()
    y = decode_out(rows.view(np.uint32 if out == "f32" else np.uint16), out)
    # the gap after row 0 was never written
    gap = tC[N:N + 4096].cpu().numpy().view(np.int32 if out == "f32" else np.int16)
    assert np.all(gap == -1)
    extra = oracle.align_bound8(A, B, fmt) if in8 else None
    assert_bound(y, oracle.gemm_f64(A, B, fmt), K, out, "ld 2^31+64", extra=extra)
    del tA, tB, tC
    torch.cuda.empty_cache()


def test_two_streams_at_once(G):
    """Two different products on two streams, enqueued back to back without a
    synchronisation between them, each checked against the oracle."""
    cases = [(2048, 1024, 1536, 3, "bf16", "bf16"), (1000, 1200, 900, 4, "e4m3", "f32")]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    keep = []
    for (M, N, K, code, fmt, out), s in zip(cases, streams):
        A = inputs.normal((M, K), 1300 + code, fmt)
        B = inputs.normal((K, N), 1310 + code, fmt)
        v = np.int8 if A.dtype == np.uint8 else np.int16
        tA = torch.from_numpy(A.view(v)).cuda()
        tB = torch.from_numpy(B.view(v)).cuda()
        tC = torch.empty((M, N), dtype=torch.int32 if out == "f32" else torch.int16, device="cuda")
        keep.append((A, B, tA, tB, tC, M, N, K, code, fmt, out, s))
    torch.cuda.synchronize()
    for (A, B, tA, tB, tC, M, N, K, code, fmt, out, s) in keep:
        for _ in range(3):
            st = G.gemm_run(M, N, K, code, tA.data_ptr(), K, tB.data_ptr(), N, tC.data_ptr(), N, s.cuda_stream)
            assert st == 0, G.gemm_strerror(st)
    torch.cuda.synchronize()
    for (A, B, tA, tB, tC, M, N, K, code, fmt, out, s) in keep:
        y = decode_out(tC.cpu().numpy().view(np.uint32 if out == "f32" else np.uint16), out)
        extra = oracle.align_bound8(A, B, fmt) if fmt == "e4m3" else None
        assert_bound(y, oracle.gemm_f64(A, B, fmt), K, out, "stream %s" % fmt, extra=extra)


def _instance(G, name):
    ids = {G.gemm_instance_name(i): i for i in range(G.gemm_num_instances())}
    return ids[name]


@pytest.mark.parametrize("code,fmt,col,shape,tile,fast,masked,same_family", [
    (3, "bf16", False, (256, 256, 128), 256, "dl_256x256x64_fd2", "dl_256x256x64_masked", True),
    (6, "e4m3", True, (256, 256, 128), 256, "dl8_256x256x128", "dl8_256x256x128_masked", True),
    (1, "f16", False, (300, 264, 200), 256, "dl_256x256x64_fd2_clamp", "dl_256x256x64_masked", True),
    (0, "f16", False, (128, 128, 256), 128, "ks_128x128x64", "dl_128x128x64_masked", False)])
def test_copy_offsets_at_the_31_bit_limit(G, code, fmt, col, shape, tile, fast, masked, same_family):
    """A full tile at the largest leading dimension that keeps its copy
    offsets under 2^31 bytes (A rows, or column-major B rows), then one
    element more on the masked kernel, which the fast one declines.  Within
    one family (dl, dl8) the two give identical bits; the k-split kernel sums
    in another order and is held to the bound."""
    M, N, K = shape
    in8 = fmt == "e4m3"
    esz = 1 if in8 else 2
    ld = (2 ** 31 - 1 - 128) // ((tile - 1) * esz)
    idt = torch.int8 if in8 else torch.int16
    A = (inputs.uniform if fmt == "f16" else inputs.normal)((M, K), 1401, fmt)
    B = (inputs.uniform if fmt == "f16" else inputs.normal)((K, N), 1402, fmt)
    lay = G.GEMM_B_COL_MAJOR if col else G.GEMM_B_ROW_MAJOR
    out = DTYPES[code][1]
    res = {}
    for name, lda in ((fast, ld), (masked, ld + 1)):
        if col:
            tA = _rows_at(A, K, idt)
            tB = _rows_at(np.ascontiguousarray(B.T), lda, idt)
            a_ld, b_ld = K, lda
        else:
            tA = _rows_at(A, lda, idt)
            tB = torch.from_numpy(B.view(np.int8 if in8 else np.int16)).cuda()
            a_ld, b_ld = lda, N
        tC = torch.empty((M, N), dtype=torch.int32 if out == "f32" else torch.int16, device="cuda")
        print("offset limit", name, lda, flush=True)
        args = (M, N, K, code, lay, tA.data_ptr(), a_ld, tB.data_ptr(), b_ld, tC.data_ptr(), N, 1.0, 0.0, None, 0,
                torch.cuda.current_stream().cuda_stream)
        st = G.gemm_run_instance_ex(_instance(G, name), *args)
        assert st == 0, G.gemm_strerror(st)
        if name == masked:          # one element more: the fast kernel declines
            assert G.gemm_run_instance_ex(_instance(G, fast), *args) == G.GEMM_ERR_INSTANCE
        torch.cuda.synchronize()
        res[name] = decode_out(tC.cpu().numpy().view(np.uint32 if out == "f32" else np.uint16), out)
        del tA, tB, tC
        torch.cuda.empty_cache()
    if same_family:
        assert np.array_equal(res[fast], res[masked])
    extra = oracle.align_bound8(A, B, fmt) if in8 else None
    ref = oracle.gemm_f64(A, B, fmt)
    for name in (fast, masked):
        assert_bound(res[name], ref, K, out, "offset limit " + name, extra=extra)
