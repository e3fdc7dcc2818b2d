"""Helpers shared by the GPU parity tests: upload with poisoned padding,
launch through the C ABI, read back with guard-band checks, and the two
comparison rules (bound and bit-exact).  Not a test module."""
import numpy as np
import torch

import oracle
from dense_half_precision_tiled_amd import inputs

DTYPES = {0: ("f16", "f32"), 1: ("f16", "f16"), 2: ("bf16", "f32"), 3: ("bf16", "bf16"),
          4: ("e4m3", "f32"), 5: ("e4m3", "f16"), 6: ("e4m3", "bf16"),
          7: ("e5m2", "f32"), 8: ("e5m2", "f16"), 9: ("e5m2", "bf16")}
POISON16 = 0x7E11      # a quiet-NaN pattern in both fp16 and bf16
POISON8 = 0x7F         # NaN in both E4M3 and E5M2
POISON32 = 0x7FC01234  # a quiet NaN in fp32
GUARD = 64             # guard elements before and after C


def _dev(bits, ld=None, offset=0):
    """Upload a rows x cols bit matrix (uint16, or uint8 for 8-bit inputs)
    into a buffer with row stride ld, starting `offset` elements into the
    allocation; padding is poisoned."""
    rows, cols = bits.shape
    ld = ld or cols
    esz = bits.dtype.itemsize
    buf = np.full(offset + max(rows * ld, 1) + 16, POISON16 if esz == 2 else POISON8, dtype=bits.dtype)
    if rows and cols:
        buf[offset:offset + rows * ld].reshape(rows, ld)[:, :cols] = bits
    t = torch.from_numpy(buf.view(np.int16) if esz == 2 else buf.view(np.int8)).cuda()
    return t, t.data_ptr() + esz * offset, ld


def decode_out(raw, out_fmt):
    if out_fmt == "f32":
        return raw.view(np.float32).astype(np.float64)
    if out_fmt == "f16":
        return raw.view(np.float16).astype(np.float64)
    with np.errstate(invalid="ignore"):
        return (raw.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def encode_out(values, out_fmt):
    """float64 values -> output-format bit patterns (RNE library casts)."""
    v = np.asarray(values, dtype=np.float64)
    if out_fmt == "f32":
        return v.astype(np.float32).view(np.uint32)
    if out_fmt == "f16":
        return v.astype(np.float16).view(np.uint16)
    return inputs.from_values(v, "bf16")


def run(G, A, B, code, lda=None, ldb=None, ldc=None, a_off=0, instance=None, stream=None,
        expect=0, layout=None, alpha=1.0, beta=0.0, bias=None, relu=0, c_init=None, c_off=0, ws=None):
    """C = A.B (or the general form) on the GPU; returns the decoded M x N result.

    B is the operand as stored: K x N for row-major, N x K for column-major
    (layout = G.GEMM_B_COL_MAJOR).  With layout None the call goes through
    gemm_run / gemm_run_instance, otherwise through the _ex entry points.
    c_init: M x N output-format bit patterns written into C before the call
    (default: poison).  bias: N float64 values or None.  c_off: C starts that
    many elements past the guard band (an odd c_off leaves a 2-byte-aligned C).
    ws: a device tensor used as the workspace of gemm_run_ws /
    gemm_run_instance_ws (the call then goes through those).
    Checks that the row padding of C and guard bands around it keep their
    poison."""
    M, K = A.shape
    N = B.shape[0] if layout == G.GEMM_B_COL_MAJOR else B.shape[1]
    out_fmt = DTYPES[code][1]
    tA, pA, lda = _dev(A, lda, a_off)
    tB, pB, ldb = _dev(B, ldb)
    ldc = ldc or N
    if out_fmt == "f32":
        cbuf = np.full(2 * GUARD + c_off + max(M * ldc, 1), POISON32, dtype=np.uint32)
        esz = 4
    else:
        cbuf = np.full(2 * GUARD + c_off + max(M * ldc, 1), POISON16, dtype=np.uint16)
        esz = 2
    if c_init is not None and M and N:
        cbuf[GUARD + c_off:GUARD + c_off + M * ldc].reshape(M, ldc)[:, :N] = c_init
    tC = torch.from_numpy(cbuf.view(np.int32 if esz == 4 else np.int16)).cuda()
    pC = tC.data_ptr() + esz * (GUARD + c_off)
    tbias = None
    pbias = None
    if bias is not None:
        tbias = torch.tensor(np.asarray(bias, dtype=np.float32), device="cuda")
        pbias = tbias.data_ptr()
    s = stream.cuda_stream if stream is not None else torch.cuda.current_stream().cuda_stream
    if ws is not None:
        lay = G.GEMM_B_ROW_MAJOR if layout is None else layout
        wsa = (ws.data_ptr(), ws.numel() * ws.element_size(), s)
        ex = (alpha, beta, pbias, relu)
        if instance is None:
            st = G.gemm_run_ws(M, N, K, code, lay, pA, lda, pB, ldb, pC, ldc, *ex, *wsa)
        else:
            st = G.gemm_run_instance_ws(instance, M, N, K, code, lay, pA, lda, pB, ldb, pC, ldc, *ex, *wsa)
    elif layout is None:
        if instance is None:
            st = G.gemm_run(M, N, K, code, pA, lda, pB, ldb, pC, ldc, s)
        else:
            st = G.gemm_run_instance(instance, M, N, K, code, pA, lda, pB, ldb, pC, ldc, s)
    else:
        ex = (alpha, beta, pbias, relu)
        if instance is None:
            st = G.gemm_run_ex(M, N, K, code, layout, pA, lda, pB, ldb, pC, ldc, *ex, s)
        else:
            st = G.gemm_run_instance_ex(instance, M, N, K, code, layout, pA, lda, pB, ldb, pC, ldc,
                                        *ex, s)
    assert st == expect, G.gemm_strerror(st)
    torch.cuda.synchronize()
    raw = tC.cpu().numpy().view(np.uint32 if esz == 4 else np.uint16)
    assert np.all(raw[:GUARD + c_off] == cbuf[:GUARD + c_off]) and np.all(raw[-GUARD:] == cbuf[-GUARD:]), \
        "guard band written"
    body = raw[GUARD + c_off:GUARD + c_off + M * ldc].reshape(M, ldc) if M else raw[:0].reshape(0, ldc)
    if ldc > N:
        assert np.all(body[:, N:] == (POISON32 if esz == 4 else POISON16)), "row padding of C written"
    del tbias
    return decode_out(np.ascontiguousarray(body[:, :N]), out_fmt)


def assert_bound(y, r, K, out_fmt, what="", extra=None):
    res = oracle.compare(y, r, K, out_fmt, extra=extra)
    assert res["ok"], "%s: %d elements outside the bound; max_abs %.3g, worst/bound %.3g" % (
        what, res["n_bad"], res["max_abs"], res["worst_ratio"])
    return res


def assert_exact(y, r, out_fmt, what=""):
    want = oracle.round_to(r, out_fmt)
    bad = ~((y == want) | (np.isnan(y) & np.isnan(want)))
    assert not bad.any(), "%s: %d elements differ, first at %s: %r vs %r" % (
        what, bad.sum(), np.argwhere(bad)[0], y[bad][0], want[bad][0])


def instances16(G):
    """Ids of the instances that run 16-bit inputs without a workspace (all but
    the dl8_* ones and the persistent pk_* ones, which need gemm_run_ws)."""
    return [i for i in range(G.gemm_num_instances())
            if not G.gemm_instance_name(i).startswith(("dl8_", "pk_"))]


def family(name):
    """Kernel family of an instance name: instances of one family do the same
    per-element arithmetic in the same order (dl and its persistent form pk
    are one family; pp splits the 256x256 tile among 8 waves but keeps the
    per-element k order of dl)."""
    f = name.split("_")[0]
    return "dl" if f in ("pk", "pp") else f


def law_for(fmt):
    return inputs.uniform if fmt == "f16" else inputs.normal
