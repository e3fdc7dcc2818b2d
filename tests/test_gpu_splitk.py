"""GPU parity of gemm_run_splitk (K cut into pieces computed by different
workgroups, partial tiles summed in piece order by a second kernel), through
the C ABI, against the oracle.

* with one piece the partial tile is the 256x256 kernel's fp32 accumulator,
  so the result equals gemm_run_instance_ex on that instance bit for bit
  (whole tiles and clamped edges, both B layouts, plain and general
  epilogue);
* on 0.25-grid inputs every partial sum is exact, so any number of pieces
  gives the oracle's value bit for bit;
* on random inputs every element lies within the bound of the general form;
* repeated calls give identical bits (the pieces are added in a fixed order);
* splits = 0 follows the library's rule: split where it pays, else exactly
  gemm_run_ex;
* 8-bit inputs split on their own 256x256 tile (one piece: that instance's
  bits; 0.25-grid inputs: exact; random data: within the bound);
* nothing outside the M x N region of C is written (checked by run()).
"""
import numpy as np
import pytest

import oracle
from dense_half_precision_tiled_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from tests.gpu_helpers import DTYPES, assert_exact, decode_out, encode_out, law_for, run  # noqa: E402


@pytest.fixture(scope="module")
def G():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from dense_half_precision_tiled_amd import gemm
    gemm.load()      # raises if the library is missing: no fallback
    return gemm


def _splitk(G, A, Bs, code, splits, col=False, alpha=1.0, beta=0.0, bias=None, relu=0, c_init=None, ws_pad=0):
    """C through gemm_run_splitk (B as stored: K x N, or N x K when col);
    returns the decoded M x N result."""
    M, K = A.shape
    N = Bs.shape[0] if col else Bs.shape[1]
    out = DTYPES[code][1]
    tA = torch.from_numpy(np.ascontiguousarray(A).view(np.int16)).cuda()
    tB = torch.from_numpy(np.ascontiguousarray(Bs).view(np.int16)).cuda()
    if c_init is not None:
        tC = torch.from_numpy(np.ascontiguousarray(c_init).view(np.int32 if out == "f32" else np.int16).copy()).cuda()
    else:
        tC = torch.full((M, N), -1, dtype=torch.int32 if out == "f32" else torch.int16, device="cuda")
    need = G.gemm_splitk_workspace_size(M, N, K, splits)
    assert need >= 0
    ws = torch.full((max(need // 4, 1) + ws_pad,), float("nan"), dtype=torch.float32, device="cuda")
    tb = torch.tensor(np.asarray(bias, dtype=np.float32), device="cuda") if bias is not None else None
    st = G.gemm_run_splitk(M, N, K, code, 1 if col else 0, tA.data_ptr(), K, tB.data_ptr(), K if col else N,
                           tC.data_ptr(), N, alpha, beta, tb.data_ptr() if tb is not None else None, relu, splits,
                           ws.data_ptr(), ws.numel() * 4, torch.cuda.current_stream().cuda_stream)
    assert st == 0, G.gemm_strerror(st)
    torch.cuda.synchronize()
    return decode_out(tC.cpu().numpy().view(np.uint32 if out == "f32" else np.uint16), out)


def _instance(G, name):
    return {G.gemm_instance_name(i): i for i in range(G.gemm_num_instances())}[name]


@pytest.mark.parametrize("col", [False, True])
@pytest.mark.parametrize("shape,inst", [((512, 768, 640), "dl_256x256x64_fd2"),
                                        ((300, 520, 301), "dl_256x256x64_fd2_clamp")])
@pytest.mark.parametrize("code,epi", [(0, False), (3, False), (1, True), (2, True)])
def test_one_piece_equals_the_256_instance(G, shape, inst, code, epi, col):
    M, N, K = shape
    fmt, out = DTYPES[code]
    A = law_for(fmt)((M, K), 500 + code, fmt)
    B = law_for(fmt)((K, N), 501 + code, fmt)
    Bs = np.ascontiguousarray(B.T) if col else B
    kw = dict(alpha=0.75, beta=-0.5, bias=np.linspace(-1, 1, N), relu=1) if epi else {}
    cold = np.random.Generator(np.random.PCG64(502)).uniform(-2, 2, (M, N)) if epi else None
    cbits = encode_out(cold, out) if epi else None
    print("split-K one piece", shape, code, epi, col, flush=True)
    y = _splitk(G, A, Bs, code, 1, col=col, c_init=cbits, **kw)
    ref = run(G, A, Bs, code, instance=_instance(G, inst), layout=G.GEMM_B_COL_MAJOR if col else G.GEMM_B_ROW_MAJOR,
              c_init=cbits, **kw)
    assert np.array_equal(y, ref)


@pytest.mark.parametrize("splits", [2, 3, 4, 8])
@pytest.mark.parametrize("shape,col", [((512, 512, 2048), False), ((300, 520, 4099), False),
                                       ((264, 250, 1000), True), ((1024, 256, 8192), False)])
def test_quarter_grid_bit_exact(G, shape, col, splits):
    M, N, K = shape
    A = inputs.quarter((M, K), 511, "bf16")
    B = inputs.quarter((K, N), 512, "bf16")
    Bs = np.ascontiguousarray(B.T) if col else B
    print("split-K quarter grid", shape, col, splits, flush=True)
    y = _splitk(G, A, Bs, 2, splits, col=col)
    assert_exact(y, oracle.gemm_f64(A, B, "bf16"), "f32", "split-K %s x%d" % (shape, splits))


@pytest.mark.parametrize("code", [0, 1, 2, 3])
@pytest.mark.parametrize("shape,splits,col", [((512, 512, 4096), 4, False), ((300, 264, 2500), 5, True),
                                              ((1000, 1016, 777), 3, False), ((256, 256, 64), 8, False)])
def test_random_inputs_within_bound(G, code, shape, splits, col):
    M, N, K = shape
    fmt, out = DTYPES[code]
    A = law_for(fmt)((M, K), 520 + code, fmt)
    B = law_for(fmt)((K, N), 521 + code, fmt)
    Bs = np.ascontiguousarray(B.T) if col else B
    bias = np.random.Generator(np.random.PCG64(522)).uniform(-1, 1, N)
    bias32 = bias.astype(np.float32).astype(np.float64)
    cold = decode_out(encode_out(np.random.Generator(np.random.PCG64(523)).uniform(-3, 3, (M, N)), out), out)
    print("split-K random", code, shape, splits, col, flush=True)
    y = _splitk(G, A, Bs, code, splits, col=col, alpha=1.5, beta=0.25, bias=bias, relu=1,
                c_init=encode_out(cold, out))
    lay = "col" if col else "row"
    r = oracle.gemm_ex_f64(A, Bs, fmt, b_layout=lay, alpha=1.5, beta=0.25, C_old=cold, bias=bias32, relu=True)
    dot = oracle.gemm_ex_f64(A, Bs, fmt, b_layout=lay)
    res = oracle.compare_ex(y, r, K, out, alpha=1.5, beta=0.25, C_old=cold, bias=bias32, dot=dot)
    assert res["ok"], res
    y0 = _splitk(G, A, Bs, code, splits, col=col)
    assert oracle.compare(y0, dot, K, out)["ok"]


def test_repeated_calls_identical_and_long_k(G):
    """A shape the split is for: 16 tiles of 256^2 and K = 16384, cut into
    16 pieces (256 workgroups); two calls give the same bits, and every
    element is within the bound."""
    M, N, K = 1024, 1024, 16384
    A = inputs.normal((M, K), 530, "bf16")
    B = inputs.normal((K, N), 531, "bf16")
    print("split-K long K", flush=True)
    y1 = _splitk(G, A, B, 3, 16)
    y2 = _splitk(G, A, B, 3, 16, ws_pad=1024)
    assert np.array_equal(y1, y2)
    res = oracle.compare(y1, oracle.gemm_f64(A, B, "bf16"), K, "bf16")
    assert res["ok"], res


def test_zero_k(G):
    M, N = 64, 48
    A = inputs.normal((M, 0), 540, "bf16")
    B = inputs.normal((0, N), 541, "bf16")
    cold = np.ones((M, N))
    y = _splitk(G, A, B, 2, 4, alpha=1.0, beta=2.0, c_init=encode_out(cold, "f32"))
    assert np.all(y == 2.0)


@pytest.mark.parametrize("col", [False, True])
@pytest.mark.parametrize("code", [4, 6, 8])
def test_8bit_inputs(G, code, col):
    """8-bit inputs on their 256x256 tile (128-deep slices, pieces of a
    multiple of 128): one piece equals the 8-bit 256x256 instance bit for bit;
    0.25-grid inputs give the oracle's value exactly (fp32 output) in any
    number of pieces; random data stays within the bound plus the 8-bit
    alignment envelope."""
    fmt, out = DTYPES[code]
    for (M, N, K), inst in (((512, 768, 1024), "dl8_256x256x128"), ((300, 528, 1100), "dl8_256x256x128_clamp")):
        A = inputs.normal((M, K), 560 + code, fmt)
        B = inputs.normal((K, N), 561 + code, fmt)
        Bs = np.ascontiguousarray(B.T) if col else B
        print("split-K 8-bit", code, col, (M, N, K), flush=True)
        y1 = _splitk8(G, A, Bs, code, 1, col)
        ref = run(G, A, Bs, code, instance=_instance(G, inst),
                  layout=G.GEMM_B_COL_MAJOR if col else G.GEMM_B_ROW_MAJOR)
        assert np.array_equal(y1, ref)
        y4 = _splitk8(G, A, Bs, code, 4, col)
        res = oracle.compare(y4, oracle.gemm_f64(A, B, fmt), K, out, extra=oracle.align_bound8(A, B, fmt))
        assert res["ok"], res
    M, N, K = 512, 528, 4096
    fq = "e4m3" if code <= 6 else "e5m2"
    A = inputs.quarter((M, K), 565, fq)
    B = inputs.quarter((K, N), 566, fq)
    Bs = np.ascontiguousarray(B.T) if col else B
    code32 = 4 if fq == "e4m3" else 7
    y = _splitk8(G, A, Bs, code32, 8, col)
    assert_exact(y, oracle.gemm_f64(A, B, fq), "f32", "split-K 8-bit quarter grid")


def _splitk8(G, A, Bs, code, splits, col):
    """gemm_run_splitk on 1-byte inputs (A M x K, B as stored)."""
    M, K = A.shape
    N = Bs.shape[0] if col else Bs.shape[1]
    out = DTYPES[code][1]
    tA = torch.from_numpy(np.ascontiguousarray(A)).cuda()
    tB = torch.from_numpy(np.ascontiguousarray(Bs)).cuda()
    tC = torch.full((M, N), -1, dtype=torch.int32 if out == "f32" else torch.int16, device="cuda")
    need = G.gemm_splitk_workspace_size(M, N, K, splits)
    ws = torch.full((max(need // 4, 1),), float("nan"), dtype=torch.float32, device="cuda")
    st = G.gemm_run_splitk(M, N, K, code, 1 if col else 0, tA.data_ptr(), K, tB.data_ptr(), K if col else N,
                           tC.data_ptr(), N, 1.0, 0.0, None, 0, splits, ws.data_ptr(), ws.numel() * 4,
                           torch.cuda.current_stream().cuda_stream)
    assert st == 0, G.gemm_strerror(st)
    torch.cuda.synchronize()
    return decode_out(tC.cpu().numpy().view(np.uint32 if out == "f32" else np.uint16), out)


def test_library_choice(G):
    """splits = 0: a long-K shape with few tiles is split as the rule says (the
    same bits as asking for that count), and a shape the rule leaves unsplit
    runs gemm_run_ex's kernels without touching a workspace."""
    M, N, K = 1024, 1024, 16384
    A = inputs.normal((M, K), 550, "bf16")
    B = inputs.normal((K, N), 551, "bf16")
    assert G.gemm_splitk_workspace_size(M, N, K, 0) == G.gemm_splitk_workspace_size(M, N, K, 12)
    print("split-K library choice", flush=True)
    assert np.array_equal(_splitk(G, A, B, 3, 0), _splitk(G, A, B, 3, 12))
    M, N, K = 512, 512, 2048
    A = inputs.normal((M, K), 552, "bf16")
    B = inputs.normal((K, N), 553, "bf16")
    assert G.gemm_splitk_workspace_size(M, N, K, 0) == 0
    tA = torch.from_numpy(A.view(np.int16)).cuda()
    tB = torch.from_numpy(B.view(np.int16)).cuda()
    tC = torch.full((M, N), -1, dtype=torch.int16, device="cuda")
    st = G.gemm_run_splitk(M, N, K, 3, 0, tA.data_ptr(), K, tB.data_ptr(), N, tC.data_ptr(), N, 1.0, 0.0, None, 0,
                           0, None, 0, torch.cuda.current_stream().cuda_stream)
    assert st == 0, G.gemm_strerror(st)
    torch.cuda.synchronize()
    y = decode_out(tC.cpu().numpy().view(np.uint16), "bf16")
    assert np.array_equal(y, run(G, A, B, 3, layout=G.GEMM_B_ROW_MAJOR))


def test_random_sweep(G):
    """Seeded random cases: ragged shapes, every dtype, both B layouts, the
    general epilogue, 0 (the library's choice) to 9 pieces; every element
    against the oracle (plus the 8-bit alignment envelope for 8-bit inputs)."""
    rng = np.random.Generator(np.random.PCG64(20261203))
    dims = [1, 17, 64, 200, 256, 257, 300, 511, 520, 528]
    ran = 0
    for case in range(80):
        M, N = int(rng.choice(dims)), int(rng.choice(dims))
        K = int(rng.choice([1, 63, 64, 130, 700, 1100, 2048, 4099, 5000]))
        code = int(rng.integers(0, 10))
        col = bool(rng.random() < 0.5)
        splits = int(rng.integers(0, 10))
        fmt, out = DTYPES[code]
        if not col and N % (16 if fmt in ("e4m3", "e5m2") else 8) != 0 and (M % 256 or N % 256):
            N = N + (-N) % 16                    # row-major B with a partial tile: whole 16-byte column chunks
        epi = rng.random() < 0.5
        alpha = float(rng.choice([1.0, -0.5, 2.0])) if epi else 1.0
        beta = float(rng.choice([0.0, 1.0])) if epi else 0.0
        bias = rng.uniform(-1, 1, N) if epi and rng.random() < 0.5 else None
        relu = int(epi and rng.random() < 0.5)
        A = law_for(fmt)((M, K), 7000 + 2 * case, fmt) if fmt not in ("e4m3", "e5m2") else \
            inputs.normal((M, K), 7000 + 2 * case, fmt)
        B = law_for(fmt)((K, N), 7001 + 2 * case, fmt) if fmt not in ("e4m3", "e5m2") else \
            inputs.normal((K, N), 7001 + 2 * case, fmt)
        Bs = np.ascontiguousarray(B.T) if col else B
        cold = decode_out(encode_out(rng.uniform(-2, 2, (M, N)), out), out)
        print("split-K sweep", case, (M, N, K), code, col, splits, epi, flush=True)
        if fmt in ("e4m3", "e5m2"):
            y = _splitk8_ex(G, A, Bs, code, splits, col, alpha, beta, bias, relu, encode_out(cold, out))
        else:
            y = _splitk(G, A, Bs, code, splits, col=col, alpha=alpha, beta=beta, bias=bias, relu=relu,
                        c_init=encode_out(cold, out))
        lay = "col" if col else "row"
        bias32 = None if bias is None else bias.astype(np.float32).astype(np.float64)
        r = oracle.gemm_ex_f64(A, Bs, fmt, b_layout=lay, alpha=alpha, beta=beta, C_old=cold, bias=bias32,
                               relu=bool(relu))
        dot = oracle.gemm_ex_f64(A, Bs, fmt, b_layout=lay)
        extra = oracle.align_bound8(A, B, fmt) if fmt in ("e4m3", "e5m2") else None
        res = oracle.compare_ex(y, r, K, out, alpha=alpha, beta=beta, C_old=cold, bias=bias32, dot=dot,
                                extra=extra)
        assert res["ok"], (case, res)
        ran += 1
    assert ran == 80


def _splitk8_ex(G, A, Bs, code, splits, col, alpha, beta, bias, relu, cbits):
    M, K = A.shape
    N = Bs.shape[0] if col else Bs.shape[1]
    out = DTYPES[code][1]
    tA = torch.from_numpy(np.ascontiguousarray(A)).cuda()
    tB = torch.from_numpy(np.ascontiguousarray(Bs)).cuda()
    tC = torch.from_numpy(np.ascontiguousarray(cbits).view(np.int32 if out == "f32" else np.int16).copy()).cuda()
    need = G.gemm_splitk_workspace_size(M, N, K, splits)
    ws = torch.full((max(need // 4, 1),), float("nan"), dtype=torch.float32, device="cuda")
    tb = torch.tensor(np.asarray(bias, dtype=np.float32), device="cuda") if bias is not None else None
    st = G.gemm_run_splitk(M, N, K, code, 1 if col else 0, tA.data_ptr(), K, tB.data_ptr(), K if col else N,
                           tC.data_ptr(), N, alpha, beta, tb.data_ptr() if tb is not None else None, relu, splits,
                           ws.data_ptr(), ws.numel() * 4, torch.cuda.current_stream().cuda_stream)
    assert st == 0, G.gemm_strerror(st)
    torch.cuda.synchronize()
    return decode_out(tC.cpu().numpy().view(np.uint32 if out == "f32" else np.uint16), out)
