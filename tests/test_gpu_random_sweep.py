"""Seeded random sweep of the boundary against the oracle.

Each case draws a shape (including ragged edges, tiny and one-sided sizes),
padded or 2-byte-misaligned leading dimensions and base offset, a dtype pair,
a B layout, an epilogue (alpha, beta, bias, ReLU) and either the library's
own instance choice or a forced instance that can run the shape, then checks
every element of the result against the fp64 oracle within the bound of the
general form (the accumulation bound scaled by alpha, plus the epilogue's
fp32 roundings and one ulp of a half-precision output), and that nothing
outside the M x N region of C is written (checked by the run helper).
"""
import numpy as np
import pytest

import oracle
from dense_half_precision_tiled_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from tests.gpu_helpers import DTYPES, decode_out, encode_out, law_for, run  # noqa: E402

N_CASES = 200


@pytest.fixture(scope="module")
def G():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from dense_half_precision_tiled_amd import gemm
    gemm.load()      # raises if the library is missing: no fallback
    return gemm


def _draw(rng, G, n_inst):
    dims = [1, 2, 7, 8, 31, 64, 65, 127, 128, 129, 200, 255, 256, 257, 384, 511, 640]
    M, N, K = (int(rng.choice(dims)) for _ in range(3))
    if rng.random() < 0.2:
        K = int(rng.choice([2048, 2112]))
        M, N = int(rng.choice([256, 384])), int(rng.choice([256, 264]))
    code = int(rng.integers(0, 4))
    col = bool(rng.random() < 0.4)
    pad = rng.random() < 0.5
    lda = K + (int(rng.integers(1, 24)) if pad else 0)
    ldb_min = K if col else N
    ldb = ldb_min + (int(rng.integers(1, 24)) if pad else 0)
    ldc = N + (int(rng.integers(1, 24)) if pad else 0)
    a_off = int(rng.integers(0, 8)) if rng.random() < 0.3 else 0
    epi = rng.random() < 0.5
    alpha = float(rng.choice([1.0, 0.5, -2.0, 1.25])) if epi else 1.0
    beta = float(rng.choice([0.0, 1.0, -0.5])) if epi else 0.0
    use_bias = bool(epi and rng.random() < 0.5)
    relu = int(epi and rng.random() < 0.5)
    inst = None
    if rng.random() < 0.4:
        inst = int(rng.integers(0, n_inst))
    return dict(M=M, N=N, K=K, code=code, col=col, lda=lda, ldb=ldb, ldc=ldc, a_off=a_off, alpha=alpha,
                beta=beta, use_bias=use_bias, relu=relu, inst=inst)


def test_random_sweep(G):
    rng = np.random.Generator(np.random.PCG64(20260101))
    n_inst = G.gemm_num_instances()
    ran = refused = 0
    for case in range(N_CASES):
        c = _draw(rng, G, n_inst)
        M, N, K, code = c["M"], c["N"], c["K"], c["code"]
        fmt, out = DTYPES[code]
        A = law_for(fmt)((M, K), 9000 + 3 * case, fmt)
        B = law_for(fmt)((K, N), 9001 + 3 * case, fmt)
        Bs = np.ascontiguousarray(B.T) if c["col"] else B
        cold_v = np.random.Generator(np.random.PCG64(9002 + 3 * case)).uniform(-4, 4, (M, N))
        cbits = encode_out(cold_v, out)
        cold = decode_out(cbits, out)
        bias = np.random.Generator(np.random.PCG64(50 + case)).uniform(-2, 2, N) if c["use_bias"] else None
        bias32 = None if bias is None else bias.astype(np.float32).astype(np.float64)
        layout = G.GEMM_B_COL_MAJOR if c["col"] else G.GEMM_B_ROW_MAJOR
        expect = 0
        # the drawn arguments are valid: the library picks an instance for them
        assert G.gemm_select_instance_ex(M, N, K, code, layout, 1 << 32, c["lda"], 1 << 36, c["ldb"],
                                         1 << 40, c["ldc"], c["alpha"], c["beta"], None, c["relu"]) >= 0
        desc = "case %d %s" % (case, c)
        print(desc, flush=True)
        # a persistent instance runs through gemm_run_instance_ws with a fresh workspace
        ws = None
        if c["inst"] is not None and G.gemm_instance_name(c["inst"]).startswith("pk_"):
            ws = torch.zeros(G.gemm_workspace_size() // 4, dtype=torch.int32, device="cuda")
        try:
            y = run(G, A, Bs, code, lda=c["lda"], ldb=c["ldb"], ldc=c["ldc"], a_off=c["a_off"],
                    instance=c["inst"], layout=layout, alpha=c["alpha"], beta=c["beta"], bias=bias,
                    relu=c["relu"], c_init=cbits, expect=expect, ws=ws)
        except AssertionError as e:
            # a forced instance that cannot run the shape refuses it before any launch
            if c["inst"] is not None and "cannot run this shape" in str(e):
                refused += 1
                continue
            raise
        ran += 1
        r = oracle.gemm_ex_f64(A, Bs, fmt, b_layout="col" if c["col"] else "row", alpha=c["alpha"],
                               beta=c["beta"], C_old=cold, bias=bias32, relu=bool(c["relu"]))
        dot = oracle.gemm_ex_f64(A, Bs, fmt, b_layout="col" if c["col"] else "row")
        res = oracle.compare_ex(y, r, K, out, alpha=c["alpha"], beta=c["beta"], C_old=cold, bias=bias32,
                                dot=dot)
        assert res["ok"], "%s: %s" % (desc, res)
    print("ran", ran, "refused", refused, flush=True)
    assert ran >= N_CASES // 2


N_CASES8 = 120


def test_random_sweep_8bit(G):
    """The same sweep for the 8-bit inputs (E4M3 / E5M2, every output type):
    both B layouts, odd leading dimensions and byte offsets, epilogues, and
    forced 8-bit instances; the bound adds the 8-bit MFMA's alignment loss."""
    rng = np.random.Generator(np.random.PCG64(20260202))
    ids8 = [i for i in range(G.gemm_num_instances()) if G.gemm_instance_name(i).startswith("dl8_")]
    dims = [1, 3, 16, 17, 64, 100, 127, 128, 129, 255, 256, 257, 300, 513]
    ran = refused = 0
    for case in range(N_CASES8):
        M, N, K = (int(rng.choice(dims)) for _ in range(3))
        if rng.random() < 0.2:
            K = int(rng.choice([1024, 1100]))
            M, N = int(rng.choice([256, 384])), int(rng.choice([256, 272]))
        code = int(rng.integers(4, 10))
        col = bool(rng.random() < 0.5)
        pad = rng.random() < 0.5
        lda = K + (int(rng.integers(1, 24)) if pad else 0)
        ldb = (K if col else N) + (int(rng.integers(1, 24)) if pad else 0)
        ldc = N + (int(rng.integers(1, 24)) if pad else 0)
        a_off = int(rng.integers(0, 16)) if rng.random() < 0.3 else 0
        epi = rng.random() < 0.5
        alpha = float(rng.choice([1.0, 0.5, -2.0])) if epi else 1.0
        beta = float(rng.choice([0.0, 1.0, -0.5])) if epi else 0.0
        use_bias = bool(epi and rng.random() < 0.5)
        relu = int(epi and rng.random() < 0.5)
        inst = int(rng.choice(ids8)) if rng.random() < 0.4 else None
        fmt, out = DTYPES[code]
        A = inputs.normal((M, K), 19000 + 3 * case, fmt)
        B = inputs.normal((K, N), 19001 + 3 * case, fmt)
        Bs = np.ascontiguousarray(B.T) if col else B
        cold = decode_out(encode_out(np.random.Generator(np.random.PCG64(19002 + 3 * case)).uniform(-4, 4, (M, N)),
                                     out), out)
        bias = np.random.Generator(np.random.PCG64(500 + case)).uniform(-2, 2, N) if use_bias else None
        bias32 = None if bias is None else bias.astype(np.float32).astype(np.float64)
        layout = G.GEMM_B_COL_MAJOR if col else G.GEMM_B_ROW_MAJOR
        desc = "case %d M %d N %d K %d code %d col %s lda %d ldb %d ldc %d off %d inst %s" % (
            case, M, N, K, code, col, lda, ldb, ldc, a_off, inst)
        print(desc, flush=True)
        try:
            y = run(G, A, Bs, code, lda=lda, ldb=ldb, ldc=ldc, a_off=a_off, instance=inst, layout=layout,
                    alpha=alpha, beta=beta, bias=bias, relu=relu, c_init=encode_out(cold, out))
        except AssertionError as e:
            if inst is not None and "cannot run this shape" in str(e):
                refused += 1
                continue
            raise
        ran += 1
        lay = "col" if col else "row"
        r = oracle.gemm_ex_f64(A, Bs, fmt, b_layout=lay, alpha=alpha, beta=beta, C_old=cold, bias=bias32,
                               relu=bool(relu))
        dot = oracle.gemm_ex_f64(A, Bs, fmt, b_layout=lay)
        res = oracle.compare_ex(y, r, K, out, alpha=alpha, beta=beta, C_old=cold, bias=bias32, dot=dot,
                                extra=oracle.align_bound8(A, B, fmt))
        assert res["ok"], "%s: %s" % (desc, res)
    print("8-bit sweep: ran", ran, "refused", refused, flush=True)
    assert ran >= N_CASES8 // 2
