"""Lane-layout pins for the gfx950 instructions the GEMM kernels rely on, and
the MFMA issue-rate measurement (the register-resident rate probe of the Ada
tensor-core GEMM write-up, its table of measured mma rates per clock and its
warning about measuring against the clock actually held: FLOP per clock per
compute unit from an in-kernel clock, independent of the clock frequency).

Every probe runs one wave on buffers it owns; addresses are checked here and
masked in the kernel."""
import ctypes
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "tests", "probes", "libdhpt_probes.so")


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__.build_probes()
    lib = ctypes.CDLL(LIB)
    vp = ctypes.c_void_p
    lib.probe_tr16.argtypes = [vp, vp]
    lib.probe_load_lds.argtypes = [vp, vp, ctypes.c_int, vp]
    lib.probe_mfma.argtypes = [ctypes.c_int, vp, vp, vp]
    lib.probe_mfma_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp]
    lib.probe_lds_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp]
    lib.probe_dma_rate.argtypes = [ctypes.c_int, ctypes.c_int, vp, ctypes.c_int, vp, vp]
    lib.probe_mfma_f8.argtypes = [ctypes.c_int, vp, vp, vp]
    lib.probe_tr8.argtypes = [vp, ctypes.c_int, vp]
    lib.probe_tr8.restype = ctypes.c_int
    lib.probe_mfma_f8_acc.argtypes = [ctypes.c_int, vp, vp, vp, vp]
    lib.probe_mfma_f8_acc.restype = ctypes.c_int
    lib.probe_mfma_f8_rate.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp]
    for f in (lib.probe_tr16, lib.probe_load_lds, lib.probe_mfma, lib.probe_mfma_rate,
              lib.probe_lds_rate, lib.probe_dma_rate, lib.probe_mfma_f8, lib.probe_mfma_f8_rate):
        f.restype = ctypes.c_int
    return lib


@pytest.mark.parametrize("pattern", ["linear", "perm5", "rows32"])
def test_ds_read_tr16_b64_layout(P, pattern):
    """Within each group of 16 lanes, lane i receives element i % 4 of the
    8-byte rows addressed by lanes 4j + i/4 of its group, j = 0..3: one read
    hands every lane a column of a 4 x 16 block of 16-bit values."""
    addr = {"linear": [8 * l for l in range(64)],
            "perm5": [8 * ((5 * l) % 64) for l in range(64)],
            "rows32": [32 * (l % 16) + 8 * (l // 16) + 512 for l in range(64)]}[pattern]
    assert all(a % 8 == 0 and 0 <= a <= 2040 for a in addr)
    a = torch.tensor(addr, dtype=torch.int32, device="cuda")
    o = torch.zeros(256, dtype=torch.int16, device="cuda")
    assert P.probe_tr16(a.data_ptr(), o.data_ptr()) == 0
    got = o.cpu().numpy().reshape(64, 4).astype(np.int64)
    for l in range(64):
        g, i = l // 16, l % 16
        for j in range(4):
            src_lane = 16 * g + 4 * j + i // 4
            assert got[l, j] == addr[src_lane] // 2 + i % 4, (l, j)


@pytest.mark.parametrize("pattern", ["linear", "perm5", "rows16"])
def test_ds_read_tr8_b64_layout(P, pattern):
    """Within each group of 16 lanes, lane i receives byte i % 8 of the 8-byte
    rows addressed by lanes 2j + i/8 of its group, j = 0..7: one read hands
    every lane a column of an 8 x 16 block of bytes (8 values of k of one
    column of a row-major 8-bit tile).  Each source byte is named by two runs
    (LDS byte n holds n & 255, then n >> 8)."""
    addr = {"linear": [8 * l for l in range(64)],
            "perm5": [8 * ((5 * l) % 64) for l in range(64)],
            "rows16": [128 * ((l % 16) // 2) + 8 * (l % 2) + 16 * (l // 16) for l in range(64)]}[pattern]
    assert all(a % 8 == 0 and 0 <= a <= 2040 for a in addr)
    a = torch.tensor(addr, dtype=torch.int32, device="cuda")
    src = np.zeros(512, np.int64)
    for shift in (0, 8):
        o = torch.zeros(512, dtype=torch.uint8, device="cuda")
        assert P.probe_tr8(a.data_ptr(), shift, o.data_ptr()) == 0
        src += o.cpu().numpy().astype(np.int64) << shift
    src = src.reshape(64, 8)
    for l in range(64):
        g, i = l // 16, l % 16
        for j in range(8):
            assert src[l, j] == addr[16 * g + 2 * j + i // 8] + i % 8, (l, j)


def test_global_load_lds_dwordx4_layout(P):
    """Lane l's 16 bytes land at LDS base + 16*l; nothing else is written."""
    src = torch.arange(256, dtype=torch.int32, device="cuda")
    chunks = [(7 * l) % 64 for l in range(64)]
    ch = torch.tensor(chunks, dtype=torch.int32, device="cuda")
    out = torch.zeros(1024, dtype=torch.int32, device="cuda")
    base = 256
    assert P.probe_load_lds(src.data_ptr(), ch.data_ptr(), base, out.data_ptr()) == 0
    lds = out.cpu().numpy().astype(np.int64)
    for l in range(64):
        assert lds[base // 4 + 4 * l: base // 4 + 4 * l + 4].tolist() == list(range(4 * chunks[l], 4 * chunks[l] + 4))
    rest = np.concatenate([lds[:base // 4], lds[base // 4 + 256:]])
    assert np.all(rest == -1)


@pytest.mark.parametrize("kind", [0, 1, 2, 3])
def test_mfma_operand_and_accumulator_maps(P, kind):
    """32x32x16: A row l%32, B column l%32, 8 values of k = 8(l/32)+j; D
    element i of lane l is row 8(i/4) + 4(l/32) + i%4, column l%32.
    16x16x32: A row l%16, B column l%16, k = 8(l/16)+j; D element i is row
    4(l/16) + i, column l%16."""
    rng = np.random.Generator(np.random.PCG64(10 + kind))
    a = rng.integers(-3, 4, 512).astype(np.float32)
    b = rng.integers(-3, 4, 512).astype(np.float32)
    dt = torch.bfloat16 if kind in (1, 3) else torch.float16
    ta = torch.from_numpy(a).to(dt).cuda().view(torch.int16)
    tb = torch.from_numpy(b).to(dt).cuda().view(torch.int16)
    td = torch.zeros(1024, dtype=torch.float32, device="cuda")
    assert P.probe_mfma(kind, ta.data_ptr(), tb.data_ptr(), td.data_ptr()) == 0
    d = td.cpu().numpy().astype(np.float64)
    a = a.reshape(64, 8)
    b = b.reshape(64, 8)
    if kind in (0, 1):
        A = np.zeros((32, 16)); B = np.zeros((16, 32)); got = np.zeros((32, 32))
        for l in range(64):
            A[l % 32, 8 * (l // 32):8 * (l // 32) + 8] = a[l]
            B[8 * (l // 32):8 * (l // 32) + 8, l % 32] = b[l]
            for i in range(16):
                got[8 * (i // 4) + 4 * (l // 32) + i % 4, l % 32] = d[16 * l + i]
    else:
        A = np.zeros((16, 32)); B = np.zeros((32, 16)); got = np.zeros((16, 16))
        for l in range(64):
            A[l % 16, 8 * (l // 16):8 * (l // 16) + 8] = a[l]
            B[8 * (l // 16):8 * (l // 16) + 8, l % 16] = b[l]
            for i in range(4):
                got[4 * (l // 16) + i, l % 16] = d[4 * l + i]
    assert np.array_equal(got, A @ B)


def _run_mfma_f8(P, fmt, A_codes, B_codes):
    """One v_mfma_f32_32x32x64_f8f6f4 on a 32 x 64 A and a 64 x 32 B of 8-bit
    codes, placed as the GEMM kernels place them: lane l holds row (A) or
    column (B) l % 32 and the 32 consecutive k from 32 (l / 32); the 32 x 32
    result is read with the 32x32 accumulator map of test_mfma_operand_and_accumulator_maps."""
    a = np.zeros((64, 32), np.uint8)
    b = np.zeros((64, 32), np.uint8)
    for l in range(64):
        a[l] = A_codes[l % 32, 32 * (l // 32):32 * (l // 32) + 32]
        b[l] = B_codes[32 * (l // 32):32 * (l // 32) + 32, l % 32]
    ta = torch.from_numpy(a.reshape(-1).view(np.int32).copy()).cuda()
    tb = torch.from_numpy(b.reshape(-1).view(np.int32).copy()).cuda()
    td = torch.zeros(1024, dtype=torch.float32, device="cuda")
    assert P.probe_mfma_f8(0 if fmt == "e4m3" else 1, ta.data_ptr(), tb.data_ptr(), td.data_ptr()) == 0
    d = td.cpu().numpy().astype(np.float64)
    got = np.zeros((32, 32))
    for l in range(64):
        for i in range(16):
            got[8 * (i // 4) + 4 * (l // 32) + i % 4, l % 32] = d[16 * l + i]
    return got


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_mfma_f8_operand_map(P, fmt):
    """With A and B placed alike (lane half h and byte p both mean k = 32h + p),
    the 8-bit MFMA returns exactly A.B: the k assignment the kernels rely on is
    shared by the two operands."""
    import oracle
    from dense_half_precision_tiled_amd import inputs
    for seed in (1, 2, 3):
        A = inputs.ints((32, 64), 70 + seed, fmt)
        B = inputs.ints((64, 32), 80 + seed, fmt)
        want = oracle.decode(A, fmt) @ oracle.decode(B, fmt)
        assert np.array_equal(_run_mfma_f8(P, fmt, A, B), want)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_mfma_f8_decodes_every_code(P, fmt):
    """Every finite code, multiplied by 1.0 and summed with exact zeros, comes
    back as the oracle's OFP8 value: the MFMA reads E4M3 / E5M2 as the OCP
    formats.  (NaN and infinity codes are left out: they would poison every
    sum of their row.)"""
    import oracle
    codes = ((64 * np.arange(32)[:, None] + np.arange(64)[None, :]) % 256).astype(np.uint8)
    vals = oracle.decode(codes, fmt)
    codes = np.where(np.isfinite(vals), codes, 0).astype(np.uint8)
    vals = oracle.decode(codes, fmt)
    one = 0x38 if fmt == "e4m3" else 0x3C
    for t in (0, 1):                   # B selects k = j + 32 t for column j
        B = np.zeros((64, 32), np.uint8)
        B[np.arange(32) + 32 * t, np.arange(32)] = one
        got = _run_mfma_f8(P, fmt, codes, B)
        assert np.array_equal(got, vals[:, 32 * t:32 * t + 32]), t


def _run_mfma_f8_acc(P, fmt, A_codes, B_codes, Cm):
    """As _run_mfma_f8, with the 32 x 32 accumulator Cm fed in (same map)."""
    a = np.zeros((64, 32), np.uint8)
    b = np.zeros((64, 32), np.uint8)
    c = np.zeros(1024, np.float32)
    for l in range(64):
        a[l] = A_codes[l % 32, 32 * (l // 32):32 * (l // 32) + 32]
        b[l] = B_codes[32 * (l // 32):32 * (l // 32) + 32, l % 32]
        for i in range(16):
            c[16 * l + i] = Cm[8 * (i // 4) + 4 * (l // 32) + i % 4, l % 32]
    ta = torch.from_numpy(a.reshape(-1).view(np.int32).copy()).cuda()
    tb = torch.from_numpy(b.reshape(-1).view(np.int32).copy()).cuda()
    tc = torch.from_numpy(c).cuda()
    td = torch.zeros(1024, dtype=torch.float32, device="cuda")
    assert P.probe_mfma_f8_acc(0 if fmt == "e4m3" else 1, ta.data_ptr(), tb.data_ptr(), tc.data_ptr(),
                               td.data_ptr()) == 0
    d = td.cpu().numpy().astype(np.float64)
    got = np.zeros((32, 32))
    for l in range(64):
        for i in range(16):
            got[8 * (i // 4) + 4 * (l // 32) + i % 4, l % 32] = d[16 * l + i]
    return got


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_mfma_f8_alignment_model(P, fmt):
    """The summation arithmetic the 8-bit tolerance (oracle.align_bound8) is
    derived from: (1) a product 2^-x beside a product 1 of the same group
    survives for x <= 13 and is dropped (cut toward zero) for x >= 14, either
    sign; (2) the groups are the runs of 8 consecutive k; (3) the incoming
    accumulator is not cut: C = 1 plus a lone product 2^-x keeps it to x = 18."""
    import oracle
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.decode(codes, fmt)
    enc = {float(v): int(c) for c, v in zip(codes, vals) if np.isfinite(v) and c != 0x80}
    E = lambda x: enc[float(x)]
    # (1) rows: small factor 2^-e (e = i % 10, negative for i >= 16); columns: 2^-f
    A = np.zeros((32, 64), np.uint8)
    B = np.zeros((64, 32), np.uint8)
    for i in range(32):
        A[i, 0], A[i, 1] = E(1.0), E((-1.0 if i >= 16 else 1.0) * 2.0 ** -(i % 10))
    for j in range(32):
        B[0, j], B[1, j] = E(1.0), E(2.0 ** -(j % 10))
    got = _run_mfma_f8(P, fmt, A, B)
    for i in range(32):
        for j in range(32):
            x, sgn = i % 10 + j % 10, (-1.0 if i >= 16 else 1.0)
            assert got[i, j] == (1.0 + sgn * 2.0 ** -x if x <= 13 else 1.0), (i, j)
    # (2) a product 2^-14 at k' is dropped iff k' shares the run of 8 with the product 1 at `anchor`
    for anchor in (0, 13, 40, 63):
        for half in (0, 1):
            A = np.zeros((32, 64), np.uint8)
            B = np.zeros((64, 32), np.uint8)
            for i in range(32):
                kp = 32 * half + i
                A[i, anchor] = E(1.0)
                if kp != anchor:
                    A[i, kp] = E(2.0 ** -7)
            B[:, :] = E(2.0 ** -7)
            B[anchor, :] = E(1.0)
            got = _run_mfma_f8(P, fmt, A, B)[:, 0]
            for i in range(32):
                kp = 32 * half + i
                if kp == anchor:
                    continue
                same = kp // 8 == anchor // 8
                assert got[i] == (1.0 if same else 1.0 + 2.0 ** -14), (anchor, kp)
    # (3) the accumulator: C = 1 plus one product 2^-x, x = e + f up to 18
    A = np.zeros((32, 64), np.uint8)
    B = np.zeros((64, 32), np.uint8)
    for i in range(32):
        A[i, 0] = E(2.0 ** -(i % 10))
    for j in range(32):
        B[0, j] = E(2.0 ** -(j % 10))
    got = _run_mfma_f8_acc(P, fmt, A, B, np.ones((32, 32)))
    want = 1.0 + oracle.decode(A, fmt) @ oracle.decode(B, fmt)
    assert np.array_equal(got, want)


def test_mfma_f8_issue_rate(P):
    """Eight independent v_mfma_f32_32x32x64_f8f6f4 per wave, one wave per SIMD
    on every CU: FLOP per shader clock per CU against the 8192 of the CDNA4
    design for 8-bit inputs (twice the 16-bit rate)."""
    blocks, iters = 256, 2000
    cyc = torch.zeros(blocks * 4, dtype=torch.int64, device="cuda")
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    P.probe_mfma_f8_rate(blocks, 100, cyc.data_ptr(), sink.data_ptr())
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    assert P.probe_mfma_f8_rate(blocks, iters, cyc.data_ptr(), sink.data_ptr()) == 0
    e1.record()
    torch.cuda.synchronize()
    cycles = float(cyc.cpu().numpy().mean())
    flop = 4 * iters * 8 * 131072.0
    ms = e0.elapsed_time(e1)
    print("mfma e4m3: %.0f FLOP/clk/CU, %.0f TFLOP/s" % (flop / cycles, blocks * flop / ms / 1e9))
    assert 7000 < flop / cycles <= 8192 * 1.01


def test_mfma_issue_rate(P):
    """Eight independent v_mfma_f32_32x32x16 per wave, one wave per SIMD on
    every CU: FLOP per shader clock per CU should be the 4096 of the CDNA4
    design (32768 FLOP every 32 cycles on each of 4 SIMDs)."""
    blocks, iters = 256, 4000
    cyc = torch.zeros(blocks * 4, dtype=torch.int64, device="cuda")
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    for bf16 in (0, 1):
        P.probe_mfma_rate(bf16, blocks, 100, cyc.data_ptr(), sink.data_ptr())     # warm
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        assert P.probe_mfma_rate(bf16, blocks, iters, cyc.data_ptr(), sink.data_ptr()) == 0
        e1.record()
        torch.cuda.synchronize()
        cycles = float(cyc.cpu().numpy().mean())
        flop_per_clk_cu = 4 * iters * 8 * 32768.0 / cycles
        ms = e0.elapsed_time(e1)
        clock_ghz = cycles / (ms * 1e-3) / 1e9
        print("mfma %s: %.0f FLOP/clk/CU, shader clock under load ~%.2f GHz, %.0f TFLOP/s" % (
            "bf16" if bf16 else "f16", flop_per_clk_cu, clock_ghz, blocks * 4 * iters * 8 * 32768 / ms / 1e9))
        assert 3500 < flop_per_clk_cu <= 4096 * 1.01


def _a_fragment_addresses(row_bytes):
    """The GEMM's A-fragment reads: wave (wm, wn) = (w >> 1, w & 1), lane l reads
    row wm*128 + (l & 31), logical chunk l >> 5, XOR-swizzled as in the kernel."""
    out = []
    for w in range(4):
        for l in range(64):
            r = (w >> 1) * 128 + (l & 31)
            c = l >> 5
            out.append(r * row_bytes + 16 * (c ^ (r & 7) ^ ((r >> 3) & 1)))
    return out


def _b_fragment_addresses(swizzle):
    """The GEMM's B-fragment transposing reads (512-byte rows of k)."""
    out = []
    for w in range(4):
        for l in range(64):
            g, ip = l >> 4, l & 15
            k = 8 * (g >> 1) + (ip >> 2)
            n = (w & 1) * 128 + 16 * (g & 1) + 4 * (ip & 3)
            out.append(k * 512 + (((n >> 3) ^ swizzle(k)) * 16) + (n & 7) * 2)
    return out


def test_lds_read_rate(P):
    """LDS cost of the fragment-read instructions in shader clocks per
    instruction per CU (4 waves per CU).  Recorded, gated only for sanity;
    the GEMM's swizzles are the ones that measured fastest here."""
    blocks, iters = 256, 1500
    cyc = torch.zeros(blocks * 4, dtype=torch.int64, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    cases = [
        ("ds_read_b128 A fragments, swizzled", 0, 1024, _a_fragment_addresses(128)),
        ("ds_read_b128 A fragments, unswizzled", 0, 1024,
         [((w >> 1) * 128 + (l & 31)) * 128 + 16 * (l >> 5) for w in range(4) for l in range(64)]),
        ("ds_read_b128 consecutive", 0, 1024, [w * 1024 + 16 * l for w in range(4) for l in range(64)]),
        ("ds_read_b64 consecutive", 1, 512, [w * 512 + 8 * l for w in range(4) for l in range(64)]),
        ("ds_read_b64_tr_b16 B fragments, c^2(k&3)", 2, 512, _b_fragment_addresses(lambda k: 2 * (k & 3))),
        ("ds_read_b64_tr_b16 B fragments, unswizzled", 2, 512, _b_fragment_addresses(lambda k: 0)),
        ("ds_write_b128 consecutive", 3, 1024, [w * 1024 + 16 * l for w in range(4) for l in range(64)]),
    ]
    res = {}
    for name, kind, nbytes, addr in cases:
        assert len(addr) == 256 and all(0 <= a < 65536 for a in addr)
        t = torch.tensor(addr, dtype=torch.int32, device="cuda")
        assert P.probe_lds_rate(kind, blocks, 20, t.data_ptr(), cyc.data_ptr(), sink.data_ptr()) == 0
        assert P.probe_lds_rate(kind, blocks, iters, t.data_ptr(), cyc.data_ptr(), sink.data_ptr()) == 0
        clk = float(cyc.cpu().numpy().mean()) / (4 * iters * 8)
        res[name] = clk
        print("%-44s %5.2f clk/instr/CU  %6.1f bytes/clk/CU" % (name, clk, nbytes / clk))
        assert 0.5 < clk < 200
    assert res["ds_read_b128 A fragments, swizzled"] < res["ds_read_b128 A fragments, unswizzled"]


def test_dma_rate(P):
    """global_load_lds_dwordx4 throughput into LDS (bytes per shader clock
    per CU) from an L2-resident source of 4 MiB and from an HBM-sized one.
    Recorded; gated only for sanity."""
    blocks, iters = 256, 400
    cyc = torch.zeros(blocks * 4, dtype=torch.int64, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for nbytes in (1 << 22, 1 << 30):
        src = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        assert P.probe_dma_rate(blocks, 20, src.data_ptr(), nbytes, cyc.data_ptr(), sink.data_ptr()) == 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        assert P.probe_dma_rate(blocks, iters, src.data_ptr(), nbytes, cyc.data_ptr(), sink.data_ptr()) == 0
        e1.record()
        torch.cuda.synchronize()
        cycles = float(cyc.cpu().numpy().mean())
        rate = 4 * iters * 8 * 1024 / cycles
        gbs = blocks * 4 * iters * 8 * 1024 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        print("global_load_lds from %4d MiB: %.1f bytes/clk/CU, %.2f clk per 1 KiB copy per CU, %.0f GB/s total"
              % (nbytes >> 20, rate, cycles / (4 * iters * 8), gbs))
        assert 4 < rate < 1024
        del src


@pytest.mark.parametrize("offset", [0, 1, 2, 3, 6, 7, 10, 13, 14, 15])
def test_unaligned_16_byte_global_loads(P, offset):
    """Record whether global_load_dwordx4 and global_load_lds_dwordx4 return
    the 16 bytes at an unaligned address (unaligned mode) or those of the
    aligned-down address (strict mode), at even and odd byte offsets.  The
    GEMM's misaligned-row paths rely on exact bytes (2-byte-aligned rows of
    16-bit values, any byte alignment for 8-bit rows): pinned here."""
    P.probe_unaligned.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    P.probe_unaligned.restype = ctypes.c_int
    nbytes = 4096
    src = torch.arange(nbytes, dtype=torch.int32, device="cuda").to(torch.uint8)
    ov = torch.zeros(256, dtype=torch.int32, device="cuda")
    ol = torch.zeros(256, dtype=torch.int32, device="cuda")
    assert P.probe_unaligned(src.data_ptr(), nbytes, offset, ov.data_ptr(), ol.data_ptr()) == 0
    host = src.cpu().numpy()
    vec = ov.cpu().numpy().view(np.uint8).reshape(64, 16)
    lds = ol.cpu().numpy().view(np.uint8).reshape(64, 16)
    exact = np.stack([host[offset + 32 * l: offset + 32 * l + 16] for l in range(64)])
    down = np.stack([host[(offset + 32 * l) & ~15: ((offset + 32 * l) & ~15) + 16] for l in range(64)])
    kind = lambda got: "exact" if np.array_equal(got, exact) else ("aligned-down" if np.array_equal(got, down) else "other")
    print("offset %2d: global_load_dwordx4 -> %s, global_load_lds_dwordx4 -> %s" % (offset, kind(vec), kind(lds)))
    assert kind(vec) == "exact" and kind(lds) == "exact"


def test_permlane32_swap_lanes(P):
    """v_permlane32_swap_b32 x, y: lanes 32-63 of x trade with lanes 0-31 of y.
    The whole-tile epilogues rely on it to turn two 32-column pieces of rows
    R and R+4 into one 64-column piece of each row."""
    P.probe_permlane32_swap.argtypes = [ctypes.c_void_p]
    P.probe_permlane32_swap.restype = ctypes.c_int
    out = torch.zeros(128, dtype=torch.int32, device="cuda")
    assert P.probe_permlane32_swap(out.data_ptr()) == 0
    got = out.cpu().numpy()
    lane = np.arange(64)
    want_x = np.where(lane < 32, 1000 + lane, 2000 + lane - 32)
    want_y = np.where(lane < 32, 1000 + lane + 32, 2000 + lane)
    assert (got[:64] == want_x).all() and (got[64:] == want_y).all(), got

