"""C-ABI checks that need no GPU: the library loads, exports every function
include/gemm.h declares, rejects bad arguments before touching the device,
and its instance choice and tile visit order are what they claim."""
import ctypes
import os
import re

import numpy as np
import pytest

from dense_half_precision_tiled_amd import gemm as G

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm.h")

# Fake, never dereferenced device addresses for validation-only calls.
PA, PB, PC = 0x10000000, 0x20000000, 0x30000000


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(G.LIB_PATH):
        from dense_half_precision_tiled_amd import build
        build.build()
    return G.load()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(G.EXPORTED)
    raw = ctypes.CDLL(G.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_strerror_covers_every_status(lib):
    for st in range(0, -11, -1):
        s = G.gemm_strerror(st)
        assert s and s != "unknown status"
    assert G.gemm_strerror(12345) == "unknown status"


@pytest.mark.parametrize("args,want", [
    ((-1, 4, 4, 0, PA, 4, PB, 4, PC, 4), G.GEMM_ERR_DIM),
    ((4, -1, 4, 0, PA, 4, PB, 4, PC, 4), G.GEMM_ERR_DIM),
    ((4, 4, -1, 0, PA, 4, PB, 4, PC, 4), G.GEMM_ERR_DIM),
    ((4, 4, 4, 10, PA, 4, PB, 4, PC, 4), G.GEMM_ERR_DTYPE),
    ((4, 4, 4, -1, PA, 4, PB, 4, PC, 4), G.GEMM_ERR_DTYPE),
    ((4, 4, 8, 0, PA, 7, PB, 4, PC, 4), G.GEMM_ERR_LD),
    ((4, 4, 8, 0, PA, 8, PB, 3, PC, 4), G.GEMM_ERR_LD),
    ((4, 4, 8, 0, PA, 8, PB, 4, PC, 3), G.GEMM_ERR_LD),
    ((4, 4, 8, 0, PA, -8, PB, 4, PC, 4), G.GEMM_ERR_LD),
    ((4, 4, 8, 0, PA, 8, PB, 4, 0, 4), G.GEMM_ERR_NULL),
    ((4, 4, 8, 0, 0, 8, PB, 4, PC, 4), G.GEMM_ERR_NULL),
    ((4, 4, 8, 0, PA, 8, 0, 4, PC, 4), G.GEMM_ERR_NULL),
    ((4, 4, 8, 0, PA + 1, 8, PB, 4, PC, 4), G.GEMM_ERR_ALIGN),
    ((4, 4, 8, 0, PA, 8, PB, 4, PC + 2, 4), G.GEMM_ERR_ALIGN),     # fp32 C needs 4 B
    ((1 << 31, 4, 8, 0, PA, 8, PB, 4, PC, 4), G.GEMM_ERR_RANGE),
    ((4, 4, 8, 0, PA, (1 << 40) + 8, PB, 4, PC, 4), G.GEMM_ERR_RANGE),
    ((1 << 20, 4, 8, 0, PA, 1 << 30, PB, 4, PC, 4), G.GEMM_ERR_RANGE),
    # C overlapping A, then B
    ((4, 4, 8, 0, PA, 8, PB, 4, PA + 16, 4), G.GEMM_ERR_ALIAS),
    ((4, 4, 8, 3, PA, 8, PB, 4, PB + 8, 4), G.GEMM_ERR_ALIAS),
])
def test_invalid_arguments_rejected_before_launch(lib, args, want):
    assert G.gemm_run(*args, None) == want
    assert G.gemm_select_instance(*args) == want
    for inst in range(G.gemm_num_instances()):
        assert G.gemm_run_instance(inst, *args, None) == want


def test_empty_output_is_a_noop_without_launch(lib):
    # M == 0 or N == 0: success, nothing enqueued, pointers may be null
    assert G.gemm_run(0, 5, 7, 0, 0, 7, 0, 5, 0, 5, None) == G.GEMM_OK
    assert G.gemm_run(5, 0, 7, 0, 0, 7, 0, 0, 0, 0, None) == G.GEMM_OK
    assert G.gemm_select_instance(5, 0, 7, 0, 0, 7, 0, 0, 0, 0) == G.GEMM_OK


def test_adjacent_buffers_are_not_aliases(lib):
    # C starts exactly where A ends: allowed (only overlap is rejected)
    M, N, K = 4, 4, 8
    a_end = PA + ((M - 1) * K + K) * 2
    assert G.gemm_select_instance(M, N, K, 0, PA, K, PB, N, a_end, N) >= 0


def test_unknown_instance(lib):
    n = G.gemm_num_instances()
    assert n >= 2
    assert G.gemm_run_instance(n, 4, 4, 4, 0, PA, 4, PB, 4, PC, 4, None) == G.GEMM_ERR_INSTANCE
    assert G.gemm_instance_name(n) == "?"
    for i in range(n):
        assert G.gemm_instance_name(i).startswith(("dl_", "ks_", "dl8_", "pk_", "pp_"))


def _pick(M, N, K, dtype=3, lda=None, ldb=None, ldc=None, pa=PA, pb=PB):
    return G.gemm_instance_name(G.gemm_select_instance(
        M, N, K, dtype, pa, lda or K, pb, ldb or N, 0x7000000000, ldc or N))


def test_whole_tile_kernels_need_64_byte_aligned_c_rows(lib):
    """The whole-tile kernels store C non-temporally in 64-column row pieces;
    the host gives them only C whose rows start on 64-byte boundaries and
    sends other whole-tile problems to the clamped kernel."""
    def pick(c, ldc, dtype=3):
        return G.gemm_instance_name(G.gemm_select_instance(8192, 8192, 8192, dtype, PA, 8192, PB, 8192, c, ldc))
    base = 0x7000000000
    assert pick(base, 8192) == "dl_256x256x64_fd2"
    assert pick(base, 8192 + 32) == "dl_256x256x64_fd2"          # 16448 bytes per bf16 row
    assert pick(base, 8192 + 8) == "dl_256x256x64_fd2_clamp"     # 16400 bytes: rows off 64-byte boundaries
    assert pick(base + 2, 8192) == "dl_256x256x64_fd2_clamp"     # C itself one element off
    assert pick(base + 32, 8192, dtype=2) == "dl_256x256x64_fd2_clamp"   # fp32 C, 32 bytes off
    assert pick(base, 8192 + 16, dtype=2) == "dl_256x256x64_fd2"  # fp32 rows of 32832 bytes


def test_instance_choice(lib):
    assert _pick(8192, 8192, 8192) == "dl_256x256x64_fd2"
    assert _pick(4096, 4096, 4096) == "dl_256x256x64_fd2"
    # under 128 tiles of 256x256: K split across the waves of a 128x128 tile
    # when K >= 2048 (and >= 64 such tiles); 64x64 tiles for small problems
    # (under 128 tiles of 128x128, K <= 2048); else 128x128 tiles
    assert _pick(2048, 2048, 2048, 0) == "ks_128x128x64"
    assert _pick(256, 256, 256, 0) == "dl_64x64x64_fd2"
    assert _pick(1024, 1024, 1024, 0) == "dl_64x64x64_fd2"
    assert _pick(512, 512, 4096, 0) == "dl_128x128x64_fd2"
    assert _pick(2048, 2048, 1984, 0) == "dl_128x128x64_fd2"
    assert _pick(1000, 1000, 2100, 3) == "ks_128x128x64_clamp"
    assert _pick(1000, 1000, 1000, 3) == "dl_64x64x64_fd2_clamp"
    assert _pick(1000, 1001, 4096, 3) == "dl_128x128x64_masked"
    # ragged shape, 2-byte-aligned lda, N a multiple of 8: clamped-edge kernel
    assert _pick(3000, 5000, 4099, 1) == "dl_256x256x64_fd2_clamp"
    # misaligned base pointer: unaligned 16-byte loads are fine, same kernel
    assert _pick(4096, 4096, 4096, pa=PA + 2) == "dl_256x256x64_fd2"
    # K not a multiple of 64: clamped-edge kernel with the zero-filled tail slice
    assert _pick(4096, 4096, 4000) == "dl_256x256x64_fd2_clamp"
    # N not a multiple of 8 with row-major B: the masked fallback
    assert _pick(4096, 4100, 4096) == "dl_256x256x64_masked"
    assert _pick(100, 7, 33, 0) == "dl_128x128x64_masked"


def test_copy_offsets_beyond_31_bits_take_the_masked_kernels(lib):
    """The whole-tile and clamped kernels address their copies as byte
    offsets below 2^31 from a per-tile base: the farthest is tile - 1 rows of
    A (or of column-major B) plus one 128-byte slice, or the 128 bytes' worth
    of k rows of row-major B plus a tile width.  One element more of leading
    dimension and the choice falls to the masked kernel of the same tiles."""
    far = dict(pa=1 << 40, pb=2 << 40)        # operands far apart: no aliasing at these extents
    lim = 2 ** 31 - 1
    L = (lim - 128) // (255 * 2)               # A rows, 256x256 tiles, 2-byte elements
    assert _pick(4096, 4096, 4096, lda=L, **far) == "dl_256x256x64_fd2"
    assert _pick(4096, 4096, 4096, lda=L + 1, **far) == "dl_256x256x64_masked"
    L = (lim - 256 * 2) // 128                 # row-major B: 64 rows of 2-byte elements per slice
    assert _pick(4096, 4096, 4096, ldb=L, **far) == "dl_256x256x64_fd2"
    assert _pick(4096, 4096, 4096, ldb=L + 1, **far) == "dl_256x256x64_masked"
    L = (lim - 128) // (127 * 2)               # the k-split kernel's 128x128 tiles
    assert _pick(2048, 2048, 2048, 0, lda=L, **far) == "ks_128x128x64"
    assert _pick(2048, 2048, 2048, 0, lda=L + 1, **far) == "dl_128x128x64_masked"
    L = (lim - 128) // 255                     # column-major 8-bit B: 255 rows of 1-byte elements
    col = G.GEMM_B_COL_MAJOR
    pick8 = lambda ldb: G.gemm_instance_name(G.gemm_select_instance_ex(
        8192, 8192, 8192, 6, col, far["pa"], 8192, far["pb"], ldb, 0x7000000000, 8192, 1.0, 0.0, None, 0))
    assert pick8(L) == "dl8_256x256x128"
    assert pick8(L + 1) == "dl8_256x256x128_masked"


def _pick_ex(M, N, K, layout, dtype=3, alpha=1.0, beta=0.0, bias=None, relu=0):
    ldb = K if layout == G.GEMM_B_COL_MAJOR else N
    return G.gemm_instance_name(G.gemm_select_instance_ex(
        M, N, K, dtype, layout, PA, K, PB, ldb, 0x7000000000, N, alpha, beta, bias, relu))


def test_instance_choice_general_form(lib):
    col, row = G.GEMM_B_COL_MAJOR, G.GEMM_B_ROW_MAJOR
    assert _pick_ex(8192, 8192, 8192, col) == "dl_256x256x64_fd2"
    # column-major B reads B in rows of K like A: any N stays on the clamped kernel
    assert _pick_ex(4096, 4100, 4096, col) == "dl_256x256x64_fd2_clamp"
    assert _pick_ex(100, 7, 33, col, 0) == "dl_64x64x64_fd2_clamp"
    assert _pick_ex(4096, 4100, 4096, row, relu=1) == "dl_256x256x64_masked"
    assert _pick_ex(4096, 4096, 4096, row, alpha=2.0, beta=1.0, bias=PC, relu=1) == "dl_256x256x64_fd2"
    # the plain form through gemm_run_ex selects what gemm_run selects
    assert _pick_ex(3000, 5000, 4099, row, 1) == _pick(3000, 5000, 4099, 1)


def test_instance_choice_8bit_inputs(lib):
    """8-bit float inputs run on the dl8 instances only; tile size by the
    number of tiles, clamped edges for anything but whole tiles with K a
    multiple of 128 (row-major B: N % 16 == 0), else the masked fallback."""
    col = G.GEMM_B_COL_MAJOR
    for dt in range(4, 10):
        assert _pick_ex(8192, 8192, 8192, col, dt) == "dl8_256x256x128"
    assert _pick_ex(4096, 4096, 4096, col, 6) == "dl8_256x256x128"
    assert _pick_ex(4096, 4096, 4160, col, 6) == "dl8_256x256x128_clamp"      # K % 128 == 64
    assert _pick_ex(2048, 2048, 2048, col, 4) == "dl8_128x128x128"
    assert _pick_ex(3000, 5000, 4099, col, 5) == "dl8_256x256x128_clamp"
    assert _pick_ex(256, 256, 256, col, 4) == "dl8_64x64x128"
    assert _pick_ex(100, 7, 33, col, 7) == "dl8_64x64x128_clamp"
    # odd byte addresses and leading dimensions are fine for 1-byte elements
    ex = G.gemm_select_instance_ex
    assert ex(4096, 4096, 4096, 6, col, PA + 1, 4097, PB + 3, 4099, PC, 4096, 1.0, 0.0, None, 0) >= 0
    # 16-bit dtypes never land on the 8-bit instances and vice versa
    ids = {G.gemm_instance_name(i): i for i in range(G.gemm_num_instances())}
    st = G.gemm_run_instance_ex(ids["dl8_256x256x128"], 256, 256, 128, 3, col, PA, 128, PB, 128, PC, 256,
                                1.0, 0.0, None, 0, None)
    assert st == G.GEMM_ERR_INSTANCE
    st = G.gemm_run_instance_ex(ids["dl_256x256x64_fd2"], 256, 256, 128, 4, col, PA, 128, PB, 128, PC, 256,
                                1.0, 0.0, None, 0, None)
    assert st == G.GEMM_ERR_INSTANCE
    # an 8-bit whole-tile instance needs K % 128 == 0
    st = G.gemm_run_instance_ex(ids["dl8_256x256x128"], 256, 256, 64, 4, col, PA, 64, PB, 64, PC, 256,
                                1.0, 0.0, None, 0, None)
    assert st == G.GEMM_ERR_INSTANCE
    # row-major B: the same tiles; N % 16 != 0 falls to the masked kernels
    assert _pick(8192, 8192, 8192, 6) == "dl8_256x256x128"
    assert _pick(3000, 5008, 4099, 5) == "dl8_256x256x128_clamp"
    assert _pick(3000, 5000, 4099, 5) == "dl8_256x256x128_masked"        # 5000 % 16 == 8
    assert _pick(4096, 4104, 4096, 4) == "dl8_256x256x128_masked"
    assert _pick(1000, 1001, 777, 9) == "dl8_128x128x128_masked"
    assert _pick(100, 7, 33, 7) == "dl8_128x128x128_masked"
    assert _pick(256, 256, 256, 4) == "dl8_64x64x128"
    assert _pick(2048, 2048, 2048, 4, pa=PA + 1) == "dl8_128x128x128"
    # extents count 1-byte elements: C starting right after an 8-bit A is no alias
    a_end = PA + 4 * 128
    assert ex(4, 4, 128, 4, col, PA, 128, PB, 128, a_end, 4, 1.0, 0.0, None, 0) >= 0
    assert ex(4, 4, 128, 4, col, PA, 128, PB, 128, a_end - 4, 4, 1.0, 0.0, None, 0) == G.GEMM_ERR_ALIAS


def test_general_form_validation(lib):
    col = G.GEMM_B_COL_MAJOR
    ex = G.gemm_select_instance_ex
    # unknown layout
    assert ex(4, 4, 8, 0, 2, PA, 8, PB, 8, PC, 4, 1.0, 0.0, None, 0) == G.GEMM_ERR_LAYOUT
    assert G.gemm_run_ex(4, 4, 8, 0, -1, PA, 8, PB, 8, PC, 4, 1.0, 0.0, None, 0, None) == G.GEMM_ERR_LAYOUT
    # column-major B needs ldb >= K, row-major B needs ldb >= N
    assert ex(4, 4, 8, 0, col, PA, 8, PB, 7, PC, 4, 1.0, 0.0, None, 0) == G.GEMM_ERR_LD
    assert ex(4, 16, 8, 0, col, PA, 8, PB, 8, PC, 16, 1.0, 0.0, None, 0) >= 0
    assert ex(4, 16, 8, 0, 0, PA, 8, PB, 8, PC, 16, 1.0, 0.0, None, 0) == G.GEMM_ERR_LD
    # bias: 4-byte aligned, not overlapping C
    assert ex(4, 4, 8, 0, col, PA, 8, PB, 8, PC, 4, 1.0, 0.0, PC + 4096 + 2, 0) == G.GEMM_ERR_ALIGN
    assert ex(4, 4, 8, 0, col, PA, 8, PB, 8, PC, 4, 1.0, 0.0, PC + 8, 0) == G.GEMM_ERR_ALIAS
    assert ex(4, 4, 8, 0, col, PA, 8, PB, 8, PC, 4, 1.0, 0.0, PC + 4 * 16, 0) >= 0
    # C overlapping a column-major B (N x K extent), adjacent is fine
    b_end = PB + ((4 - 1) * 8 + 8) * 2
    assert ex(4, 4, 8, 3, col, PA, 8, PB, 8, b_end - 2, 4, 1.0, 0.0, None, 0) == G.GEMM_ERR_ALIAS
    assert ex(4, 4, 8, 3, col, PA, 8, PB, 8, b_end, 4, 1.0, 0.0, None, 0) >= 0
    # K == 0: the plain form is a zero fill (no instance); the general form
    # still evaluates act(beta*C + bias) on an instance
    assert ex(4, 4, 0, 0, 0, 0, 0, 0, 4, PC, 4, 1.0, 0.0, None, 0) == G.GEMM_OK
    assert ex(4, 4, 0, 0, 0, 0, 0, 0, 4, PC, 4, 1.0, 1.0, None, 0) >= 0
    # instances that cannot run a problem refuse it before any launch: the
    # prefetch-distance-1 kernels exist for the plain row-major form only, and
    # whole-tile kernels need whole tiles (fake pointers are never touched)
    for inst in range(G.gemm_num_instances()):
        name = G.gemm_instance_name(inst)
        if "_fd1" in name:
            st = G.gemm_run_instance_ex(inst, 256, 256, 64, 0, col, PA, 64, PB, 64, PC, 256,
                                        1.0, 0.0, None, 0, None)
            assert st == G.GEMM_ERR_INSTANCE, name
            st = G.gemm_run_instance_ex(inst, 256, 256, 64, 0, 0, PA, 64, PB, 256, PC, 256,
                                        2.0, 0.0, None, 0, None)
            assert st == G.GEMM_ERR_INSTANCE, name
        if name.endswith(("x64_fd2", "x64_fd1", "x64")):
            st = G.gemm_run_instance_ex(inst, 4, 4, 8, 0, col, PA, 8, PB, 8, PC, 4, 1.0, 0.0, None, 0, None)
            assert st == G.GEMM_ERR_INSTANCE, name


@pytest.mark.parametrize("shape", [(8192, 8192), (4096, 4096), (2048, 2048), (3000, 5000),
                                   (256, 256), (2, 2), (257, 263), (100000, 128), (128, 70000)])
def test_tile_order_is_a_bijection(lib, shape):
    M, N = shape
    for inst in range(G.gemm_num_instances()):
        tm, tn = G.gemm_tile_order(inst, M, N)
        name = G.gemm_instance_name(inst)
        bm = int(name.split("_")[1].split("x")[0])
        bn = int(name.split("_")[1].split("x")[1])
        assert bm == bn
        tilesM, tilesN = -(-M // bm), -(-N // bn)
        assert tm.size == tilesM * tilesN
        assert tm.min() >= 0 and tm.max() < tilesM and tn.min() >= 0 and tn.max() < tilesN
        flat = tm.astype(np.int64) * tilesN + tn
        assert np.unique(flat).size == flat.size


def _panels(tm, tn):
    """Distinct A row-panels plus B column-panels that a set of tiles needs."""
    return np.unique(tm).size + np.unique(tn).size


def test_panel_count_page_example():
    """The page's count for eight tiles in flight ("The Asynchronous Kernel:
    Tensor Cores & TMA", section "Scheduling is geometry"): eight tiles along
    one row of the tile grid need one A panel and eight B panels, nine in
    all; the same eight as a 4x2 block need four and two, six."""
    row = np.arange(8)
    assert _panels(np.zeros(8, int), row) == 9
    blk_m, blk_n = np.divmod(np.arange(8), 2)
    assert _panels(blk_m, blk_n) == 6


@pytest.mark.parametrize("n", [4096, 8192])
def test_tile_order_keeps_each_xcd_compact(lib, n):
    """The first 32 workgroups dealt to one XCD (w = x, x+8, x+16, ... under
    round-robin dispatch) share that XCD's L2.  With the remap they cover a
    4x8 or 8x4 block of tiles: at most 12 distinct A row-panels plus B
    column-panels, never more than plain row-major order needs."""
    tm, tn = G.gemm_tile_order(0, n, n)
    tiles_n = n // 256
    for x in range(8):
        sel = np.arange(x, 256, 8)
        panels = _panels(tm[sel], tn[sel])
        row_major = np.unique(sel // tiles_n).size + np.unique(sel % tiles_n).size
        assert panels <= 12 and panels <= row_major, (x, panels, row_major)


# ------------------------------------------------------------ workspace entry points
WS = 0x5000000000          # a fake, 256-byte-aligned device address (never touched)


def ws_call(*args, ws=WS, nbytes=None):
    nb = G.gemm_workspace_size() if nbytes is None else nbytes
    return G.gemm_run_ws(*args, ws, nb, None)


def test_workspace_size_is_a_small_constant(lib):
    assert G.gemm_workspace_size() == 4096


@pytest.mark.parametrize("ws,nbytes", [(0, 4096), (WS, 4095), (WS, 0), (WS + 4, 4096), (WS + 128, 8192)])
def test_bad_workspace_rejected_before_launch(lib, ws, nbytes):
    args = (512, 512, 512, 3, 0, PA, 512, PB, 512, PC, 512, 1.0, 0.0, None, 0)
    assert ws_call(*args, ws=ws, nbytes=nbytes) == G.GEMM_ERR_WORKSPACE
    assert G.gemm_run_instance_ws(22, *args, ws, nbytes, None) == G.GEMM_ERR_WORKSPACE
    assert G.gemm_select_instance_ws(*args, ws, nbytes) == G.GEMM_ERR_WORKSPACE


def test_workspace_must_not_overlap_the_operands(lib):
    M, N, K = 64, 64, 64
    base = (M, N, K, 2, 0)
    # inside C, inside A, inside B, inside the bias
    assert ws_call(*base, PA, K, PB, N, PC, N, 1.0, 0.0, None, 0, ws=PC + 256) == G.GEMM_ERR_ALIAS
    assert ws_call(*base, PA, K, PB, N, PC, N, 1.0, 0.0, None, 0, ws=PA) == G.GEMM_ERR_ALIAS
    assert ws_call(*base, PA, K, PB, N, PC, N, 1.0, 0.0, None, 0, ws=PB + 1024) == G.GEMM_ERR_ALIAS
    bias = WS + 1024
    assert ws_call(*base, PA, K, PB, N, PC, N, 1.0, 0.0, bias, 0, ws=WS) == G.GEMM_ERR_ALIAS
    # the other argument checks still come first
    assert ws_call(-1, N, K, 2, 0, PA, K, PB, N, PC, N, 1.0, 0.0, None, 0) == G.GEMM_ERR_DIM
    assert ws_call(M, N, K, 2, 5, PA, K, PB, N, PC, N, 1.0, 0.0, None, 0) == G.GEMM_ERR_LAYOUT


def test_persistent_instances_need_a_workspace(lib):
    ids = {G.gemm_instance_name(i): i for i in range(G.gemm_num_instances())}
    for name in ("pk_256x256x64", "pk_256x256x64_clamp"):
        st = G.gemm_run_instance(ids[name], 512, 512, 512, 3, PA, 512, PB, 512, PC, 512, None)
        assert st == G.GEMM_ERR_INSTANCE
        st = G.gemm_run_instance_ex(ids[name], 512, 512, 512, 3, 1, PA, 512, PB, 512, PC, 512,
                                    1.0, 0.0, None, 0, None)
        assert st == G.GEMM_ERR_INSTANCE


def test_splitk_workspace_size(lib):
    """One fp32 256 x 256 partial tile per output tile and per piece of K;
    pieces of ceil(K / splits) rounded up to 64, so fewer pieces than asked
    for when K is short."""
    tile = 256 * 256 * 4
    assert G.gemm_splitk_workspace_size(2048, 2048, 2048, 4) == 64 * 4 * tile
    assert G.gemm_splitk_workspace_size(1000, 1000, 100, 4) == 16 * 2 * tile      # Kc = 64: two pieces
    assert G.gemm_splitk_workspace_size(1024, 1024, 16384, 16) == 16 * 16 * tile
    assert G.gemm_splitk_workspace_size(300, 5000, 4099, 3) == 2 * 20 * 3 * tile  # Kc = 1408
    assert G.gemm_splitk_workspace_size(256, 256, 0, 4) == 0
    # splits = 0: the library's choice
    assert G.gemm_splitk_workspace_size(1024, 1024, 16384, 0) == 16 * 12 * tile      # 12 pieces of 1408
    assert G.gemm_splitk_workspace_size(512, 512, 32768, 0) == 4 * 32 * tile         # 32 pieces of 1024
    assert G.gemm_splitk_workspace_size(256, 256, 65536, 0) == 1 * 64 * tile         # capped at 64
    assert G.gemm_splitk_workspace_size(2048, 2048, 8192, 0) == 0                    # 256 tiles of 128^2: unsplit
    assert G.gemm_splitk_workspace_size(512, 512, 2048, 0) == 0                      # K too short
    assert G.gemm_splitk_workspace_size(256, 256, 256, -1) == G.GEMM_ERR_RANGE
    assert G.gemm_splitk_workspace_size(-1, 256, 256, 4) == G.GEMM_ERR_DIM
    assert G.gemm_splitk_workspace_size(256, 256, 256, 65) == G.GEMM_ERR_RANGE


def test_splitk_arguments_rejected_before_launch(lib):
    M = N = K = 512
    need = G.gemm_splitk_workspace_size(M, N, K, 4)
    args = (M, N, K, 3, 0, PA, K, PB, N, PC, N, 1.0, 0.0, None, 0)
    assert G.gemm_run_splitk(*args, 4, 0, need, None) == G.GEMM_ERR_WORKSPACE             # no workspace
    assert G.gemm_run_splitk(*args, 4, WS, need - 1, None) == G.GEMM_ERR_WORKSPACE        # too small
    assert G.gemm_run_splitk(*args, 4, WS + 4, need, None) == G.GEMM_ERR_WORKSPACE        # misaligned
    assert G.gemm_run_splitk(*args, -1, WS, need, None) == G.GEMM_ERR_RANGE
    assert G.gemm_run_splitk(*args, 65, WS, need, None) == G.GEMM_ERR_RANGE
    assert G.gemm_run_splitk(*args, 4, PC, need, None) == G.GEMM_ERR_ALIAS                # inside C
    assert G.gemm_run_splitk(M, N, K, 10, 0, PA, K, PB, N, PC, N, 1.0, 0.0, None, 0, 4, WS, need,
                             None) == G.GEMM_ERR_DTYPE                                      # no such dtype
    assert G.gemm_run_splitk(-1, N, K, 3, 0, PA, K, PB, N, PC, N, 1.0, 0.0, None, 0, 4, WS, need,
                             None) == G.GEMM_ERR_DIM
    assert G.gemm_run_splitk(0, N, K, 3, 0, PA, K, PB, N, PC, N, 1.0, 0.0, None, 0, 4, 0, 0, None) == G.GEMM_OK
