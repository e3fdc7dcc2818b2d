"""The epilogue of the clamped (ragged-shape) kernels: tiles wholly inside
M x N store without per-element masks, tiles on the M or N edge mask every
element.  Every output must land where it belongs, and nothing else in C may
be written.

The fp32-output kernel and the half-precision-output kernel of one instance
run the same k order and the same fp32 epilogue arithmetic, then round once
(fp32 stores as is).  So rounding the fp32 result to the half-precision type
must give the half-precision kernel's bits exactly: an element stored to the
wrong place, stored twice or not at all shows as a mismatch.  Each case runs
at packed strides, at an odd ldc with C one element off its alignment, and
with a padded ldc.  The run helper checks that the row padding and the guard
bands of C keep their poison.
"""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from tests.gpu_helpers import DTYPES, assert_bound, decode_out, encode_out, law_for, run  # noqa: E402

# half-precision output code -> the fp32 output code of the same inputs
F32_OF = {1: 0, 3: 2, 5: 4, 6: 4, 8: 7, 9: 7}
CLAMPED16 = ["dl_256x256x64_fd2_clamp", "dl_256x256x64_fd1_clamp", "dl_128x128x64_fd2_clamp",
             "dl_64x64x64_fd2_clamp"]
CLAMPED8 = ["dl8_256x256x128_clamp", "dl8_128x128x128_clamp"]


@pytest.fixture(scope="module")
def G():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from dense_half_precision_tiled_amd import gemm
    gemm.load()
    return gemm


def _instance(G, name):
    for i in range(G.gemm_num_instances()):
        if G.gemm_instance_name(i) == name:
            return i
    raise AssertionError("no instance " + name)


def _shape(col, in8):
    """Ragged M and K, several interior tiles and an edge row and column of
    tiles; with column-major B the last column group is 1 column wide."""
    if col:
        return 600, 517, 200
    return 600, (528 if in8 else 520), 200


@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("name,code", [(n, c) for n in CLAMPED16 for c in (1, 3)] +
                         [(n, c) for n in CLAMPED8 for c in (5, 6, 8, 9)])
def test_interior_and_edge_tiles_match_rounded_fp32(G, name, code, layout):
    fmt, out = DTYPES[code]
    col = layout == "col"
    if col and "_fd1" in name:
        pytest.skip("the fd1 instances take row-major B only")
    in8 = fmt in ("e4m3", "e5m2")
    M, N, K = _shape(col, in8)
    inst = _instance(G, name)
    seed = 1500 + 10 * code + (5 if col else 0)
    A = law_for(fmt)((M, K), seed, fmt)
    B = law_for(fmt)((K, N), seed + 1, fmt)
    Bs = np.ascontiguousarray(B.T) if col else B
    lay = G.GEMM_B_COL_MAJOR if col else None
    print("epilogue", name, code, layout, (M, N, K), flush=True)
    y32 = run(G, A, Bs, F32_OF[code], instance=inst, layout=lay)
    extra = oracle.align_bound8(A, B, fmt) if in8 else None
    assert_bound(y32, oracle.gemm_f64(A, B, fmt), K, "f32", name, extra=extra)
    want = decode_out(encode_out(y32, out), out)
    for ldc_pad, c_off in [(0, 0), (1, 1), (24, 0)]:
        y = run(G, A, Bs, code, instance=inst, layout=lay, ldc=N + ldc_pad, c_off=c_off)
        bad = y != want
        assert not bad.any(), "%s code %d %s ldc=N+%d c_off=%d: %d elements differ, first at %s" % (
            name, code, layout, ldc_pad, c_off, bad.sum(), np.argwhere(bad)[0])


@pytest.mark.parametrize("name,code", [("dl_256x256x64_fd2_clamp", 3), ("dl_128x128x64_fd2_clamp", 1),
                                       ("dl8_256x256x128_clamp", 6)])
def test_general_epilogue_interior_and_edge_tiles(G, name, code):
    """alpha, bias and ReLU (beta = 0, so the old C is not read): the same
    fp32 value rounded once in both output types."""
    fmt, out = DTYPES[code]
    in8 = fmt in ("e4m3", "e5m2")
    M, N, K = _shape(True, in8)
    inst = _instance(G, name)
    A = law_for(fmt)((M, K), 1701 + code, fmt)
    B = law_for(fmt)((K, N), 1702 + code, fmt)
    Bt = np.ascontiguousarray(B.T)
    bias = np.linspace(-2.0, 2.0, N)
    ex = dict(instance=inst, layout=G.GEMM_B_COL_MAJOR, alpha=0.75, bias=bias, relu=1)
    y32 = run(G, A, Bt, F32_OF[code], **ex)
    want = decode_out(encode_out(y32, out), out)
    y = run(G, A, Bt, code, ldc=N + 1, c_off=1, **ex)
    assert np.array_equal(y, want)
    assert (y == 0).any() and (y > 0).any()       # ReLU clipped some, kept some
