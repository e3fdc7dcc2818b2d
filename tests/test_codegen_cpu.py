"""Code-generation checks of the gfx950 kernels (CPU only: hipcc cross-compiles).

Each instantiation unit is compiled to device assembly and every GEMM kernel in
it is checked for properties the design relies on:
* no scratch (spill) access between a kernel's first and last MFMA: the main
  loop runs from registers and LDS only;
* no scratch at all in the whole-tile kernels with the plain epilogue (the
  configurations of the large workloads);
* M0 is written only by the asynchronous-copy helper (its s_mov_b32 m0 is
  followed by s_nop 0 and the global_load_lds it addresses), so no other code
  can move a copy's LDS destination, and every copy uses the scalar-base
  address form;
* every kernel uses at most 512 VGPR+AGPR registers (one wave per SIMD) and the
  MFMA instructions the design names (32x32x16 for 16-bit inputs, the unscaled
  32x32x64 8-bit form for 8-bit inputs).
"""
import concurrent.futures
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from dense_half_precision_tiled_amd import build as B

UNITS = ["gemm_dl_nn.hip", "gemm_dl_nn_epi.hip", "gemm_dl_tn.hip", "gemm_dl_tn_epi.hip",
         "gemm_ks.hip", "gemm_ks_epi.hip", "gemm_dl_f8_tn.hip", "gemm_dl_f8_tn_epi.hip",
         "gemm_dl_f8_nn.hip", "gemm_dl_f8_nn_epi.hip",
         "gemm_pk_nn.hip", "gemm_pk_nn_epi.hip", "gemm_pk_tn.hip", "gemm_pk_tn_epi.hip", "gemm_pp.hip",
         "gemm_sk.hip"]

pytestmark = pytest.mark.skipif(not os.path.exists(B.hipcc()), reason="hipcc not available")


def _compile(unit, outdir):
    out = os.path.join(outdir, unit + ".s")
    cmd = [B.hipcc()] + [f for f in B.HIP_FLAGS if f != "-fPIC"] + \
        ["--cuda-device-only", "-S", os.path.join(B.CSRC, unit), "-o", out]
    subprocess.run(cmd, check=True, stderr=subprocess.DEVNULL)
    return unit, out


@pytest.fixture(scope="module")
def kernels():
    """{mangled kernel name: (unit, list of instruction lines, metadata dict)}."""
    d = tempfile.mkdtemp(prefix="dhpt_asm_")
    try:
        with concurrent.futures.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
            outs = list(ex.map(lambda u: _compile(u, d), UNITS))
        res = {}
        for unit, path in outs:
            text = open(path).read().split("\n")
            cur = None
            for ln in text:
                m = re.match(r"^(_ZN4dhpt\S*gemm_\w\w(?:_persist)?_kernel\S*):", ln)
                if m:
                    cur = m.group(1)
                    res[cur] = (unit, [], {})
                    continue
                if cur is not None and ln.startswith(".Lfunc_end"):
                    cur = None
                elif cur is not None:
                    s = ln.split(";")[0].strip()
                    if s:
                        res[cur][1].append(s)
                m = re.match(r"^\s*\.set\s+(_ZN4dhpt\S*gemm_\w\w(?:_persist)?_kernel\S*)\.(\w+),\s*(\d+)", ln)
                if m and m.group(1) in res:
                    res[m.group(1)][2][m.group(2)] = int(m.group(3))
        return res
    finally:
        shutil.rmtree(d, ignore_errors=True)


def _short(name):
    return re.search(r"kernelI(.*?)EEv", name).group(1)


def test_every_unit_has_kernels(kernels):
    units = {u for u, _, _ in kernels.values()}
    assert units == set(UNITS)
    assert len(kernels) >= 100


def _slice_loop(ins):
    """The K loop of a persistent kernel: the shortest backward branch whose
    body holds MFMAs and exactly one barrier (the per-slice barrier)."""
    labels = {s[:-1]: i for i, s in enumerate(ins) if s.endswith(":")}
    best = None
    for j, s in enumerate(ins):
        m = re.match(r"s_(?:cbranch_\w+|branch) (\.LBB\S+)", s)
        i = labels.get(m.group(1)) if m else None
        if i is not None and i < j:
            body = ins[i:j]
            if any(x.startswith("v_mfma") for x in body) and sum(x.startswith("s_barrier") for x in body) == 1:
                if best is None or j - i < best[1] - best[0]:
                    best = (i, j)
    return best


def test_no_scratch_inside_the_mfma_loop(kernels):
    """One-tile kernels: no scratch access between the first and the last
    MFMA.  Persistent kernels run many tiles, so there the slice loop itself
    must be free of scratch, and what they spill (once per tile, in the tile's
    set-up and epilogue) stays below 96 bytes."""
    for name, (unit, ins, meta) in kernels.items():
        mf = [i for i, s in enumerate(ins) if s.startswith("v_mfma_f32_")]
        assert mf, name
        if "persist" in name:
            a, b = _slice_loop(ins)
            assert sum(ins[i].startswith("v_mfma") for i in range(a, b)) == 64, _short(name)
            lo, hi = a, b
            assert meta.get("private_seg_size", 0) <= 96, "%s spills %d bytes" % (
                _short(name), meta["private_seg_size"])
        else:
            lo, hi = mf[0], mf[-1]
        inside = [ins[i] for i in range(lo, hi) if ins[i].startswith("scratch_")]
        assert not inside, "%s (%s): %d scratch accesses between MFMAs, e.g. %s" % (
            _short(name), unit, len(inside), inside[0])


def test_whole_tile_plain_kernels_use_no_scratch(kernels):
    # template arguments <IN, OUT, BM, BN, FD, EDGE=0, BT, EPI=false> (dl and
    # its persistent form), <IN, OUT, EDGE=0, BT, EPI=false> (ks),
    # <IN, OUT, BT, EPI=false> (pp) and <IN, EDGE=0, BT> (sk: fp32 partial
    # tiles, no epilogue)
    checked = 0
    for name, (unit, ins, meta) in kernels.items():
        args = re.findall(r"Li(\d+)E|Lb(\d)E", _short(name))
        vals = [int(a or b) for a, b in args]
        if "gemm_dl" in name:
            edge, epi = vals[5], vals[7]
        elif "gemm_pp" in name:                 # <IN, OUT, BT, EPI>: whole tiles only
            edge, epi = 0, vals[3]
        elif "gemm_sk" in name:                 # <IN, EDGE, BT>
            edge, epi = vals[1], 0
        else:
            edge, epi = vals[2], vals[4]
        if edge == 0 and epi == 0:
            assert meta.get("private_seg_size", 0) == 0, "%s uses %d bytes of scratch" % (
                _short(name), meta["private_seg_size"])
            checked += 1
    assert checked >= 36


def test_m0_is_written_only_by_the_copy_helper(kernels):
    for name, (unit, ins, meta) in kernels.items():
        for i, s in enumerate(ins):
            if re.search(r"\bm0\b", s.split(",")[0] if "," in s else s) and not s.startswith("global_load_lds"):
                # a write of m0: only the helper's s_mov_b32 m0, sN; s_nop 0; global_load_lds
                assert s.startswith("s_mov_b32 m0,"), "%s: %s" % (_short(name), s)
                assert ins[i + 1] == "s_nop 0", "%s: %s then %s" % (_short(name), s, ins[i + 1])
                assert ins[i + 2].startswith("global_load_lds_dwordx4"), "%s: %s" % (_short(name), ins[i + 2])


def test_copies_use_a_scalar_base(kernels):
    """Every global -> LDS copy takes a uniform base in a scalar register pair
    and one 32-bit offset VGPR (global_load_lds_dwordx4 vN, s[a:b]): the
    form that halves the address registers a copy reads and lets a slice
    advance two scalar bases instead of every lane's 64-bit pointers."""
    checked = 0
    for name, (unit, ins, meta) in kernels.items():
        for s in ins:
            if s.startswith("global_load_lds"):
                assert re.match(r"global_load_lds_dwordx4 v\d+, s\[\d+:\d+\]", s), "%s: %s" % (_short(name), s)
                checked += 1
    assert checked > 1000


def test_register_budget_and_mfma_shape(kernels):
    for name, (unit, ins, meta) in kernels.items():
        # one wave per SIMD (512 registers), or two for the 8-wave ping-pong kernel
        budget = 256 if "gemm_pp" in name else 512
        assert meta["num_vgpr"] + meta["num_agpr"] <= budget, _short(name)
        ops = {s.split()[0] for s in ins if s.startswith("v_mfma")}
        in8 = unit.startswith("gemm_dl_f8") or ("gemm_sk" in name and
                                                int(re.findall(r"Li(\d+)E", _short(name))[0]) >= 2)
        if in8:
            assert ops == {"v_mfma_f32_32x32x64_f8f6f4"}, (_short(name), ops)
        else:
            assert ops <= {"v_mfma_f32_32x32x16_f16", "v_mfma_f32_32x32x16_bf16"}, (_short(name), ops)


def test_no_scalar_memory_writes(kernels):
    """No kernel writes memory through the scalar data cache (scalar stores,
    scalar atomics, its write-back): counters and outputs go through vector
    memory instructions only."""
    for name, (unit, ins, meta) in kernels.items():
        bad = [s for s in ins if re.match(r"s_(store|buffer_store|atomic|buffer_atomic|dcache_wb)", s)]
        assert not bad, "%s: %s" % (_short(name), bad[0])


def test_persistent_kernels_pull_tiles_with_vector_atomics(kernels):
    pk = [n for n in kernels if "persist" in n]
    assert len(pk) == 32
    for name in pk:
        ins = kernels[name][1]
        assert any(s.startswith("global_atomic_add") for s in ins), _short(name)
        assert any(s.startswith("s_getreg_b32") and "HW_REG_XCC_ID" in s for s in ins), _short(name)
