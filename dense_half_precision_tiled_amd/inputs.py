"""Seeded synthetic inputs for C = A.B (shared by the GPU tests, the bench and
the oracle's tests; it holds no GEMM arithmetic).

Every generator returns row-major bit patterns: ``uint16`` for fp16 and bf16
values, ``uint8`` for the 8-bit float formats E4M3 and E5M2 (OCP OFP8).
Samples come from ``numpy.random.Generator(PCG64(seed))``.  They are rounded
to the input format by a library conversion: numpy's correctly rounded
float64 -> float16 cast for fp16, torch's float32 -> bfloat16 /
float8_e4m3fn / float8_e5m2 casts (round to nearest, ties to even) for the
others.

Workload recipes (the shapes and value laws of the GEMM configurations):

* ``uniform``  i.i.d. U[-1, 1)  (fp16 workloads; a sample may round to +1.0)
* ``normal``   i.i.d. N(0, 1)   (bf16 workloads)
* ``ints``     i.i.d. integers in {lo..hi} (bit-exact fixture: every partial sum
  of an fp32 accumulation is an integer far below 2^24, hence exact)
* ``quarter``  i.i.d. multiples of 0.25 in [-2, 2] (exact in fp16 and bf16;
  every product is a multiple of 1/16, so fp32 partial sums stay exact while
  their magnitude is below 2^19)
"""
from __future__ import annotations

import numpy as np

F16, BF16, E4M3, E5M2 = "f16", "bf16", "e4m3", "e5m2"
EIGHT_BIT = (E4M3, E5M2)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(int(seed)))


def _to_bits(x: np.ndarray, fmt: str) -> np.ndarray:
    if fmt == F16:
        return np.ascontiguousarray(x.astype(np.float16)).view(np.uint16)
    if fmt == BF16:
        import torch
        t = torch.from_numpy(np.ascontiguousarray(x.astype(np.float32)))
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    if fmt in EIGHT_BIT:
        import torch
        dt = torch.float8_e4m3fn if fmt == E4M3 else torch.float8_e5m2
        t = torch.from_numpy(np.ascontiguousarray(x.astype(np.float32))).to(dt)
        if not bool(torch.isfinite(t.to(torch.float32)).all()):
            raise ValueError("value outside the range of %s" % fmt)
        return t.view(torch.uint8).numpy().copy()
    raise ValueError("unknown format %r" % (fmt,))


def uniform(shape, seed: int, fmt: str = F16, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    return _to_bits(_rng(seed).uniform(lo, hi, size=shape), fmt)


def normal(shape, seed: int, fmt: str = BF16) -> np.ndarray:
    if fmt == BF16 or fmt in EIGHT_BIT:
        x = _rng(seed).standard_normal(size=shape, dtype=np.float32)
    else:
        x = _rng(seed).standard_normal(size=shape)
    return _to_bits(x, fmt)


def signed_magnitude(shape, seed: int, fmt: str, lo: float = 0.5, hi: float = 2.0) -> np.ndarray:
    """Random signs times magnitudes uniform in [lo, hi), rounded to the format
    (round to nearest even; hi itself can be reached)."""
    g = _rng(seed)
    mag = g.uniform(lo, hi, size=shape)
    sign = np.where(g.random(size=shape) < 0.5, -1.0, 1.0)
    return _to_bits(sign * mag, fmt)


def ints(shape, seed: int, fmt: str = F16, lo: int = -2, hi: int = 2) -> np.ndarray:
    return _to_bits(_rng(seed).integers(lo, hi + 1, size=shape).astype(np.float64), fmt)


def quarter(shape, seed: int, fmt: str = F16) -> np.ndarray:
    return _to_bits(_rng(seed).integers(-8, 9, size=shape).astype(np.float64) * 0.25, fmt)


def from_values(values, fmt: str) -> np.ndarray:
    """Exactly representable values (fixtures) -> bit patterns."""
    x = np.asarray(values, dtype=np.float64)
    bits = _to_bits(x, fmt)
    return bits


def padded(bits: np.ndarray, ld: int, fill: int | None = None) -> np.ndarray:
    """Copy a rows x cols matrix into a rows x ld buffer (ld >= cols); the
    padding columns hold ``fill`` (by default a NaN pattern of the format:
    0x7E00 for 16-bit, 0x7F for 8-bit patterns, so any read of them shows up
    in the result).  Returns the full rows x ld array."""
    rows, cols = bits.shape
    if ld < cols:
        raise ValueError("ld < cols")
    if fill is None:
        fill = 0x7F if bits.dtype == np.uint8 else 0x7E00
    out = np.full((rows, ld), fill, dtype=bits.dtype)
    out[:, :cols] = bits
    return out


# Seeds per workload: A = 100*c + 1, B = 100*c + 2, integer fixture +10.
WORKLOADS = {
    "f16_256": dict(M=256, N=256, K=256, fmt=F16, out="f32", law="uniform", c=1),
    "f16_256_int": dict(M=256, N=256, K=256, fmt=F16, out="f32", law="ints", c=1),
    "f16_2048": dict(M=2048, N=2048, K=2048, fmt=F16, out="f32", law="uniform", c=2),
    "bf16_4096": dict(M=4096, N=4096, K=4096, fmt=BF16, out="bf16", law="normal", c=3),
    "bf16_8192": dict(M=8192, N=8192, K=8192, fmt=BF16, out="bf16", law="normal", c=4),
    "f16_ragged": dict(M=3000, N=5000, K=4099, fmt=F16, out="f16", law="uniform", c=5),
    # 8-bit float inputs, B stored column-major by default (the usual 8-bit layout)
    "e4m3_8192": dict(M=8192, N=8192, K=8192, fmt=E4M3, out="bf16", law="normal", c=6, layout="col"),
    "e4m3_4096": dict(M=4096, N=4096, K=4096, fmt=E4M3, out="bf16", law="normal", c=7, layout="col"),
    "e5m2_8192": dict(M=8192, N=8192, K=8192, fmt=E5M2, out="bf16", law="normal", c=8, layout="col"),
    "e4m3_2048": dict(M=2048, N=2048, K=2048, fmt=E4M3, out="f32", law="normal", c=9, layout="col"),
    # long K with few output tiles (the case for splitting K across workgroups)
    "bf16_longk_1024": dict(M=1024, N=1024, K=16384, fmt=BF16, out="bf16", law="normal", c=10),
    "bf16_longk_512": dict(M=512, N=512, K=32768, fmt=BF16, out="bf16", law="normal", c=11),
}


def workload_inputs(name: str):
    """(A_bits, B_bits, spec) for a named workload."""
    w = WORKLOADS[name]
    law = {"uniform": uniform, "normal": normal, "ints": ints, "quarter": quarter}[w["law"]]
    off = 10 if w["law"] == "ints" else 0
    A = law((w["M"], w["K"]), 100 * w["c"] + 1 + off, w["fmt"])
    B = law((w["K"], w["N"]), 100 * w["c"] + 2 + off, w["fmt"])
    return A, B, w
