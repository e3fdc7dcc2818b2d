"""Pin of ``oracle.bound_ex`` against an exact emulation of the fp32 epilogue
(no GPU).

The general form act(alpha*A.B + beta*C_old + bias) is evaluated on the
device in fp32, one rounding per step, in this order: the accumulator acc
(within the plain accumulation bound K*2^-20 of the exact dot product d),
v1 = fl(alpha * acc), v2 = fl(beta * C_old + v1) as one fused step when
beta != 0, v3 = fl(v2 + bias), ReLU, then one rounding to the output format.
The acceptance bound ``bound_ex`` claims that

    |y - r| <= e32 = |alpha|*K*2^-20
                     + 2^-22*(|alpha|*(|d| + K*2^-20) + |beta*C_old| + |bias|)
               (+ one ulp of a half-precision output at |r| + e32)

for r = act(alpha*d + beta*C_old + bias), the oracle's exact value.  This
test does not restate that formula as its evidence: it runs the steps above
in exact rational arithmetic (``fractions.Fraction``) with an IEEE
round-to-nearest-even written out here from the definition of the binary
formats (p significand bits, minimum normal exponent), on adversarial
operands -- the accumulator at either end of its allowed interval,
cancellation between alpha*d and beta*C_old, |beta*C_old| >> |alpha*d|,
dominant biases, exact rounding ties, ReLU at the kink, half outputs -- and
checks that

* no emulated error exceeds the bound (the bound is valid), and
* the worst emulated error reaches at least half of the bound (the bound is
  no more than a factor 2 looser than the epilogue it is used for), and, with
  the accumulation term made negligible (K = 1), at least a quarter of the
  rounding part alone.

The rounding routine is itself checked against numpy's IEEE float32 and
float16 casts of exactly representable products.  Precision facts used:
IEEE 754 binary32 (p = 24, emin = -126), binary16 (p = 11, emin = -14) and
bfloat16 (p = 8, emin = -126).
"""
import math
import random
from fractions import Fraction

import numpy as np

import oracle

FMT = {"f32": (24, -126), "f16": (11, -14), "bf16": (8, -126)}


def rne(x: Fraction, fmt: str) -> Fraction:
    """Round the rational x to the nearest value of the binary format ``fmt``,
    ties to the even significand (no overflow in the ranges used here)."""
    if x == 0:
        return Fraction(0)
    p, emin = FMT[fmt]
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()    # 2^e <= a < 2^(e+2)
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)                                              # subnormal quantum below emin
    q = Fraction(2) ** (e - p + 1)
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * q
    return v if x > 0 else -v


def directed(x: Fraction, fmt: str, up: bool) -> Fraction:
    """x rounded toward +infinity (up) or -infinity to the format ``fmt``."""
    if x == 0:
        return Fraction(0)
    p, emin = FMT[fmt]
    e = max(emin, math.floor(math.log2(abs(x))))
    if Fraction(2) ** e > abs(x):                  # log2 rounded up at a power of two
        e -= 1
    q = Fraction(2) ** (max(e, emin) - p + 1)
    n = x / q
    fl = n.numerator // n.denominator              # floor, also for negative n
    if up and fl * q != x:
        fl += 1
    return fl * q


def extreme_acc(d: Fraction, K: int, side: int):
    """The fp32 accumulator farthest from d on one side (side = +1 above,
    -1 below) while still within the accumulation allowance K * 2^-20 of it,
    or None when no fp32 value lies that close to d."""
    lim = Fraction(K, 2 ** 20)
    a = directed(d + lim, "f32", False) if side > 0 else directed(d - lim, "f32", True)
    return a if abs(a - d) <= lim else None


def epilogue(acc, alpha, beta, cold, bias, relu, out):
    """The device epilogue, one IEEE rounding per step."""
    v = rne(alpha * acc, "f32")
    if beta != 0:
        v = rne(beta * cold + v, "f32")            # fused multiply-add: one rounding
    v = rne(v + bias, "f32")
    if relu and v < 0:
        v = Fraction(0)
    return rne(v, out) if out != "f32" else v


def exact(d, alpha, beta, cold, bias, relu):
    v = alpha * d + beta * cold + bias
    return Fraction(0) if relu and v < 0 else v


def ratio(d, K, alpha, beta, cold, bias, relu, out, side):
    """err / bound_ex for one adversarial evaluation."""
    acc = extreme_acc(d, K, side)
    if acc is None:
        return None
    y = epilogue(acc, alpha, beta, cold, bias, relu, out)
    r = exact(d, alpha, beta, cold, bias, relu)
    b = oracle.bound_ex(K, out, np.array([[float(r)]]), alpha=float(alpha), beta=float(beta),
                        C_old=np.array([[float(cold)]]) if beta != 0 else None,
                        bias=np.array([float(bias)]), dot=np.array([[float(d)]]))[0, 0]
    err = abs(y - r)
    return float(err) / b


def f32(x) -> Fraction:
    return rne(Fraction(x), "f32")


def half_value(x, fmt) -> Fraction:
    return rne(Fraction(x), fmt)


def test_rne_matches_ieee_casts():
    """The emulator's rounding against numpy's IEEE casts of exact values
    (products of two fp32 values are exact in float64, so one cast rounds)."""
    rng = random.Random(5)
    for _ in range(3000):
        a = np.float32(rng.uniform(-4, 4) * 2.0 ** rng.randint(-30, 30))
        b = np.float32(rng.uniform(-4, 4) * 2.0 ** rng.randint(-30, 30))
        exact_prod = Fraction(float(a)) * Fraction(float(b))
        assert rne(exact_prod, "f32") == Fraction(float(a * b))
        h = np.float64(rng.uniform(-70000, 70000) * 2.0 ** rng.randint(-30, 0))
        if abs(h) < 65504:
            assert rne(Fraction(float(h)), "f16") == Fraction(float(np.float16(h)))
    # ties go to the even neighbour
    assert rne(Fraction(1) + Fraction(1, 2 ** 24), "f32") == 1
    assert rne(Fraction(1) + Fraction(3, 2 ** 24), "f32") == Fraction(1) + Fraction(2, 2 ** 23)
    assert rne(Fraction(2049), "f16") == 2048 and rne(Fraction(2051), "f16") == 2052
    # subnormal quantum
    assert rne(Fraction(3, 2 ** 26), "f16") == Fraction(1, 2 ** 24)
    assert directed(Fraction(1) + Fraction(1, 2 ** 30), "f32", True) == Fraction(1) + Fraction(1, 2 ** 23)
    assert directed(Fraction(1) - Fraction(1, 2 ** 30), "f32", False) == Fraction(1) - Fraction(1, 2 ** 24)
    assert directed(-Fraction(1) - Fraction(1, 2 ** 30), "f32", True) == -1
    assert directed(-Fraction(1) - Fraction(1, 2 ** 30), "f32", False) == -Fraction(1) - Fraction(1, 2 ** 23)


def _cases():
    """Adversarial (d, K, alpha, beta, C_old, bias, relu, out) tuples.  All
    operands are values the device sees: alpha, beta and bias in fp32, C_old
    in the output format, d a multiple of a small power of two (a dot product
    of half-precision values)."""
    rng = random.Random(11)
    cases = []
    outs = ("f32", "f16", "bf16")
    for out in outs:
        for _ in range(220):
            K = rng.choice([1, 2, 16, 4099])
            # |d| up to 8K: beyond that no fp32 value lies within K*2^-20 of
            # a general d, and the plain accumulation bound cannot hold
            lo, hi = 2.0 ** -12, 8.0 * K
            mag = math.exp(rng.uniform(math.log(lo), math.log(hi)))
            d = Fraction(round(rng.uniform(-1, 1) * mag * 2 ** 24), 2 ** 24)
            alpha = f32(rng.choice([1.0, -1.0, 0.75, -2.5, rng.uniform(-3, 3), 1.0 + 2.0 ** -23]))
            kind = rng.randrange(5)
            beta = Fraction(0)
            cold = Fraction(0)
            bias = Fraction(0)
            if kind == 0:                     # cancellation: beta*C_old ~ -alpha*d
                beta = f32(rng.choice([1.0, -1.0, 0.5, 1.25]))
                cold = half_value(-alpha * d / beta * (1 + rng.uniform(-1e-3, 1e-3)), out)
            elif kind == 1:                   # |beta*C_old| >> |alpha*d|
                beta = f32(rng.uniform(-2, 2))
                cold = half_value(float(d) * rng.uniform(50, 5000) * rng.choice([-1, 1]), out)
            elif kind == 2:                   # dominant bias, possibly cancelling
                bias = f32(-float(alpha * d) * (1 + rng.uniform(-1e-4, 1e-4)))
            elif kind == 3:                   # everything of one sign and size
                beta = f32(rng.uniform(0.5, 2))
                cold = half_value(abs(float(d)) * rng.uniform(0.5, 2) * (1 if d >= 0 else -1), out)
                bias = f32(abs(float(d)) * rng.uniform(0.5, 2) * (1 if d >= 0 else -1))
            relu = rng.random() < 0.3
            cases.append((d, K, alpha, beta, cold, bias, relu, out))
        # exact ties: alpha*acc halfway between fp32 neighbours at every step
        for e in (-20, 0, 7, 15):
            for K in (1, 64):
                unit = Fraction(2) ** e
                d = unit * (1 + Fraction(1, 2 ** 23))            # odd last bit
                cases.append((d, K, Fraction(3, 2), f32(0.5), half_value(unit * 3, out), f32(float(unit)),
                              False, out))
                cases.append((d, K, Fraction(-3, 2), f32(1.0), half_value(unit * Fraction(3, 2), out),
                              Fraction(0), True, out))
    return cases


def test_bound_ex_holds_and_is_tight_on_the_emulated_epilogue():
    worst = {o: 0.0 for o in FMT}
    n = 0
    for (d, K, alpha, beta, cold, bias, relu, out) in _cases():
        for side in (1, -1):
            q = ratio(d, K, alpha, beta, cold, bias, relu, out, side)
            if q is None:
                continue
            assert q <= 1.0, ("bound_ex exceeded", float(d), K, float(alpha), float(beta), float(cold),
                              float(bias), relu, out, side, q)
            worst[out] = max(worst[out], q)
            n += 1
    assert n > 1000
    # The bound is no more than a factor 2 looser than the worst emulated case.
    for out, q in worst.items():
        assert q >= 0.5, (out, q)


def test_rounding_terms_dominate_when_K_is_small():
    """With K = 1 the accumulation allowance is 2^-20, negligible next to
    large operands, so the worst case isolates the epilogue's roundings.
    The bound allows four roundings of 2^-24 of the summed magnitudes; the
    epilogue makes three, each at most half an ulp (2^-24 relative only at
    the bottom of a binade), so random operands reach about 0.4 of it: the
    rounding allowance is valid and within a factor 4 of what the epilogue
    reaches."""
    rng = random.Random(3)
    best = 0.0
    for _ in range(4000):
        d = Fraction(rng.randrange(2 ** 23, 2 ** 24), 2 ** 4)      # an fp32 value: acc = d
        alpha = f32(rng.uniform(0.5, 2.0))
        beta = f32(rng.uniform(0.5, 2.0))
        cold = f32(float(d) * rng.uniform(0.5, 2.0))
        bias = f32(float(d) * rng.uniform(0.5, 2.0))
        q = ratio(d, 1, alpha, beta, cold, bias, False, "f32", 1)
        assert q <= 1.0
        best = max(best, q)
    assert 0.25 <= best <= 0.8, best
