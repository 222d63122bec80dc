"""The kernels' exact-quotient arithmetic, checked in exact rational arithmetic on the CPU.

The GPU quantizers form the code of y from fl32(y / s) without a division:
r = fl32(1/s) (correctly rounded), t = fl32(y * r), e = fl32(y - t * s) (one
FMA), q = fl32(t + e * r) (one FMA).  A row whose nonzero scale is below 2^-90
has its values and scale multiplied by 2^64 first.  The claim is that q equals
the IEEE quotient fl32(y / s) wherever a code depends on it (|y / s| >= 2^-10,
E4M3FN's smallest rounding boundary; int8's is 1/2) -- in fact everywhere the
residual stays out of the subnormal range -- so the int8 codes
(round half to even of q) and E4M3FN codes are those of the IEEE division.

Each fp32 operation is emulated here with one correct rounding of its exact
rational result (round to nearest even, subnormals included), which is what the
GPU's multiply and FMA do.  Cases: random pairs over the scale range, quotients
placed within a few ulps of int8 and E4M3FN rounding boundaries, and scales
from the smallest subnormal up, on both sides of the 2^-90 threshold.  This pins
the method, not the oracle (which divides) and not the GPU (whose bytes the GPU
parity tests compare with the oracle's).
"""
import random
from fractions import Fraction as F

import numpy as np

TINY = 2.0 ** -90
RESCALE = 2.0 ** 64


def rn32(x: F) -> float:
    """Nearest binary32 value of the rational x, ties to even, subnormals included."""
    if x == 0:
        return 0.0
    sign = -1.0 if x < 0 else 1.0
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if F(2) ** e > a:
        e -= 1
    elif F(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    quantum = F(2) ** (e - 23)
    n = a / quantum
    m = n.numerator // n.denominator
    rem = n - m
    if rem > F(1, 2) or (rem == F(1, 2) and m % 2 == 1):
        m += 1
    v = float(m * quantum)
    assert v < 2.0 ** 128, "no overflow in these cases"
    return sign * v


def kernel_quotient(y: float, s: float) -> float:
    """The kernels' steps, each fp32 operation rounded once."""
    pre = 1.0
    if 0.0 < s < TINY:
        pre = RESCALE
        s = rn32(F(s) * F(pre))          # exact: a power-of-two product
        y = rn32(F(y) * F(pre))
    r = rn32(1 / F(s)) if s > 0 else 0.0
    t = rn32(F(y) * F(r))
    e = rn32(F(y) - F(t) * F(s))         # fma(-t, s, y)
    return rn32(F(e) * F(r) + F(t))      # fma(e, r, t)


def f32(v) -> float:
    return float(np.float32(v))


def rand_f32(rng: random.Random, lo_exp: int, hi_exp: int) -> float:
    m = rng.randint(1 << 23, (1 << 24) - 1)
    return f32(m * 2.0 ** (rng.randint(lo_exp, hi_exp) - 23))


def check(y: float, s: float) -> bool:
    """Kernel quotient == IEEE quotient where a code depends on it; False if skipped."""
    exact = F(y) / F(s)
    if abs(exact) < F(1, 1024):
        return False
    want = rn32(exact)
    got = kernel_quotient(y, s)
    assert got == want, f"y={y!r} s={s!r}: kernel {got!r}, IEEE {want!r}"
    # the scaled values must be exact (the pre-factor loses nothing)
    if 0.0 < s < TINY:
        assert F(rn32(F(y) * F(RESCALE))) == F(y) * F(RESCALE)
    return True


def test_rn32_matches_numpy_on_doubles():
    rng = random.Random(1)
    for _ in range(3000):
        d = rng.uniform(-1, 1) * 2.0 ** rng.randint(-160, 100)
        assert rn32(F(d)) == float(np.float32(d)) or abs(d) < 2.0 ** -150


def test_random_pairs_across_scales():
    rng = random.Random(2)
    done = 0
    for _ in range(4000):
        s = rand_f32(rng, -126, 20)                  # normal scales (subnormal ones below)
        qmax = 127.0 if rng.random() < 0.5 else 448.0
        y = f32(rng.uniform(-qmax, qmax) * s)
        if np.isfinite(y) and y != 0.0:
            done += check(y, s)
    assert done > 3500


def test_near_rounding_boundaries():
    """Quotients within a few ulps of an int8 half-integer or an E4M3FN midpoint."""
    rng = random.Random(3)
    # E4M3FN midpoints: halfway between consecutive representable magnitudes
    e4m3 = sorted({m * 2.0 ** (e - 3) for e in range(-6, 9) for m in range(8, 16)} |
                  {m * 2.0 ** -9 for m in range(0, 8)})
    e4m3 = [v for v in e4m3 if v <= 448.0]
    mids = [(a + b) / 2 for a, b in zip(e4m3, e4m3[1:])]
    halves = [k + 0.5 for k in range(0, 127)]
    for _ in range(3000):
        s = rand_f32(rng, -100, 10)
        target = rng.choice(halves) if rng.random() < 0.5 else rng.choice(mids)
        y0 = f32(target * s)
        if y0 == 0.0:
            continue
        # y a few ulps either way of the boundary
        for k in range(-3, 4):
            y = np.float32(y0)
            for _ in range(abs(k)):
                y = np.nextafter(y, np.float32(np.inf if k > 0 else -np.inf))
            sgn = -1.0 if rng.random() < 0.5 else 1.0
            check(sgn * float(y), s)


def test_tiny_scales_on_both_sides_of_the_threshold():
    rng = random.Random(4)
    exps = list(range(-149, -80))
    for e in exps:
        for _ in range(40):
            s = f32(rng.randint(1, (1 << 24) - 1) * 2.0 ** (e - 23)) if e > -126 else f32(
                rng.randint(1, (1 << 23) - 1) * 2.0 ** -149)
            if s == 0.0:
                continue
            qmax = 127.0 if rng.random() < 0.5 else 448.0
            # mostly ordinary quotients, some just above E4M3FN's smallest boundary
            q = rng.uniform(-qmax, qmax) if rng.random() < 0.8 else rng.uniform(2.0 ** -10, 2.0 ** -8)
            y = f32(q * s)
            if y != 0.0:
                check(y, s)


def test_without_the_rescale_tiny_scales_can_fail():
    """The pre-factor is needed: without it the steps miss the IEEE quotient at small
    normal scales (here 2^-126 .. 2^-116, quotients near rounding boundaries; the
    residual falls into the subnormal range), and below 2^-128 the reciprocal
    overflows binary32 outright.  With it, the same cases all agree."""
    rng = random.Random(5)
    e4m3 = sorted({m * 2.0 ** (e - 3) for e in range(-6, 9) for m in range(8, 16)})
    mids = [(a + b) / 2 for a, b in zip(e4m3, e4m3[1:]) if b <= 448.0]
    halves = [k + 0.5 for k in range(127)]
    misses = checked = 0
    for _ in range(1500):
        s = rand_f32(rng, -126, -116)
        target = rng.choice(halves) if rng.random() < 0.5 else rng.choice(mids)
        y = f32(target * s)
        if y == 0.0:
            continue
        r = rn32(1 / F(s))
        t = rn32(F(y) * F(r))
        e = rn32(F(y) - F(t) * F(s))
        misses += rn32(F(e) * F(r) + F(t)) != rn32(F(y) / F(s))
        checked += check(y, s)          # the kernels' steps, with the pre-factor
    assert misses > 0 and checked > 1000
    assert 1 / F(2.0 ** -129) >= F(2) ** 128
