"""The fp64 constants the step kernels evaluate 2^x with, read from the HIP
source and checked against high-precision arithmetic (mpmath, 200 bits): the
table of 2^(j/32) is correctly rounded, and each polynomial stays within the
relative error its comment states over its whole interval. Host-only."""
import os
import re

import mpmath as mp
import pytest

SRC = os.path.join(os.path.dirname(__file__), "..", "fp8_optimizer_state_amd", "csrc", "coat_fp8.hip")


def _array(name):
    text = open(SRC).read()
    m = re.search(r"__device__ constexpr double " + name + r"\[\w+\] = \{(.*?)\};", text, re.S)
    assert m, name
    vals = []
    for tok in m.group(1).replace("\n", " ").split(","):
        tok = tok.strip()
        if tok:
            vals.append(float.fromhex(tok) if "0x" in tok else float(tok))
    return vals


def _worst_rel_error(coef_high_first, h, points=2001):
    """max |p(x) / 2^x - 1| over a uniform grid of [-h, h] plus the ends, in real
    arithmetic on the fp64 coefficients (rounding of the evaluation excluded)."""
    mp.mp.prec = 200
    cs = [mp.mpf(c) for c in coef_high_first]  # stored highest degree first, the Horner order
    worst = mp.mpf(0)
    for i in range(points):
        x = h * (2 * mp.mpf(i) / (points - 1) - 1)
        p = mp.mpf(0)
        for c in cs:
            p = p * x + c
        worst = max(worst, abs(p / mp.power(2, x) - 1))
    return float(mp.log(worst, 2))


def test_exp2_table_is_correctly_rounded():
    mp.mp.prec = 200
    t = _array("kExp2JT")
    assert len(t) == 32
    for j, v in enumerate(t):
        exact = mp.power(2, mp.mpf(j) / 32)
        # correctly rounded: within half an ulp of the exact value
        ulp = 2.0 ** (int(mp.floor(mp.log(exact, 2))) - 52)
        assert abs(mp.mpf(v) - exact) <= mp.mpf(ulp) / 2, j


@pytest.mark.parametrize("name, h, bound", [
    ("kExp2SC", (1 + 2.0 ** -12) / 64, -52.6),   # direct path, per element, |f| <= 1/64
    ("kExp2C", 0.5, -51.5),                       # everything else, |f| <= 1/2
    ("kExp2ShortC", 0.5, -28.5),                  # the fp32-rounded state dequantizer
])
def test_exp2_polynomial_error(name, h, bound):
    coef = _array(name)
    assert coef[-1] == 1.0
    assert _worst_rel_error(coef, h) < bound


def test_split_reproduces_exp2():
    """2^u = 2^(N >> 5) 2^((N & 31) / 32) 2^((U - N) / 32) with U = 32 u,
    N = rint(U), evaluated as the direct path does (fp64 steps, fma where it
    uses one), within 2^-50.5 of 2^u on a spread of u, negatives included."""
    import numpy as np
    mp.mp.prec = 200
    t = np.array(_array("kExp2JT"))
    c = _array("kExp2SC")
    rng = np.random.default_rng(5)
    u = np.concatenate([rng.uniform(-60, 60, 400), rng.uniform(-0.05, 0.05, 200), [0.0, -1 / 64, 1 / 64, 31 / 32]])
    U = u * 32.0
    N = np.rint(U)
    f = (U - N) * 2.0 ** -5
    p = np.full_like(f, c[0])
    for ci in c[1:]:
        p = p * f + ci
    Ni = N.astype(np.int64)
    y = np.ldexp(t[Ni & 31] * p, Ni >> 5)
    worst = max(abs(mp.mpf(float(yi)) / mp.power(2, mp.mpf(float(ui))) - 1) for yi, ui in zip(y, u))
    assert float(mp.log(worst, 2)) < -50.5
