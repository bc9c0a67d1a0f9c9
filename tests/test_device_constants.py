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
    """2^(u + l) = 2^(N >> 5) 2^((N & 31) / 32) 2^((U - N) / 32) 2^l with
    U = 32 u, N = rint(U) and l a small low part, evaluated as the direct path
    does: the polynomial in d = U - N with its coefficients scaled by 32^-i and
    its constant term 1 + l ln 2 (which drops l ln 2 (2^f - 1), at most
    |l| 2^-7 relative). Within 2^-50.3 of 2^(u + l) on a spread of u
    (negatives included) and |l| up to 2^-44, the low part's size for |u|
    near 2^8; within 2^-50.9 for |l| up to 2^-47."""
    import numpy as np
    mp.mp.prec = 200
    t = np.array(_array("kExp2JT"))
    c = _array("kExp2SC")
    deg = len(c) - 1
    cd = [c[i] * 2.0 ** (-5 * (deg - i)) for i in range(deg)]  # highest degree first, without the constant
    rng = np.random.default_rng(5)
    u = np.concatenate([rng.uniform(-60, 60, 400), rng.uniform(-0.05, 0.05, 200), [0.0, -1 / 64, 1 / 64, 31 / 32]])
    for lo_max, bound in ((2.0 ** -44, -50.3), (2.0 ** -47, -50.9)):
        _check_split(t, cd, u, rng.uniform(-1, 1, u.size) * lo_max, bound)


def _check_split(t, cd, u, lo, bound):
    import numpy as np
    U = u * 32.0
    N = np.rint(U)
    d = U - N
    p = np.full_like(d, cd[0])
    for ci in cd[1:]:
        p = p * d + ci
    p = p * d + (1.0 + lo * float.fromhex("0x1.62e42fefa39efp-1"))
    Ni = N.astype(np.int64)
    y = np.ldexp(t[Ni & 31] * p, Ni >> 5)
    worst = max(abs(mp.mpf(float(yi)) / mp.power(2, mp.mpf(float(ui)) + mp.mpf(float(li))) - 1)
                for yi, ui, li in zip(y, u, lo))
    assert float(mp.log(worst, 2)) < bound
