"""Pins for the oracle's per-group quantization with dynamic range expansion.

What fixes the method without retyping it: the expanded group spans exactly
the FP8 range, its extremes land on the largest code and on the smallest
subnormal, k is the largest exponent that keeps every nonzero member at or
above the smallest subnormal (brute force), k = 1 is plain absmax
quantization (torch's float8 cast), and grid values round-trip.
"""
import numpy as np
import pytest
import torch

import oracle

E4, E5, NOEXP = oracle.FMT_E4M3, oracle.FMT_E5M2, oracle.FMT_NO_EXPAND
FPMAX = {E4: 448.0, E5: 57344.0}
MINSUB = {E4: 2.0 ** -9, E5: 2.0 ** -16}
TOP = {E4: 0x7E, E5: 0x7B}
TORCH_T = {E4: torch.float8_e4m3fn, E5: torch.float8_e5m2}


def page_groups(ng, G, kind, seed):
    """Groups shaped like the article's states: m spans ~1000:1, v ~10:1."""
    rng = np.random.default_rng(seed)
    scale = 10.0 ** rng.uniform(-5, -2, ng).repeat(G)
    if kind == "m":
        x = np.where(rng.random(ng * G) < 0.5, -1.0, 1.0) * scale * 10.0 ** rng.uniform(-3, 0, ng * G)
    else:
        x = scale * scale * 10.0 ** rng.uniform(-1, 0, ng * G)
    return x


@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("kind", ["m", "v"])
def test_expanded_range_equals_fp8_range(fmt, kind):
    G, ng = 128, 500
    x = page_groups(ng, G, kind, 1 + fmt)
    q, s, k = oracle.quantize(x, G, fmt)
    xs = np.abs(x.reshape(ng, G))
    amax, amin = xs.max(1), np.where(xs > 0, xs, np.inf).min(1)
    expanded_ratio = (amax / amin) ** k.astype(np.float64)  # max|f| / min|f|
    rf = oracle.fp8_range(fmt)
    assert np.all(np.abs(expanded_ratio / rf - 1) < 1e-4)
    # stored s is max|f| / fpmax
    assert np.allclose(s, amax ** k.astype(np.float64) / FPMAX[fmt], rtol=1e-14, atol=0)
    # the largest member takes the largest code, the smallest nonzero the smallest subnormal
    qg = q.reshape(ng, G) & 0x7F
    rows = np.arange(ng)
    assert np.all(qg[rows, xs.argmax(1)] == TOP[fmt])
    assert np.all(qg[rows, np.where(xs > 0, xs, np.inf).argmin(1)] == 0x01)


@pytest.mark.parametrize("fmt", [E4, E5])
def test_codes_monotone_in_magnitude(fmt):
    G, ng = 64, 200
    x = page_groups(ng, G, "m", 9)
    q, _, _ = oracle.quantize(x, G, fmt)
    for gi in range(ng):
        xs = np.abs(x[gi * G:(gi + 1) * G])
        c = q[gi * G:(gi + 1) * G] & 0x7F
        order = np.argsort(xs, kind="stable")
        assert np.all(np.diff(c[order].astype(int)) >= 0)
    assert np.array_equal(q >> 7, (np.signbit(x)).astype(np.uint8))


@pytest.mark.parametrize("fmt", [E4, E5])
def test_k_is_largest_exponent_keeping_all_members_representable(fmt):
    """Brute force over a fine k grid on tiny groups (G = 4..16)."""
    rng = np.random.default_rng(31 + fmt)
    kgrid = np.arange(0.05, 40.0, 1e-4)
    for trial in range(60):
        G = int(rng.integers(4, 17))
        x = 10.0 ** rng.uniform(-6, -1, G) * np.where(rng.random(G) < 0.5, -1, 1)
        if trial % 7 == 0:
            x[: G // 2] = 0.0  # zeros do not count as the minimum
        _, _, k = oracle.quantize(x, G, fmt)
        a = np.abs(x)
        amax, amin = a.max(), a[a > 0].min()
        ok = FPMAX[fmt] * (amin / amax) ** kgrid >= MINSUB[fmt]
        k_brute = kgrid[ok].max()
        assert abs(k[0] - k_brute) <= 2e-4 * max(1.0, k_brute)


@pytest.mark.parametrize("fmt", [E4, E5])
def test_no_expansion_is_plain_absmax_quantization(fmt):
    """k forced to 1 equals torch's float8 cast of x / (amax / fpmax)."""
    G, ng = 128, 300
    x = page_groups(ng, G, "m", 5)
    q, s, k = oracle.quantize(x, G, fmt | NOEXP)
    assert np.all(k == 1.0)
    xs = x.reshape(ng, G)
    amax = np.abs(xs).max(1, keepdims=True)
    assert np.array_equal(s, amax[:, 0] / FPMAX[fmt])
    ref = torch.from_numpy(xs / (amax / FPMAX[fmt])).to(TORCH_T[fmt]).view(torch.uint8).numpy()
    mism = (ref.ravel() != q).mean()
    assert mism <= 1e-4  # only exact ties could differ (different rounding of y)
    # and dequantization is then just code value times s
    xd = oracle.dequantize(q, s, k, G, fmt)
    want = oracle.fp8_decode(q, fmt) * s.repeat(G)
    assert np.allclose(xd, want, rtol=1e-15, atol=0)


@pytest.mark.parametrize("fmt", [E4, E5])
def test_grid_values_roundtrip(fmt):
    """x_c = amax (v_c / fpmax)^(1/k): quantizes back to c, dequantizes to x_c."""
    rng = np.random.default_rng(77 + fmt)
    vals = oracle.fp8_decode(np.arange(128, dtype=np.uint8), fmt)
    G = 32
    for trial in range(50):
        codes = rng.integers(1, TOP[fmt] + 1, G).astype(np.uint8)
        codes[0], codes[1] = TOP[fmt], 0x01  # span the whole range so k is what we chose
        k = float(np.float32(oracle.group_k(1.0, 1.0 / 10 ** rng.uniform(0.5, 8), fmt)))
        amax = 10.0 ** rng.uniform(-9, 0)
        x = amax * (vals[codes] / FPMAX[fmt]) ** (1.0 / k)
        x *= np.where(rng.random(G) < 0.5, -1, 1)
        q, s, kk = oracle.quantize(x, G, fmt)
        assert abs(kk[0] - k) <= 2e-7 * k
        assert np.array_equal(q & 0x7F, codes)
        xd = oracle.dequantize(q, s, kk, G, fmt)
        assert np.allclose(xd, x, rtol=1e-9, atol=0)


def test_degenerate_groups():
    G = 16
    # all zero, with signed zeros kept in the sign bit
    x = np.zeros(G)
    x[3] = -0.0
    q, s, k = oracle.quantize(x, G, E4)
    assert s[0] == 0.0 and k[0] == 1.0
    assert q[3] == 0x80 and np.all(np.delete(q, 3) == 0)
    assert np.all(oracle.dequantize(q, s, k, G, E4) == 0.0)
    # one nonzero member: ratio 1 -> k = 1, member takes the top code
    x = np.zeros(G)
    x[5] = -3e-4
    q, s, k = oracle.quantize(x, G, E4)
    assert k[0] == 1.0 and q[5] == (0x80 | 0x7E) and np.isclose(s[0], 3e-4 / 448)
    # near-constant group: ratio <= 1 + 1e-6 -> k = 1
    x = 1e-3 * (1 + np.linspace(0, 0.9e-6, G))
    _, _, k = oracle.quantize(x, G, E4)
    assert k[0] == 1.0
    # just above the threshold: the formula's k (about 8.9e6) is cut by the range
    # guard to the largest value with amax^k / R_fp8 still a normal fp64
    x = 1e-3 * (1 + np.linspace(0, 2e-6, G))
    _, s, k = oracle.quantize(x, G, E4)
    bound = (1022 - np.log2(oracle.fp8_range(E4))) / -np.log2(x.max())
    assert abs(k[0] - bound) < 1e-4 * bound and np.isfinite(s[0]) and s[0] >= 2.0 ** -1022


def test_k_below_one_when_group_outspans_fp8():
    """No clamp: a group wider than R_fp8 gets k < 1 and keeps its smallest member."""
    G = 8
    x = np.array([1.0, 1e-9, 0.5, 1e-3, 2e-7, 0.1, 3e-2, 4e-8])
    q, s, k = oracle.quantize(x, G, E4)
    assert k[0] < 1.0
    assert q[1] & 0x7F == 0x01 and q[0] == 0x7E
    assert np.allclose(oracle.dequantize(q, s, k, G, E4)[[0, 1]], [1.0, 1e-9], rtol=1e-12)


def test_short_tail_group_and_independence():
    G = 128
    rng = np.random.default_rng(3)
    x = page_groups(3, G, "m", 4)[: 2 * G + 37]
    q, s, k = oracle.quantize(x, G, E4)
    assert q.size == x.size and s.size == 3
    q2, s2, k2 = oracle.quantize(x[2 * G:], G, E4)
    assert np.array_equal(q[2 * G:], q2) and s[2] == s2[0] and k[2] == k2[0]


def test_nonfinite_member_poisons_only_its_group():
    G = 32
    x = page_groups(3, G, "m", 8)
    x[G + 5] = np.nan
    q, s, k = oracle.quantize(x, G, E4)
    q0, s0, k0 = oracle.quantize(np.concatenate([x[:G], x[2 * G:]]), G, E4)
    assert np.isnan(s[1]) and k[1] == 1.0 and np.all(q[G:2 * G] == 0x7F)
    assert np.array_equal(q[:G], q0[:G]) and np.array_equal(q[2 * G:], q0[G:])
    assert np.isnan(oracle.dequantize(q, s, k, G, E4)[G:2 * G]).all()
    x[G + 5] = np.inf
    q, s, k = oracle.quantize(x, G, E5)
    assert np.isnan(s[1]) and np.all(q[G:2 * G] == 0x7F)


@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("amax", [1e-300, 3e-250, 1e-200, 1e250, 1e300])
def test_range_guard_keeps_scale_normal(fmt, amax):
    """Tiny or huge narrow groups: k is lowered so amax^k and amax^k/R_fp8 stay in
    [2^-1022, 2^1023]; the result is the largest such fp32 k."""
    G = 16
    x = amax * (1 + np.linspace(0, 1.0, G))  # ratio 2 -> unguarded k is 17.8 / 31.8
    q, s, k = oracle.quantize(x, G, fmt)
    kk = float(k[0])
    rf = oracle.fp8_range(fmt)
    top = np.abs(x).max()
    f_max = top ** kk
    assert f_max <= 2.0 ** 1023 and f_max / rf >= 2.0 ** -1022
    assert kk <= float(oracle.group_k(top, np.abs(x).min(), fmt | 0)) + 0
    # k is the largest fp32 with that property
    k_up = float(np.nextafter(np.float32(kk), np.float32(np.inf)))
    unguarded = np.log(rf) / np.log(top / np.abs(x).min())
    if k_up <= unguarded:
        f_up = top ** k_up
        assert f_up > 2.0 ** 1023 or f_up / rf < 2.0 ** -1022
    assert np.isfinite(s[0]) and s[0] >= 2.0 ** -1022
    xd = oracle.dequantize(q, s, k, G, fmt)
    assert np.all(np.isfinite(xd))
    assert np.allclose(xd[-1], x[-1], rtol=1e-12)


def test_fp64_subnormal_members():
    G = 8
    x = np.array([5e-324, 1e-320, 2e-310, 1e-308, 3e-309, 0.0, 7e-322, 1e-315])
    q, s, k = oracle.quantize(x, G, E4)
    assert np.isfinite(s[0]) and s[0] > 0
    xd = oracle.dequantize(q, s, k, G, E4)
    assert xd[3] == pytest.approx(1e-308, rel=1e-9) and xd[5] == 0.0


def test_near_constant_threshold_is_the_rounded_quotient():
    """k = 1 exactly when the fp64 quotient amax / amin rounds to at most
    1 + 1e-6 (the constant as fp64): pairs whose rounded quotient is that
    constant minus two ulps up to plus two ulps, at several scales."""
    T = 1.0 + 1e-6
    U = np.spacing(T)
    rng = np.random.default_rng(5)
    seen = set()
    for _ in range(4000):
        b = float(np.ldexp(1.0 + rng.random(), int(rng.integers(-200, 200))))
        a = float(b * T)
        for _k in range(int(rng.integers(0, 5))):
            a = float(np.nextafter(a, np.inf if rng.random() < 0.5 else -np.inf))
        off = round((a / b - T) / U)
        if abs(off) > 2 or a / b != T + off * U:
            continue
        seen.add(off)
        for fmt in (E4, E5):
            k = oracle.group_k(a, b, fmt)
            assert (k == 1.0) == (off <= 0), (a, b, off, k)
    assert seen == {-2, -1, 0, 1, 2}


def test_step_poisons_each_moment_on_its_own():
    """A poisoned stored first moment (s = NaN, codes 0x7F) leaves the second
    moment's group finite, and the reverse."""
    G, n = 32, 128
    rng = np.random.default_rng(6)
    m = rng.uniform(1e-4, 1e-3, n) * np.where(rng.random(n) < 0.5, -1, 1)
    v = rng.uniform(1e-8, 1e-7, n)
    mq, ms, mk = oracle.quantize(m, G, E4)
    vq, vs, vk = oracle.quantize(v, G, E5)
    mq[:G], ms[0], mk[0] = 0x7F, np.nan, 1.0
    vq[2 * G:3 * G], vs[2], vk[2] = 0x7F, np.nan, 1.0
    p = rng.normal(0, 0.02, n).astype(np.float32)
    g = (rng.normal(0, 1e-3, n).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    r = oracle.adamw_step(p, g, mq, ms, mk, vq, vs, vk, G, E4, E5, 1e-4, 0.9, 0.95, 1e-8, 0.1, 10)
    assert np.isnan(r["ms"][0]) and (r["mq"][:G] == 0x7F).all() and np.isfinite(r["vs"][0])
    assert np.isnan(r["vs"][2]) and (r["vq"][2 * G:3 * G] == 0x7F).all() and np.isfinite(r["ms"][2])
    assert np.isfinite(r["ms"][[1, 3]]).all() and np.isfinite(r["vs"][[1, 3]]).all()
    assert np.isnan(r["p"][:G]).all() and np.isfinite(r["p"][G:2 * G]).all()


def test_step_with_huge_grads_stays_finite():
    """Grads near the bf16 maximum give moments beyond the fp32 range but
    finite in fp64: no group is poisoned and the update equals the dense
    AdamW of the dequantized state (the quantization being the only other
    step)."""
    G, n = 32, 64
    rng = np.random.default_rng(7)
    m = rng.uniform(1e-4, 1e-3, n)
    v = rng.uniform(1e-8, 1e-7, n)
    mq, ms, mk = oracle.quantize(m, G, E4)
    vq, vs, vk = oracle.quantize(v, G, E5)
    gf = rng.normal(0, 1e-3, n).astype(np.float32)
    gf[:5] = [1e20, -3e20, 3e38, -3.3e38, 2e25]
    g = (gf.view(np.uint32) >> 16).astype(np.uint16)
    p = rng.normal(0, 0.02, n).astype(np.float32)
    r = oracle.adamw_step(p, g, mq, ms, mk, vq, vs, vk, G, E4, E5, 1e-4, 0.9, 0.95, 1e-8, 0.1, 10)
    assert np.isfinite(r["ms"]).all() and np.isfinite(r["vs"]).all()
    md = oracle.dequantize(mq, ms, mk, G, E4)
    vd = oracle.dequantize(vq, vs, vk, G, E5)
    pd, _, _, _ = oracle.adamw_dense(p, g, md, vd, 1e-4, 0.9, 0.95, 1e-8, 0.1, 10)
    assert np.array_equal(r["p"], pd)
    assert np.isfinite(r["p"]).all()
