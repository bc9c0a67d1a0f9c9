"""Pins for the oracle's FP8 codec against the pages, torch's float8 types and
the closed form of the formats (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_fp8_constants.json")
TORCH_T = {oracle.FMT_E4M3: torch.float8_e4m3fn, oracle.FMT_E5M2: torch.float8_e5m2}
FPMAX = {oracle.FMT_E4M3: 448.0, oracle.FMT_E5M2: 57344.0}
MINSUB = {oracle.FMT_E4M3: 2.0 ** -9, oracle.FMT_E5M2: 2.0 ** -16}
FMTS = [oracle.FMT_E4M3, oracle.FMT_E5M2]


def torch_decode(codes: np.ndarray, fmt: int) -> np.ndarray:
    return torch.from_numpy(codes.astype(np.uint8)).view(TORCH_T[fmt]).to(torch.float64).numpy()


def torch_encode(y: np.ndarray, fmt: int) -> np.ndarray:
    return torch.from_numpy(y.astype(np.float64)).to(TORCH_T[fmt]).view(torch.uint8).numpy()


@pytest.mark.parametrize("fmt", FMTS)
def test_decode_all_codes_match_torch(fmt):
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.fp8_decode(codes, fmt)
    ref = torch_decode(codes, fmt)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def test_decode_special_counts():
    e4 = oracle.fp8_decode(np.arange(256, dtype=np.uint8), oracle.FMT_E4M3)
    e5 = oracle.fp8_decode(np.arange(256, dtype=np.uint8), oracle.FMT_E5M2)
    assert np.isnan(e4).sum() == 2 and np.isinf(e4).sum() == 0
    assert np.isnan(e5).sum() == 6 and np.isinf(e5).sum() == 2
    assert oracle.fp8_decode(np.array([0x7F, 0xFF], np.uint8), 0).tolist() != [0, 0]


@pytest.mark.parametrize("fmt", FMTS)
def test_decode_closed_form(fmt):
    """Every finite magnitude equals 2^(e-bias)(1+m/2^M) or 2^(1-bias) m/2^M."""
    eb, mb, bias = (4, 3, 7) if fmt == oracle.FMT_E4M3 else (5, 2, 15)
    vals = oracle.fp8_decode(np.arange(128, dtype=np.uint8), fmt)
    for c in range(128):
        e, m = c >> mb, c & ((1 << mb) - 1)
        if not np.isfinite(vals[c]):
            continue
        want = (2.0 ** (e - bias)) * (1 + m / 2 ** mb) if e else (2.0 ** (1 - bias)) * m / 2 ** mb
        assert vals[c] == want
    assert vals[0x7E if fmt == 0 else 0x7B] == FPMAX[fmt]
    assert vals[1] == MINSUB[fmt]
    assert oracle.fp8_range(fmt) == FPMAX[fmt] / MINSUB[fmt]


def test_page_printed_constants():
    """The article's E4M3 extremes and range, and the guide's bit layouts."""
    g = json.load(open(GOLDEN))
    vals = oracle.fp8_decode(np.arange(128, dtype=np.uint8), oracle.FMT_E4M3)
    fin = vals[np.isfinite(vals) & (vals > 0)]
    assert fin.max() == g["e4m3_max_representable_printed"]
    assert round(fin.min(), 5) == g["e4m3_min_representable_printed"]
    rng = oracle.fp8_range(oracle.FMT_E4M3)
    assert rng == 229376.0
    # "about 200000": one significant figure
    assert round(rng, -5) == g["e4m3_dynamic_range_printed_approx"]
    # bit layouts: 2^(exponent bits) binades, 2^(mantissa bits) steps per binade
    for fmt, key in ((0, "e4m3_sign_exponent_mantissa_bits"), (1, "e5m2_sign_exponent_mantissa_bits")):
        sb, eb, mb = g[key]
        assert sb + eb + mb == 8
        v = oracle.fp8_decode(np.arange(128, dtype=np.uint8), fmt)
        # the first normal binade [2^(1-bias), 2^(2-bias)) holds 2^mb codes
        bias = 2 ** (eb - 1) - 1
        lo, hi = 2.0 ** (1 - bias), 2.0 ** (2 - bias)
        assert ((v >= lo) & (v < hi)).sum() == 2 ** mb


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_roundtrips_every_finite_code(fmt):
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.fp8_decode(codes, fmt)
    fin = np.isfinite(vals)
    back = oracle.fp8_encode(vals[fin], fmt)
    assert np.array_equal(back, codes[fin])


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_midpoints_tie_to_even(fmt):
    vals = oracle.fp8_decode(np.arange(128, dtype=np.uint8), fmt)
    top = 0x7E if fmt == 0 else 0x7B
    lo = vals[:top]
    hi = vals[1:top + 1]
    mid = 0.5 * (lo + hi)
    got = oracle.fp8_encode(mid, fmt)
    c = np.arange(top)
    want = np.where(c % 2 == 0, c, c + 1)
    assert np.array_equal(got, want)
    # a hair below/above goes to the nearer neighbour
    assert np.array_equal(oracle.fp8_encode(np.nextafter(mid, -np.inf), fmt), c)
    assert np.array_equal(oracle.fp8_encode(np.nextafter(mid, np.inf), fmt), c + 1)
    # negative side mirrors with the sign bit
    assert np.array_equal(oracle.fp8_encode(-mid, fmt), want | 0x80)


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_matches_torch_cast_in_range(fmt):
    rng = np.random.default_rng(123 + fmt)
    y = np.concatenate([
        rng.uniform(-FPMAX[fmt], FPMAX[fmt], 200000),
        np.sign(rng.standard_normal(200000)) * 10.0 ** rng.uniform(-8, np.log10(FPMAX[fmt]), 200000),
        rng.uniform(-4 * MINSUB[fmt], 4 * MINSUB[fmt], 50000),
    ])
    assert np.array_equal(oracle.fp8_encode(y, fmt), torch_encode(y, fmt))


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_saturates_and_specials(fmt):
    top = 0x7E if fmt == 0 else 0x7B
    big = np.array([FPMAX[fmt] * 1.0001, FPMAX[fmt] * 1.1, 1e30, np.inf])
    assert np.all(oracle.fp8_encode(big, fmt) == top)
    assert np.all(oracle.fp8_encode(-big, fmt) == (top | 0x80))
    assert oracle.fp8_encode(np.array([np.nan]), fmt)[0] == 0x7F
    assert oracle.fp8_encode(np.array([0.0]), fmt)[0] == 0x00
    assert oracle.fp8_encode(np.array([-0.0]), fmt)[0] == 0x80
    # below half the smallest subnormal rounds to zero; exactly half ties to 0 (even)
    assert oracle.fp8_encode(np.array([MINSUB[fmt] * 0.5]), fmt)[0] == 0x00
    assert oracle.fp8_encode(np.array([MINSUB[fmt] * 0.5000001]), fmt)[0] == 0x01


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_is_nearest_by_brute_force(fmt):
    """Against a linear scan over all finite values (nearest, ties to even code)."""
    vals = oracle.fp8_decode(np.arange(128, dtype=np.uint8), fmt)
    top = 0x7E if fmt == 0 else 0x7B
    grid = vals[:top + 1]
    rng = np.random.default_rng(7)
    y = 10.0 ** rng.uniform(np.log10(MINSUB[fmt]) - 1, np.log10(FPMAX[fmt]), 3000)
    got = oracle.fp8_encode(y, fmt)
    for yi, gi in zip(y, got):
        d = np.abs(grid - yi)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert gi == want
