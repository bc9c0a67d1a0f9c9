"""The sweep's quantization-error metric (bench.quant_error_sums), pinned on the
CPU against its definition written out element by element: per-group normwise
error ||x_hat - x||_2 / ||x||_2 over groups of G consecutive elements (a short
last group included, zero groups skipped) and the element-wise relative error
over nonzero elements."""
import math

import numpy as np
import torch

import bench


def brute(x, xh, G):
    n = len(x)
    sn, cn, se, ce = 0.0, 0, 0.0, 0
    for g0 in range(0, n, G):
        num = math.sqrt(sum((xh[i] - x[i]) ** 2 for i in range(g0, min(n, g0 + G))))
        den = math.sqrt(sum(x[i] ** 2 for i in range(g0, min(n, g0 + G))))
        if den > 0:
            sn += num / den
            cn += 1
    for i in range(n):
        if x[i] != 0:
            se += abs(xh[i] - x[i]) / abs(x[i])
            ce += 1
    return sn, cn, se, ce


def test_closed_form():
    # every element off by 10 %: both metrics are 0.1
    x = torch.linspace(-3, 5, 96, dtype=torch.float64)
    x[x == 0] = 1.0
    sn, cn, se, ce = bench.quant_error_sums(x.float(), (1.1 * x).float(), 32)
    assert cn == 3 and ce == 96
    assert abs(sn / cn - 0.1) < 1e-6 and abs(se / ce - 0.1) < 1e-6


def test_against_brute_force():
    rng = np.random.default_rng(7)
    for n, G in ((1000, 32), (257, 16), (64, 64), (130, 128)):
        x = rng.standard_normal(n).astype(np.float32)
        x[rng.random(n) < 0.1] = 0.0
        x[:G] = 0.0  # one all-zero group, skipped by the normwise mean
        xh = (x * (1 + 0.01 * rng.standard_normal(n))).astype(np.float32)
        got = bench.quant_error_sums(torch.from_numpy(x), torch.from_numpy(xh), G)
        want = brute(x.astype(np.float64).tolist(), xh.astype(np.float64).tolist(), G)
        assert got[1] == want[1] and got[3] == want[3]
        assert abs(got[0] - want[0]) <= 1e-12 * max(1.0, want[0])
        assert abs(got[2] - want[2]) <= 1e-12 * max(1.0, want[2])
