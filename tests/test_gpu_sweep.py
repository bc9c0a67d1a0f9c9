"""The variant sweep's codec errors on the GPU against the oracle.

For each group size, format and expansion setting, page-shaped prior moments
(about 1000:1 for m and 10:1 for v within a group) are quantized and
dequantized through the C ABI, and bench.quant_error_sums of the result must
match the same errors of the oracle's quantize/dequantize, computed here with
numpy. The article's orderings ("Solution: dynamic range expansion":
expansion lowers the error; E4M3 suits the first moment better than E5M2) are
checked on the GPU figures."""
import numpy as np
import pytest
import torch

import bench
import oracle
import synth
from _parity import log

pytestmark = pytest.mark.gpu
E4, E5, NOEXP = 0, 1, 0x100


@pytest.fixture(scope="module")
def coat():
    import fp8_optimizer_state_amd as c
    assert torch.cuda.is_available()
    c.lib()
    return c


def oracle_errors(x, G, fmt):
    q, s, k = oracle.quantize(x, G, fmt)
    xd = oracle.dequantize(q, s, k, G, fmt & 0xFF)
    n = x.size
    pad = (-n) % G
    xs = np.pad(x, (0, pad)).reshape(-1, G)
    d = np.pad(xd - x, (0, pad)).reshape(-1, G)
    nx = np.linalg.norm(xs, axis=1)
    live = nx > 0
    nz = x != 0
    return (np.mean(np.linalg.norm(d, axis=1)[live] / nx[live]),
            np.mean(np.abs(xd - x)[nz] / np.abs(x)[nz]))


def gpu_errors(coat, x, G, fmt):
    xt = torch.from_numpy(x.astype(np.float32)).cuda()
    n = xt.numel()
    ng = (n + G - 1) // G
    q = torch.empty(n, dtype=torch.uint8, device="cuda")
    s = torch.empty(ng, dtype=torch.float64, device="cuda")
    k = torch.empty(ng, dtype=torch.float32, device="cuda")
    coat.quantize(xt, q, s, k, group=G, fmt=fmt)
    xh = torch.empty_like(xt)
    coat.dequantize(q, s, k, xh, group=G, fmt=fmt & 0xFF)
    sn, cn, se, ce = bench.quant_error_sums(xt, xh, G)
    return sn / cn, se / ce


@pytest.mark.parametrize("G", [32, 64, 128, 256])
def test_sweep_errors_match_oracle(coat, G):
    n = (1 << 17) + 3 * G // 2  # a ragged last group
    m, v = synth.prior_moments(n, G, seed=11, tensor=G)
    out = {}
    for name, x in (("m", m.numpy().astype(np.float64)), ("v", v.numpy().astype(np.float64))):
        for fmt in (E4, E5):
            for exp in (True, False):
                f = fmt if exp else fmt | NOEXP
                got = gpu_errors(coat, x, G, f)
                want = oracle_errors(x, G, f)
                log(f"[sweep G={G} {name} fmt={fmt} expand={exp}] gpu {got[0]:.6g} {got[1]:.6g} "
                    f"oracle {want[0]:.6g} {want[1]:.6g}")
                assert abs(got[0] - want[0]) <= 1e-6 * want[0]
                assert abs(got[1] - want[1]) <= 1e-6 * want[1]
                out[(name, fmt, exp)] = got[0]
    for name in ("m", "v"):
        for fmt in (E4, E5):
            assert out[(name, fmt, True)] < out[(name, fmt, False)]
    assert out[("m", E4, True)] < out[("m", E5, True)]
