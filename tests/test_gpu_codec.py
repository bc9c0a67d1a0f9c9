"""GPU parity of the codec entry points against the oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
from _parity import code_steps, log, rel_err

pytestmark = pytest.mark.gpu
E4, E5, NOEXP = 0, 1, 0x100
FMTS = [E4, E5]
FPMAX = {E4: 448.0, E5: 57344.0}


@pytest.fixture(scope="module")
def coat():
    import fp8_optimizer_state_amd as c
    assert torch.cuda.is_available()
    c.lib()
    return c


@pytest.mark.parametrize("fmt", FMTS)
def test_decode_all_codes(coat, fmt):
    log(f"test_decode_all_codes fmt={fmt}")
    q = torch.arange(256, dtype=torch.uint8, device="cuda")
    y = torch.empty(256, dtype=torch.float32, device="cuda")
    coat.decode(q, y, fmt=fmt)
    got = y.cpu().numpy().astype(np.float64)
    want = oracle.fp8_decode(np.arange(256, dtype=np.uint8), fmt)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    fin = ~np.isnan(want)
    assert np.array_equal(got[fin], want[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(want[fin]))


def encode_cases(fmt, seed=0):
    """Every finite code value and the midpoints between neighbours with their
    fp32 neighbours, strided sweeps over the fp32 range, and specials."""
    vals = oracle.fp8_decode(np.arange(128, dtype=np.uint8), fmt)
    top = 0x7E if fmt == E4 else 0x7B
    grid = vals[:top + 1].astype(np.float32)
    mids = (0.5 * (vals[:top] + vals[1:top + 1])).astype(np.float32)  # exact in fp32
    near = []
    for base in (grid, mids):
        b = base.astype(np.float32)
        for k in range(1, 4):
            up, dn = b.copy(), b.copy()
            for _ in range(k):
                up = np.nextafter(up, np.float32(np.inf))
                dn = np.nextafter(dn, np.float32(-np.inf))
            near += [up, dn]
    rng = np.random.default_rng(seed)
    sweep = np.arange(0x30000000, 0x48000000, 997, dtype=np.uint32).view(np.float32)  # ~2^-31 .. 2^17
    rnd = (10.0 ** rng.uniform(-12, 6, 200000)).astype(np.float32)
    spec = np.array([0.0, np.inf, FPMAX[fmt] * 2, FPMAX[fmt] * 1.04, 1e-45, 1e-40, 3e38],
                    np.float32)
    y = np.concatenate([grid, mids, *near, sweep, rnd, spec])
    y = np.concatenate([y, -y, np.array([np.nan], np.float32)])
    return y


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_is_exact_rne_saturating(coat, fmt):
    y = encode_cases(fmt)
    log(f"test_encode fmt={fmt} n={y.size}")
    Y = torch.from_numpy(y).cuda()
    Q = torch.empty(y.size, dtype=torch.uint8, device="cuda")
    coat.encode(Y, Q, fmt=fmt)
    got = Q.cpu().numpy()
    want = oracle.fp8_encode(y.astype(np.float64), fmt)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(float(y[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


def page_like(n, G, kind, seed):
    rng = np.random.default_rng(seed)
    ng = (n + G - 1) // G
    scale = np.repeat(10.0 ** rng.uniform(-5, -2, ng), G)[:n]
    if kind == "m":
        x = np.where(rng.random(n) < 0.5, -1.0, 1.0) * scale * 10.0 ** rng.uniform(-3, 0, n)
    else:
        x = scale * scale * 10.0 ** rng.uniform(-1, 0, n)
    return x.astype(np.float32)


@pytest.mark.parametrize("fmt", [E4, E5, E4 | NOEXP, E5 | NOEXP])
@pytest.mark.parametrize("G", [16, 32, 64, 128, 256, 1024])
@pytest.mark.parametrize("n", [1, 1000, 1024 * 37 + 333])
def test_quantize_parity(coat, fmt, G, n):
    for kind in ("m", "v"):
        x = page_like(n, G, kind, seed=G + n + fmt)
        log(f"test_quantize_parity fmt={fmt:#x} G={G} n={n} kind={kind}")
        X = torch.from_numpy(x).cuda()
        ng = (n + G - 1) // G
        Q = torch.empty(n, dtype=torch.uint8, device="cuda")
        S = torch.empty(ng, dtype=torch.float64, device="cuda")
        K = torch.empty(ng, dtype=torch.float32, device="cuda")
        coat.quantize(X, Q, S, K, group=G, fmt=fmt)
        q, s, k = oracle.quantize(x.astype(np.float64), G, fmt)
        assert rel_err(K.cpu().numpy(), k).max() <= 1e-5
        assert rel_err(S.cpu().numpy(), s).max() <= 1e-5
        d = code_steps(Q.cpu().numpy(), q)
        assert d.max() <= 1 and (d != 0).mean() <= 1e-4
        if fmt & NOEXP:
            # k = 1: s = amax / fpmax and every code exactly as the oracle's
            assert np.array_equal(S.cpu().numpy(), s) and np.all(K.cpu().numpy() == 1.0)
            assert np.array_equal(Q.cpu().numpy(), q)


@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("G", [32, 128, 256, 1024])
def test_dequantize_parity(coat, fmt, G):
    # whole tiles (the table path for groups of 128 and more) and a ragged last tile
    n = 1024 * 50 + 77
    x = page_like(n, G, "m", seed=5)
    q, s, k = oracle.quantize(x.astype(np.float64), G, fmt)
    log(f"test_dequantize_parity fmt={fmt} G={G}")
    X = torch.empty(n, dtype=torch.float32, device="cuda")
    coat.dequantize(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda(), torch.from_numpy(k).cuda(),
                    X, group=G, fmt=fmt)
    got = X.cpu().numpy().astype(np.float64)
    want = oracle.dequantize(q, s, k, G, fmt)
    # fp32 output of an fp64 value: one rounding, so within one fp32 ulp of the oracle
    assert np.all(np.abs(got - want) <= np.spacing(np.abs(want).astype(np.float32)).astype(np.float64))


@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("G", [128, 1024])
def test_dequantize_every_code_and_special_groups(coat, fmt, G):
    """Every code under stored states of the kinds the quantizer and the step
    produce: expanded (k > 1), k = 1, k < 1, an all-zero group (s = 0 with
    signed-zero and NaN codes) and a poisoned group (s = NaN, every code NaN).
    NaN results must match in place."""
    rng = np.random.default_rng(9)
    ng = 40
    n = ng * G + 300  # whole tiles and a ragged last tile
    q = rng.integers(0, 256, n, dtype=np.uint8)
    q[:256] = np.arange(256, dtype=np.uint8)
    ngr = (n + G - 1) // G
    s = 10.0 ** rng.uniform(-40.0, -5.0, ngr)
    k = rng.uniform(0.7, 10.0, ngr).astype(np.float32)
    k[1::5] = 1.0
    s[2] = 0.0
    q[2 * G:3 * G] = rng.choice(np.array([0x00, 0x80, 0x7F, 0xFF], dtype=np.uint8), G)
    s[3] = np.nan
    k[3] = 1.0
    q[3 * G:4 * G] = 0x7F
    log(f"test_dequantize_every_code_and_special_groups fmt={fmt} G={G}")
    X = torch.empty(n, dtype=torch.float32, device="cuda")
    coat.dequantize(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda(), torch.from_numpy(k).cuda(),
                    X, group=G, fmt=fmt)
    got = X.cpu().numpy().astype(np.float64)
    want = oracle.dequantize(q, s, k, G, fmt)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    fin = ~np.isnan(want)
    want32 = want[fin].astype(np.float32).astype(np.float64)
    ok = (got[fin] == want32) | (np.abs(got[fin] - want[fin]) <= np.spacing(np.abs(want[fin]).astype(np.float32)))
    assert ok.all(), np.flatnonzero(~ok)[:10]
    assert np.array_equal(np.signbit(got[fin]), np.signbit(want[fin]))
    # k = 1: the plain product |q| s, rounded once to fp32, exactly as the oracle's
    k1 = np.repeat(k == 1.0, G)[:n] & fin
    assert np.array_equal(got[k1], want[k1].astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("fmt", [E4, E5])
def test_quantize_degenerate_groups(coat, fmt):
    G = 32
    groups = [
        np.zeros(G),                                      # all zero
        np.r_[np.zeros(G - 1), -3e-4],                    # one nonzero
        1e-3 * (1 + np.linspace(0, 0.9e-6, G)),           # near-constant
        np.r_[1.0, 1e-30, np.full(G - 2, 1e-3)],          # wider than the FP8 range: k < 1
        1e-35 * (1 + np.linspace(0, 1, G)),               # tiny narrow group: range guard
        np.r_[np.full(G - 1, 1e-3), np.nan],              # poisoned
        np.r_[np.full(G - 1, 1e-3), np.inf],
        np.r_[np.full(G // 2, 0.0), 10.0 ** -np.arange(G // 2)],
    ]
    x = np.concatenate(groups).astype(np.float32)
    x[3] = -0.0
    n = x.size
    log(f"test_quantize_degenerate_groups fmt={fmt}")
    X = torch.from_numpy(x).cuda()
    Q = torch.empty(n, dtype=torch.uint8, device="cuda")
    S = torch.empty(n // G, dtype=torch.float64, device="cuda")
    K = torch.empty(n // G, dtype=torch.float32, device="cuda")
    coat.quantize(X, Q, S, K, group=G, fmt=fmt)
    q, s, k = oracle.quantize(x.astype(np.float64), G, fmt)
    assert rel_err(K.cpu().numpy(), k).max() <= 1e-5, (K.cpu().numpy(), k)
    assert rel_err(S.cpu().numpy(), s).max() <= 1e-5, (S.cpu().numpy(), s)
    assert np.array_equal(Q.cpu().numpy(), q)


@pytest.mark.parametrize("G", [32, 128])
def test_quantize_near_constant_threshold(coat, G):
    """Groups at the near-constant threshold: an amax / amin of exactly
    1 + 1e-6 in real arithmetic (9000009 / 9000000, 10000010 / 10000000 and
    11000011 / 11000000, scaled) rounds to the fp64 constant 1 + 1e-6, so k = 1;
    one fp32 step more in amax is above it and expands. fp32 inputs reach the
    threshold quotient only exactly; the fp64-ulp neighbours of it are covered
    by the step's threshold test."""
    groups, expect_k1 = [], []
    for b_int, d in ((9000000, 9), (10000000, 10), (11000000, 11)):
        for extra, scale in ((0, 2.0 ** -24), (1, 2.0 ** -24), (0, 2.0 ** -40)):
            a = np.float32((b_int + d + extra) * scale)
            b = np.float32(b_int * scale)
            grp = np.full(G, b, np.float32)
            grp[G // 3] = a
            groups.append(grp)
            expect_k1.append(extra == 0)
    x = np.concatenate(groups)
    n = x.size
    log(f"test_quantize_near_constant_threshold G={G}")
    X = torch.from_numpy(x).cuda()
    Q = torch.empty(n, dtype=torch.uint8, device="cuda")
    S = torch.empty(n // G, dtype=torch.float64, device="cuda")
    K = torch.empty(n // G, dtype=torch.float32, device="cuda")
    coat.quantize(X, Q, S, K, group=G, fmt=E4)
    q, s, k = oracle.quantize(x.astype(np.float64), G, E4)
    assert np.array_equal(k == 1.0, np.array(expect_k1)), k
    assert np.array_equal(K.cpu().numpy(), k)
    assert rel_err(S.cpu().numpy(), s).max() <= 1e-5
    d = code_steps(Q.cpu().numpy(), q)
    assert d.max() <= 1 and (d != 0).mean() <= 1e-4


def test_codec_beyond_2_32_elements(coat):
    """Quantize and dequantize one buffer of 2^32 + 3149 moment values (a short
    last group): groups around elements 2^31 and 2^32, the first and the last
    groups and a stride through the buffer, against the oracle."""
    import synth
    G, fmt = 128, E4
    n = (1 << 32) + 3 * 1024 + 77
    ng = (n + G - 1) // G
    chunk = 1 << 28  # whole groups; fp64 temporaries per chunk
    X = torch.empty(n, dtype=torch.float32, device="cuda")
    for c0 in range(0, n, chunk):
        cn = min(chunk, n - c0)
        m, _ = synth.prior_moments(cn, G, 31, c0 // chunk, device="cuda")
        X[c0:c0 + cn] = m
        del m
    Q = torch.empty(n, dtype=torch.uint8, device="cuda")
    S = torch.empty(ng, dtype=torch.float64, device="cuda")
    K = torch.empty(ng, dtype=torch.float32, device="cuda")
    log(f"test_codec_beyond_2_32_elements n={n}")
    coat.quantize(X, Q, S, K, group=G, fmt=fmt)
    back = torch.empty(n, dtype=torch.float32, device="cuda")
    coat.dequantize(Q, S, K, back, group=G, fmt=fmt)
    torch.cuda.synchronize()
    picks = set([0, 1, ng - 1, ng - 2])
    for c in ((1 << 31) // G, (1 << 32) // G):
        picks.update(range(c - 3, c + 3))
    picks.update(range(5, ng, 99991))
    kd, sd, steps, deq = [], [], [], []
    for gi in sorted(picks):
        a, b = gi * G, min(n, gi * G + G)
        x = X[a:b].cpu().numpy().astype(np.float64)
        q, s, k = oracle.quantize(x, G, fmt)
        kd.append(rel_err(K[gi:gi + 1].cpu().numpy(), k).max())
        sd.append(rel_err(S[gi:gi + 1].cpu().numpy(), s).max())
        qg = Q[a:b].cpu().numpy()
        steps.append(code_steps(qg, q))
        want = oracle.dequantize(qg, S[gi:gi + 1].cpu().numpy(), K[gi:gi + 1].cpu().numpy(), G, fmt)
        got = back[a:b].cpu().numpy().astype(np.float64)
        deq.append(np.all(np.abs(got - want) <= np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)))
    d = np.concatenate(steps)
    log(f"  {len(picks)} groups: k rel max {max(kd):.3g}, s rel max {max(sd):.3g}, codes differing {int((d != 0).sum())}")
    assert max(kd) <= 1e-5 and max(sd) <= 1e-5
    assert d.max() <= 1 and (d != 0).mean() <= 1e-4
    assert all(deq)
