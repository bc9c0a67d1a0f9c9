"""The oracle's activation codec (absmax FP8 scaling per tensor or per group of
G consecutive bf16 values), pinned against torch's own float8 casts, which
are an independent implementation of the same rounding, and against closed
forms.

Article, section "Solution: mixed-granularity FP8 precision flow": layer
inputs are kept in FP8 for the backward pass with a granularity that differs
between layers. The formula is the reading taken here: s = RN32(amax / fpmax),
code = encode(RN32(x / s)), value = RN_bf16(RN32(decode(code) * s)).
"""
import numpy as np
import pytest
import torch

import oracle

E4, E5 = 0, 1
TDT = {E4: torch.float8_e4m3fn, E5: torch.float8_e5m2}
FPMAX = {E4: 448.0, E5: 57344.0}


def act_like(n, seed):
    """bf16 activations: normal values, per-channel scales over four decades
    (512 channels), and one outlier in a thousand 50x larger."""
    rng = np.random.default_rng(seed)
    ch = 10.0 ** rng.uniform(-3, 1, 512)
    x = rng.standard_normal(n) * np.resize(ch, n)
    x[rng.random(n) < 1e-3] *= 50.0
    return torch.from_numpy(x).to(torch.bfloat16)


def bits(xb):
    return xb.view(torch.int16).numpy().view(np.uint16)


def torch_reference(xb, G, fmt):
    """Codes, scales and dequantized bf16 values computed with torch fp32 ops
    and torch's float8/bf16 casts."""
    x = xb.float()
    n = x.numel()
    L = n if G == 0 else G
    pad = (-n) % L if n else 0
    xp = torch.nn.functional.pad(x, (0, pad)).view(-1, L) if n else x.view(0, 1)
    amax = xp.abs().amax(dim=1)
    s = amax / torch.tensor(FPMAX[fmt], dtype=torch.float32)
    se = s.repeat_interleave(L)[:n]
    y = x / se
    q = y.to(TDT[fmt]).view(torch.uint8).clone()
    zero = se == 0
    q[zero] = torch.where(torch.signbit(x[zero]), 0x80, 0x00).to(torch.uint8)
    back = (q.view(TDT[fmt]).float() * se).to(torch.bfloat16)
    return q.numpy(), s.numpy(), bits(back)


@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("G,n", [(0, 100003), (16, 4096), (32, 100003), (128, 65536 + 77), (1024, 50000), (7, 99)])
def test_matches_torch_casts(fmt, G, n):
    xb = act_like(n, seed=G + 3 * fmt)
    q, s = oracle.act_quantize(bits(xb), G, fmt)
    tq, ts, tback = torch_reference(xb, G, fmt)
    assert np.array_equal(s, ts)
    assert np.array_equal(q, tq)
    back = oracle.act_dequantize(q, s, G, fmt)
    assert np.array_equal(back, tback)


@pytest.mark.parametrize("fmt", [E4, E5])
def test_closed_forms(fmt):
    G = 32
    x = act_like(6 * G, seed=5).float()
    x[0:G] = 0.0                      # all-zero group
    x[G + 3] = -0.0
    x[G:2 * G] = 0.0
    x[G + 5] = -0.0                   # zero group with a negative zero
    x[2 * G + 7] = float("nan")       # poisoned group (NaN)
    x[3 * G + 1] = float("inf")       # poisoned group (Inf)
    x[4 * G:5 * G] = torch.linspace(-3, 2, G)
    xb = x.to(torch.bfloat16)
    q, s = oracle.act_quantize(bits(xb), G, fmt)
    assert s[0] == 0 and s[1] == 0
    assert np.all(q[:G] == 0) and q[G + 5] == 0x80 and np.sum(q[G:2 * G] == 0x80) == 1
    assert np.isnan(s[2]) and np.all(q[2 * G:3 * G] == 0x7F)
    assert np.isnan(s[3]) and np.all(q[3 * G:4 * G] == 0x7F)
    # the largest magnitude (-3 here) takes the largest finite code
    top = 0x7E if fmt == E4 else 0x7B
    assert q[4 * G] == 0x80 | top
    assert s[4] == np.float32(np.float32(3.0) / np.float32(FPMAX[fmt]))
    # codes are monotone in x within a group
    vals = oracle.fp8_decode(q[4 * G:5 * G], fmt)
    assert np.all(np.diff(vals) >= 0)
    back = oracle.act_dequantize(q, s, G, fmt)
    fb = torch.from_numpy(back.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.all(fb[:2 * G] == 0) and np.signbit(fb[G + 5])
    assert np.all(np.isnan(fb[2 * G:4 * G]))
    # round trip of the group: within half an FP8 step of the value
    rel = np.abs(fb[4 * G:5 * G] - x[4 * G:5 * G].numpy()) / 3.0
    assert rel.max() <= (2.0 ** -4 if fmt == E4 else 2.0 ** -3)


def test_per_tensor_equals_one_group():
    xb = act_like(4096, seed=9)
    for fmt in (E4, E5):
        q0, s0 = oracle.act_quantize(bits(xb), 0, fmt)
        q1, s1 = oracle.act_quantize(bits(xb), 4096, fmt)
        assert np.array_equal(q0, q1) and np.array_equal(s0, s1)


def test_tiny_values():
    # bf16 subnormals: the scale is an fp32 subnormal; codes saturate rather than overflow
    x = torch.tensor([2.0 ** -133, -(2.0 ** -130), 2.0 ** -128, 0.0] * 8).to(torch.bfloat16)
    for fmt in (E4, E5):
        q, s = oracle.act_quantize(bits(x), 0, fmt)
        tq, ts, tback = torch_reference(x, 0, fmt)
        assert np.array_equal(q, tq) and np.array_equal(s, ts)
        assert np.array_equal(oracle.act_dequantize(q, s, 0, fmt), tback)
