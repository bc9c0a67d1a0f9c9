"""GPU parity of the FP8 activation codec (per tensor and per group) against
the oracle, through the C ABI: codes, scales and dequantized bf16 values
bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _parity import log

pytestmark = pytest.mark.gpu
E4, E5 = 0, 1


@pytest.fixture(scope="module")
def coat():
    import fp8_optimizer_state_amd as c
    assert torch.cuda.is_available()
    c.lib()
    return c


def bits(xb):
    return xb.cpu().view(torch.int16).numpy().view(np.uint16)


def gpu_codec(coat, xb, G, fmt):
    x = xb.cuda()
    n = x.numel()
    q = torch.empty(n, dtype=torch.uint8, device="cuda")
    s = torch.empty(coat.act_nscales(n, G), dtype=torch.float32, device="cuda")
    coat.act_quantize(x, q, s, group=G, fmt=fmt)
    back = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    coat.act_dequantize(q, s, back, group=G, fmt=fmt)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy(), bits(back)


def same_f32(a, b):
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])


def same_bf16(a, b):
    na = (a & 0x7FFF) > 0x7F80
    nb = (b & 0x7FFF) > 0x7F80
    return np.array_equal(na, nb) and np.array_equal(a[~na], b[~nb])


def check(coat, xb, G, fmt, tag):
    q, s, back = gpu_codec(coat, xb, G, fmt)
    oq, os_ = oracle.act_quantize(bits(xb), G, fmt)
    oback = oracle.act_dequantize(oq, os_, G, fmt)
    diff = int(np.sum(q != oq))
    log(f"[act {tag} G={G} fmt={fmt} n={xb.numel()}] code mismatches {diff}")
    assert diff == 0
    assert same_f32(s, os_)
    assert same_bf16(back, oback)


@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("G", [0, 16, 32, 128, 1024])
@pytest.mark.parametrize("tokens,channels", [(8, 5120), (37, 2731), (1, 17), (3, 1029)])
def test_codec_matches_oracle(coat, fmt, G, tokens, channels):
    xb = synth.activations(tokens, channels, seed=1 + fmt)
    check(coat, xb, G, fmt, "random")


@pytest.mark.parametrize("fmt", [E4, E5])
def test_edge_groups(coat, fmt):
    G = 32
    x = synth.activations(1, 12 * G, seed=3).float()
    x[0:G] = 0.0
    x[G:2 * G] = 0.0
    x[G + 5] = -0.0
    x[2 * G + 7] = float("nan")
    x[3 * G + 1] = float("inf")
    x[4 * G + 2] = float("-inf")
    x[5 * G:6 * G] = 2.0 ** -133                   # bf16 subnormals: the scale is an fp32 subnormal
    x[5 * G + 1] = -(2.0 ** -130)
    fpmax = 448.0 if fmt == E4 else 57344.0
    # s = 1 exactly, and every other value an FP8 rounding midpoint or its bf16 neighbours
    grid = oracle.fp8_decode(np.arange(0x7F if fmt == E4 else 0x7C, dtype=np.uint8), fmt)
    mids = 0.5 * (grid[:-1] + grid[1:])
    row = torch.tensor(mids[-(G - 1):], dtype=torch.float32)
    x[6 * G] = fpmax
    x[6 * G + 1:7 * G] = row
    x[7 * G] = -fpmax
    x[7 * G + 1:8 * G] = -torch.tensor(mids[1:G], dtype=torch.float32)
    xb = x.to(torch.bfloat16)
    for G_ in (G, 0):
        check(coat, xb, G_, fmt, "edges")


@pytest.mark.parametrize("fmt", [E4, E5])
def test_every_bf16_value_per_tensor(coat, fmt):
    """Every finite bf16 value up to the tensor's maximum, coded with one scale:
    for a maximum of fpmax * 2^k the scale is 2^k exactly, so the quotients are
    the bf16 values themselves scaled, every FP8 rounding midpoint of the grid
    among them (ties), subnormal codes included; other maxima give scales
    with full 24-bit significands. Codes, scale and bf16 values equal the
    oracle's bit for bit."""
    fpmax = 448.0 if fmt == E4 else 57344.0
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    fin = (allb & 0x7F80) != 0x7F80
    f32 = (allb.astype(np.uint32) << 16).view(np.float32)
    rng = np.random.default_rng(11 + fmt)
    amaxes = [fpmax * 2.0 ** k for k in (-120, -40, -8, 0, 9, 60, 110)]
    amaxes += [float(np.float32(v)) for v in rng.uniform(1e-3, 1e3, 4)]
    for amax in amaxes:
        am = torch.tensor([amax], dtype=torch.float32).to(torch.bfloat16)
        amf = float(am.float())
        keep = fin & (np.abs(f32) <= amf)
        xs = np.concatenate([allb[keep], bits(am), bits(-am)])
        xb = torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16)
        check(coat, xb, 0, fmt, f"all-bf16 amax={amf:.4g}")


@pytest.mark.parametrize("fmt", [E4, E5])
def test_decode_every_code(coat, fmt):
    q = torch.arange(256, dtype=torch.uint8, device="cuda").repeat(4)
    s = torch.ones(1, dtype=torch.float32, device="cuda")
    out = torch.empty(q.numel(), dtype=torch.bfloat16, device="cuda")
    coat.act_dequantize(q, s, out, group=0, fmt=fmt)
    want = oracle.act_dequantize(q.cpu().numpy(), s.cpu().numpy(), 0, fmt)
    assert same_bf16(bits(out), want)


def test_per_tensor_many_waves(coat):
    # the largest magnitude in the very last element: the cross-wave maximum must see it
    xb = synth.activations(512, 5120, seed=7).float()
    xb[-1] = -1e4
    xb = xb.to(torch.bfloat16)
    for fmt in (E4, E5):
        check(coat, xb, 0, fmt, "waves")


@pytest.mark.parametrize("G", [0, 128])
def test_full_size_llama13b_mlp(coat, G):
    """16384 tokens x 13824 channels (the down projection's input in Llama-2-13B),
    the launch the benchmark times; per group: sampled groups against the oracle,
    per tensor: the whole tensor."""
    fmt = E4
    tokens, channels = 16384, 13824
    x = synth.activations(tokens, channels, seed=13, device="cuda")
    n = x.numel()
    q = torch.empty(n, dtype=torch.uint8, device="cuda")
    s = torch.empty(coat.act_nscales(n, G), dtype=torch.float32, device="cuda")
    coat.act_quantize(x, q, s, group=G, fmt=fmt)
    back = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    coat.act_dequantize(q, s, back, group=G, fmt=fmt)
    torch.cuda.synchronize()
    if G == 0:
        xs = bits(x)
        oq, os_ = oracle.act_quantize(xs, 0, fmt)
        assert same_f32(s.cpu().numpy(), os_)
        assert int(np.sum(q.cpu().numpy() != oq)) == 0
        assert same_bf16(bits(back), oracle.act_dequantize(oq, os_, 0, fmt))
        log(f"[act full per-tensor] n={n} s={float(os_[0]):.6g}")
        return
    ng = n // G
    rng = np.random.default_rng(5)
    groups = np.unique(np.concatenate([[0, ng - 1], rng.integers(0, ng, 20000)]))
    idx = (groups[:, None] * G + np.arange(G)[None, :]).ravel()
    it = torch.from_numpy(idx).cuda()
    xs = bits(x[it])
    oq, os_ = oracle.act_quantize(xs, G, fmt)
    assert same_f32(s[torch.from_numpy(groups).cuda()].cpu().numpy(), os_)
    assert int(np.sum(q[it].cpu().numpy() != oq)) == 0
    assert same_bf16(bits(back[it]), oracle.act_dequantize(oq, os_, G, fmt))
    log(f"[act full per-group] n={n} sampled groups {groups.size}")


@pytest.mark.parametrize("G", [0, 128])
def test_act_beyond_2_32_elements(coat, G):
    """Activation codec on 2^32 + 2148 bf16 values (a short last group): groups
    around elements 2^31 and 2^32, the first and last groups and a stride
    through the buffer, codes, scales and bf16 values against the oracle. Per
    tensor, the largest magnitude sits past 2^32 and the sample holds it, so
    the oracle's scale over the sample is the tensor's."""
    fmt = E4
    n = (1 << 32) + 2 * 1024 + 100
    chunk = 1 << 28
    x = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    gen = torch.Generator(device="cuda")
    for c0 in range(0, n, chunk):
        cn = min(chunk, n - c0)
        gen.manual_seed(7001 + c0 // chunk)
        x[c0:c0 + cn] = torch.randn(cn, device="cuda", generator=gen).mul_(0.5)
    top = (1 << 32) + 5
    x[top] = -1e4  # larger in magnitude than any other value
    q = torch.empty(n, dtype=torch.uint8, device="cuda")
    s = torch.empty(coat.act_nscales(n, G), dtype=torch.float32, device="cuda")
    log(f"test_act_beyond_2_32_elements G={G} n={n}")
    coat.act_quantize(x, q, s, group=G, fmt=fmt)
    back = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    coat.act_dequantize(q, s, back, group=G, fmt=fmt)
    torch.cuda.synchronize()
    Gs = G or 128  # sampling unit
    nu = (n + Gs - 1) // Gs
    picks = set([0, 1, nu - 1, nu - 2, top // Gs])
    for c in ((1 << 31) // Gs, (1 << 32) // Gs):
        picks.update(range(c - 3, c + 3))
    picks.update(range(9, nu, 99991))
    spans = [(u * Gs, min(n, u * Gs + Gs)) for u in sorted(picks)]
    xs = np.concatenate([bits(x[a:b]) for a, b in spans])
    qs = np.concatenate([q[a:b].cpu().numpy() for a, b in spans])
    bs = np.concatenate([bits(back[a:b]) for a, b in spans])
    if G:
        # each sampled group on its own (the last one short)
        for (a, b), off in zip(spans, np.cumsum([0] + [b - a for a, b in spans[:-1]])):
            oq, os_ = oracle.act_quantize(xs[off:off + b - a], G, fmt)
            assert np.array_equal(qs[off:off + b - a], oq)
            assert same_f32(s[a // G:a // G + 1].cpu().numpy(), os_)
            assert same_bf16(bs[off:off + b - a], oracle.act_dequantize(oq, os_, G, fmt))
    else:
        oq, os_ = oracle.act_quantize(xs, 0, fmt)
        assert same_f32(s.cpu().numpy(), os_)
        assert np.array_equal(qs, oq)
        assert same_bf16(bs, oracle.act_dequantize(oq, os_, 0, fmt))
