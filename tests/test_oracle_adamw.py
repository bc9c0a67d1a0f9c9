"""Pins for the oracle's AdamW arithmetic and for the step as a whole (CPU).

The dense update is checked against torch.optim.AdamW (the textbook
decoupled-weight-decay form), and the full FP8-state step with expansion
switched off is checked against a composition of library routines: torch's
float8 view for decoding, torch.optim.AdamW, and torch's float8 cast for
plain per-group absmax requantization.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

E4, E5, NOEXP = oracle.FMT_E4M3, oracle.FMT_E5M2, oracle.FMT_NO_EXPAND
F32 = lambda x: float(np.float32(x))  # the ABI passes hyperparameters as fp32
H = {k: (F32(v) if k != "step" else v) for k, v in synth.HYPER.items()}
TORCH_T = {E4: torch.float8_e4m3fn, E5: torch.float8_e5m2}
FPMAX = {E4: 448.0, E5: 57344.0}


def torch_adamw(p, g, m, v, step, lr, b1, b2, eps, wd):
    """One torch.optim.AdamW step in fp64 from the given state (t = step)."""
    prm = torch.nn.Parameter(torch.from_numpy(p.astype(np.float64)))
    opt = torch.optim.AdamW([prm], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd,
                            foreach=False)
    prm.grad = torch.from_numpy(g.astype(np.float64))
    opt.state[prm] = {"step": torch.tensor(float(step - 1)),
                      "exp_avg": torch.from_numpy(m.copy()),
                      "exp_avg_sq": torch.from_numpy(v.copy())}
    opt.step()
    st = opt.state[prm]
    return prm.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def inputs(n, G, seed):
    p = synth.params(n, seed).numpy()
    g = synth.grads(n, seed)
    m, v = synth.prior_moments(n, G, seed)
    return p, g, m.numpy().astype(np.float64), v.numpy().astype(np.float64)


@pytest.mark.parametrize("step", [1, 10, 1000])
def test_dense_update_matches_torch_adamw(step):
    n = 4096
    p, g, m, v = inputs(n, 128, 11)
    gb = g.view(torch.int16).numpy().view(np.uint16)
    gd = g.to(torch.float64).numpy()
    h = dict(H, step=step)
    p1, w1, m1, v1 = oracle.adamw_dense(p, gb, m, v, h["lr"], h["b1"], h["b2"], h["eps"],
                                        h["wd"], step)
    tp, tm, tv = torch_adamw(p, gd, m, v, step, h["lr"], h["b1"], h["b2"], h["eps"], h["wd"])
    assert np.allclose(m1, tm, rtol=1e-12, atol=1e-300)
    assert np.allclose(v1, tv, rtol=1e-12, atol=1e-300)
    # fp32 master: the fp64 result rounded once; allow one fp32 ulp for torch's order
    assert np.all(np.abs(p1.astype(np.float64) - tp) <= np.spacing(np.float32(np.abs(tp))).astype(np.float64))
    # bf16 copy is the RNE of the stored fp32 master
    assert np.array_equal(w1, bf16_bits(torch.from_numpy(p1)))


def test_bf16_copy_rounding_and_nan():
    p = np.array([1.0, 1.00390625, 1.01171875, -2.0 ** -130, np.nan, np.inf], np.float32)
    g = np.zeros(p.size, np.uint16)
    z = np.zeros(p.size)
    p1, w, _, _ = oracle.adamw_dense(p, g, z, z, 0.0, 0.9, 0.95, 1e-8, 0.0, 1)
    ref = bf16_bits(torch.from_numpy(p1))
    fin = np.isfinite(p1)
    assert np.array_equal(w[fin], ref[fin])
    assert (w[4] & 0x7F80) == 0x7F80 and (w[4] & 0x7F) != 0  # a NaN stays NaN
    assert w[5] == 0x7F80


@pytest.mark.parametrize("fmt_m,fmt_v", [(E4, E4), (E4, E5)])
def test_step_without_expansion_is_library_composition(fmt_m, fmt_v):
    """k = 1 everywhere: decode (torch view) * s, torch AdamW, torch-cast absmax requant."""
    n, G = 128 * 64, 128
    p, g, m, v = inputs(n, G, 21)
    fm, fv = fmt_m | NOEXP, fmt_v | NOEXP
    mq, ms, mk = oracle.quantize(m, G, fm)
    vq, vs, vk = oracle.quantize(v, G, fv)
    gb = g.view(torch.int16).numpy().view(np.uint16)
    out = oracle.adamw_step(p, gb, mq, ms, mk, vq, vs, vk, G, fm, fv, H["lr"], H["b1"],
                            H["b2"], H["eps"], H["wd"], H["step"])

    def tdec(q, s, fmt):
        return torch.from_numpy(q).view(TORCH_T[fmt]).to(torch.float64).numpy() * np.repeat(s, G)

    tp, tm, tv = torch_adamw(p, g.to(torch.float64).numpy(), tdec(mq, ms, fmt_m),
                             tdec(vq, vs, fmt_v), H["step"], H["lr"], H["b1"], H["b2"],
                             H["eps"], H["wd"])
    assert np.all(np.abs(out["p"].astype(np.float64) - tp)
                  <= np.spacing(np.float32(np.abs(tp))).astype(np.float64))

    def tquant(x, fmt):
        xs = x.reshape(-1, G)
        amax = np.abs(xs).max(1, keepdims=True)
        q = torch.from_numpy(xs / (amax / FPMAX[fmt])).to(TORCH_T[fmt]).view(torch.uint8)
        return q.numpy().ravel(), amax[:, 0] / FPMAX[fmt]

    rq, rs = tquant(tm, fmt_m)
    assert np.allclose(out["ms"], rs, rtol=1e-12, atol=0)
    assert (out["mq"] != rq).mean() <= 1e-4
    rq, rs = tquant(tv, fmt_v)
    assert np.allclose(out["vs"], rs, rtol=1e-12, atol=0)
    assert (out["vq"] != rq).mean() <= 1e-4
    assert np.all(out["mk"] == 1) and np.all(out["vk"] == 1)


def test_step_groups_are_independent_and_threading_is_exact():
    n, G = 128 * 40 + 77, 128
    p, g, m, v = inputs(n, G, 5)
    mq, ms, mk = oracle.quantize(m, G, E4)
    vq, vs, vk = oracle.quantize(v, G, E5)
    gb = g.view(torch.int16).numpy().view(np.uint16)
    args = (H["lr"], H["b1"], H["b2"], H["eps"], H["wd"], H["step"])
    a = oracle.adamw_step(p, gb, mq, ms, mk, vq, vs, vk, G, E4, E5, *args)
    b = oracle.adamw_step(p, gb, mq, ms, mk, vq, vs, vk, G, E4, E5, *args, threads=4)
    for key in a:
        assert np.array_equal(a[key], b[key], equal_nan=True), key
    # the new state is the quantization of the updated moments: dequantizing it
    # and quantizing again reproduces it (self-consistent (q, s, k))
    md = oracle.dequantize(a["mq"], a["ms"], a["mk"], G, E4)
    q2, s2, k2 = oracle.quantize(md, G, E4)
    assert (q2 != a["mq"]).mean() <= 1e-3
    assert np.allclose(s2, a["ms"], rtol=1e-9) and np.allclose(k2, a["mk"], rtol=1e-6)


def test_nan_grad_poisons_one_group_and_its_params():
    n, G = 128 * 3, 128
    p, g, m, v = inputs(n, G, 6)
    gb = g.view(torch.int16).numpy().view(np.uint16).copy()
    gb[130] = 0x7FC0  # bf16 NaN in group 1
    mq, ms, mk = oracle.quantize(m, G, E4)
    vq, vs, vk = oracle.quantize(v, G, E4)
    args = (H["lr"], H["b1"], H["b2"], H["eps"], H["wd"], H["step"])
    out = oracle.adamw_step(p, gb, mq, ms, mk, vq, vs, vk, G, E4, E4, *args)
    assert np.isnan(out["p"][130]) and np.isfinite(np.delete(out["p"], 130)).all()
    assert np.isnan(out["ms"][1]) and np.isnan(out["vs"][1])
    assert np.all(out["mq"][G:2 * G] == 0x7F)
    assert np.isfinite(out["ms"][[0, 2]]).all()
    # next step: the poisoned group decodes to NaN and stays poisoned
    gb[130] = 0
    out2 = oracle.adamw_step(out["p"], gb, out["mq"], out["ms"], out["mk"], out["vq"], out["vs"],
                             out["vk"], G, E4, E4, *args)
    assert np.isnan(out2["p"][G:2 * G]).all() and np.isfinite(out2["p"][:G]).all()
