"""Ten consecutive steps on the full Llama-2-13B list with group 32 and E4M3
for both moments, fresh seeded grads every step (t = 10..19).

Checks, on a sample of groups (every tensor's first and last group and every
997th group):
  * parity at every step on the same inputs: the oracle takes the step from the
    GPU's own sampled state after the previous step (the oracle's own state
    at t = 10) and the same grads, and the GPU's result must match it at the
    full tolerance (the article recomputes k at every training step, section
    "Solution: dynamic range expansion", so every step is held to it);
  * the two chains run side by side, each carrying its own state: where a k
    lands within an fp32 rounding boundary of the oracle's, that group's later
    states legitimately differ ("parted" groups), so this is reported and only
    loosely bounded;
  * the drift of the dequantized moments against a dense AdamW (fp64 moments,
    no quantization) started from the same dequantized prior and fed the same
    grads, with expansion and with k forced to 1 (the ablation). The article
    reports that expansion lowers the quantization error of the states
    (section "Solution: dynamic range expansion"); here it must lower the
    drift.
"""
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import synth
from _parity import HYPER, TOL_P_ABS, TOL_P_REL, TOL_SK, bf16_bits, compare, log, rel_err
from test_gpu_full import build, concat, gather, oracle_quantize_sample, overwrite_sample, read_sample

pytestmark = pytest.mark.gpu
NOEXP = 0x100


@pytest.fixture(scope="module")
def coat():
    import fp8_optimizer_state_amd as c
    assert torch.cuda.is_available()
    c.lib()
    return c


def dequant_sample_gpu(coat, st, host, G, fmt):
    """Dequantized moments of the sampled groups, through the device kernel."""
    ms, vs = [], []
    for i, h in enumerate(host):
        t = st.tensor(i)
        idx = h["idx"]
        for q, s, k, f, out in ((t.m_q, t.m_s, t.m_k, fmt, ms), (t.v_q, t.v_s, t.v_k, fmt, vs)):
            qq = q.view(-1, G)[idx].reshape(-1).contiguous()
            x = torch.empty(qq.numel(), dtype=torch.float32, device=q.device)
            coat.dequantize(qq, s[idx].contiguous(), k[idx].contiguous(), x, group=G, fmt=f)
            out.append(x.cpu().numpy().astype(np.float64))
    return np.concatenate(ms), np.concatenate(vs)


def groupwise(a, b, G):
    a, b = a.reshape(-1, G), b.reshape(-1, G)
    nb = np.linalg.norm(b, axis=1)
    keep = nb > 0
    r = np.linalg.norm(a - b, axis=1)[keep] / nb[keep]
    return float(np.linalg.norm(a - b) / np.linalg.norm(b)), float(np.mean(r)), float(np.percentile(r, 99))


def mark_parted(got, ref, G, parted):
    """Mark the groups whose stored state differs from the oracle's (any code,
    or s or k beyond the tolerance); from then on the two chains carry
    different states there."""
    for st in ("m", "v"):
        bad = (rel_err(got[f"{st}s"], ref[f"{st}s"]) > TOL_SK) | (rel_err(got[f"{st}k"], ref[f"{st}k"]) > TOL_SK)
        parted |= bad | (got[f"{st}q"] != ref[f"{st}q"]).reshape(-1, G).any(axis=1)


def chain_compare(got, ref, G, label, parted):
    """Later steps of a chain: the fraction of groups whose s, k or codes are
    off is bounded; those groups are marked in `parted` (kept across steps).
    Master weights must be within the full tolerance outside parted groups (in
    a parted group a moment one code step apart moves p by lr times a few
    percent of the update, beyond the master-weight tolerance)."""
    met = {}
    for st in ("m", "v"):
        bad = (rel_err(got[f"{st}s"], ref[f"{st}s"]) > TOL_SK) | (rel_err(got[f"{st}k"], ref[f"{st}k"]) > TOL_SK)
        codes = (got[f"{st}q"] != ref[f"{st}q"]).reshape(-1, G)
        met[f"{st}_sk_bad_frac"] = float(bad.mean())
        met[f"{st}_code_frac"] = float(codes.mean())
        met[f"{st}_code_group_frac"] = float(codes.any(axis=1).mean())
    mark_parted(got, ref, G, parted)
    pg, pr = got["p"].astype(np.float64), ref["p"].astype(np.float64)
    p_bad = (np.abs(pg - pr) > np.maximum(TOL_P_REL * np.abs(pr), TOL_P_ABS)).reshape(-1, G)
    met["parted_groups"] = int(parted.sum())
    met["p_bad"] = int(p_bad.sum())
    met["p_bad_outside_parted"] = int(p_bad[~parted].sum())
    log(f"[chain {label}] " + " ".join(f"{k}={v:.3g}" if isinstance(v, float) else f"{k}={v}"
                                       for k, v in met.items()))
    assert parted.mean() <= 1e-3, (label, met)
    assert met["p_bad_outside_parted"] == 0, (label, met)
    return met


def oracle_map(fn, items, threads=16):
    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(fn, items))


def run(coat, wl, fmt, sample):
    dev = torch.device("cuda")
    G = wl.group
    wl2 = synth.Workload(wl.name, wl.shapes, G, fmt, fmt, wl.seed, wl.steps)
    st, host = build(coat, wl2, dev, sample)
    oracle_quantize_sample(host, wl2)
    overwrite_sample(st, host, G)
    h = HYPER
    # dense reference starts from the oracle's dequantized prior
    dense = [dict(p=x["p"].copy(), m=oracle.dequantize(x["mq"], x["ms"], x["mk"], G, fmt & 0xFF),
                  v=oracle.dequantize(x["vq"], x["vs"], x["vk"], G, fmt & 0xFF)) for x in host]
    keys = ("p", "mq", "ms", "mk", "vq", "vs", "vk")
    ora = [{k: x[k] for k in keys} for x in host]    # the oracle's own chain
    prev = [{k: x[k] for k in keys} for x in host]   # the GPU's state before the step
    times, same_input = [], []
    parted = np.zeros(sum(len(x["idx"]) for x in host), dtype=bool)
    for j, step in enumerate(range(10, 10 + wl.steps)):
        # fresh grads for this step, on the device and for the sample on the host
        for i, n in enumerate(wl.sizes):
            t = st.tensor(i)
            synth.grads(n, wl.seed, i, device=dev, out=t.grads, step_index=1 + j)
            host[i]["g"] = bf16_bits(t.grads.view(-1, G)[host[i]["idx"]].reshape(-1).cpu())
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        st.step(fmt_m=fmt, fmt_v=fmt, lr=h["lr"], beta1=h["b1"], beta2=h["b2"], eps=h["eps"],
                weight_decay=h["wd"], step=step)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))

        def oracle_from(state):
            def one(ix):
                x, o = ix
                return oracle.adamw_step(o["p"], x["g"], o["mq"], o["ms"], o["mk"], o["vq"], o["vs"], o["vk"],
                                         G, fmt, fmt, h["lr"], h["b1"], h["b2"], h["eps"], h["wd"], step)
            return oracle_map(one, list(zip(host, state)))

        fed = oracle_from(prev)   # same inputs as the GPU's step
        ora = oracle_from(ora)    # the oracle's own chain
        for x, d in zip(host, dense):
            d["p"], _, d["m"], d["v"] = oracle.adamw_dense(d["p"], x["g"], d["m"], d["v"], h["lr"], h["b1"],
                                                          h["b2"], h["eps"], h["wd"], step)
        got = read_sample(st, host, G)
        label = f"{'noexp' if fmt & NOEXP else 'exp'} t={step}"
        met = compare(concat(got), concat(fed), label + " same inputs")
        same_input.append(met)
        if j == 0:
            mark_parted(concat(got), concat(ora), G, parted)
        else:
            chain_compare(concat(got), concat(ora), G, label + " chains", parted)
        prev = [{k: d[k] for k in keys} for d in got]
        log(f"  step {step}: {times[-1]:.2f} ms ({wl.n_params / (times[-1] * 1e-3):.3e} params/s)")
    md, vd = dequant_sample_gpu(coat, st, host, G, fmt & 0xFF)
    mref = np.concatenate([d["m"] for d in dense])
    vref = np.concatenate([d["v"] for d in dense])
    del st
    torch.cuda.empty_cache()
    return dict(times=times, m=groupwise(md, mref, G), v=groupwise(vd, vref, G), same_input=same_input,
                parted=int(parted.sum()), groups=int(parted.size))


def test_ten_steps_drift_and_ablation(coat):
    wl = synth.WORKLOADS["llama13b_g32"]
    sample = synth.parity_sample(wl, layer0=False)
    log(f"test_ten_steps: {wl.n_params} params, G={wl.group}, sample "
        f"{sum(len(ix) for _, ix in sample) * wl.group} params")
    t0 = time.time()
    exp = run(coat, wl, 0, sample)
    log(f"  expansion: drift m (global, mean, p99) {exp['m']}, v {exp['v']}, parted chains "
        f"{exp['parted']} of {exp['groups']} groups ({time.time() - t0:.0f} s)")
    noexp = run(coat, wl, NOEXP, sample)
    log(f"  k = 1:     drift m (global, mean, p99) {noexp['m']}, v {noexp['v']}, parted chains "
        f"{noexp['parted']} of {noexp['groups']} groups ({time.time() - t0:.0f} s)")
    for name, r in (("expansion", exp), ("k = 1", noexp)):
        worst = {k: max(m[k] for m in r["same_input"]) for k in ("m_s_rel", "v_s_rel", "m_k_rel", "v_k_rel",
                                                                 "m_code_frac", "v_code_frac")}
        log(f"  {name}: same-input parity over t = 10..19, worst {worst}")
    log(f"  median ms/step {np.median(exp['times']):.2f} (expansion), {np.median(noexp['times']):.2f} (k = 1)")
    # with k = 1 the kernels follow the definition's arithmetic exactly: from
    # the GPU's own state the step equals the oracle's in every scale and code,
    # so the two chains never part
    worst1 = {k: max(m[k] for m in noexp["same_input"]) for k in ("m_s_rel", "v_s_rel", "m_code_frac", "v_code_frac")}
    assert all(v == 0.0 for v in worst1.values()), worst1
    assert noexp["parted"] == 0
    # expansion keeps the states closer to unquantized AdamW
    assert exp["m"][0] < noexp["m"][0] and exp["v"][0] < noexp["v"][0]
    assert exp["m"][1] < noexp["m"][1] and exp["v"][1] < noexp["v"][1]
    # and the drift after ten steps stays small
    assert exp["m"][0] < 0.05 and exp["v"][0] < 0.05
