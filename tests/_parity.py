"""Shared helpers of the GPU parity tests: seeded inputs, oracle runs, tolerances.

Tolerances: per-group s and k within 1e-5 relative;
fp32 master weights within 1e-5 relative or 1e-8 absolute; FP8 codes identical
except for at most one code step on at most 1e-4 of the elements.
"""
from __future__ import annotations

import sys
from dataclasses import dataclass

import numpy as np
import torch

import oracle
import synth

F32 = lambda x: float(np.float32(x))
HYPER = dict(lr=F32(1e-4), b1=F32(0.9), b2=F32(0.95), eps=F32(1e-8), wd=F32(0.1), step=10)

TOL_SK = 1e-5
TOL_P_REL, TOL_P_ABS = 1e-5, 1e-8
TOL_CODE_FRAC = 1e-4


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@dataclass
class StepInputs:
    p: np.ndarray
    g: np.ndarray  # uint16 bf16 bits
    mq: np.ndarray
    ms: np.ndarray
    mk: np.ndarray
    vq: np.ndarray
    vs: np.ndarray
    vk: np.ndarray
    G: int
    fmt_m: int
    fmt_v: int

    @property
    def n(self):
        return self.p.size


def make_inputs(n: int, G: int, fmt_m: int, fmt_v: int, seed: int, tensor: int = 0,
                threads: int = 8) -> StepInputs:
    """Seeded p, g and prior moments, the prior quantized by the oracle."""
    p = synth.params(n, seed, tensor).numpy()
    g = bf16_bits(synth.grads(n, seed, tensor))
    m, v = synth.prior_moments(n, G, seed, tensor)
    mq, ms, mk = oracle.quantize_threaded(m.numpy(), G, fmt_m, threads)
    vq, vs, vk = oracle.quantize_threaded(v.numpy(), G, fmt_v, threads)
    return StepInputs(p, g, mq, ms, mk, vq, vs, vk, G, fmt_m, fmt_v)


def oracle_step(x: StepInputs, threads: int = 8, **hyper):
    h = dict(HYPER, **hyper)
    return oracle.adamw_step(x.p, x.g, x.mq, x.ms, x.mk, x.vq, x.vs, x.vk, x.G, x.fmt_m, x.fmt_v,
                             h["lr"], h["b1"], h["b2"], h["eps"], h["wd"], h["step"], threads=threads)


def to_dev(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def gpu_step(x: StepInputs, dev="cuda", want_bf16: bool = True, **hyper):
    import fp8_optimizer_state_amd as coat
    h = dict(HYPER, **hyper)
    n = x.n
    P = to_dev(x.p, dev)
    W = torch.empty(n, dtype=torch.bfloat16, device=dev) if want_bf16 else None
    Gd = to_dev(x.g.view(np.int16), dev).view(torch.bfloat16)
    MQ, MS, MK = to_dev(x.mq, dev), to_dev(x.ms, dev), to_dev(x.mk, dev)
    VQ, VS, VK = to_dev(x.vq, dev), to_dev(x.vs, dev), to_dev(x.vk, dev)
    coat.adamw_step(P, W, Gd, MQ, MS, MK, VQ, VS, VK, group=x.G, fmt_m=x.fmt_m, fmt_v=x.fmt_v,
                    lr=h["lr"], beta1=h["b1"], beta2=h["b2"], eps=h["eps"],
                    weight_decay=h["wd"], step=h["step"])
    torch.cuda.synchronize()
    out = dict(p=P.cpu().numpy(), mq=MQ.cpu().numpy(), ms=MS.cpu().numpy(), mk=MK.cpu().numpy(),
               vq=VQ.cpu().numpy(), vs=VS.cpu().numpy(), vk=VK.cpu().numpy())
    out["w"] = bf16_bits(W.cpu()) if want_bf16 else None
    return out


def code_steps(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in code steps between two FP8 code arrays, on the line of
    signed magnitudes; codes that differ only in the sign of zero (0x00 against
    0x80) count as one step, so a signed-zero mismatch is never invisible."""
    a = np.asarray(a, np.uint8)
    b = np.asarray(b, np.uint8)
    sa = np.where(a & 0x80, -1, 1) * (a & 0x7F).astype(np.int32)
    sb = np.where(b & 0x80, -1, 1) * (b & 0x7F).astype(np.int32)
    d = np.abs(sa - sb)
    return np.where((d == 0) & (a != b), 1, d)


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    same = (a == b) | both_nan
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.abs(a - b) / np.abs(b)
    return np.where(same, 0.0, np.where(np.isfinite(r), r, np.inf))


def compare(got: dict, ref: dict, label: str = "", check_w: bool = True) -> dict:
    """Check the step's outputs against the oracle's; returns the metrics."""
    met = {}
    for st in ("m", "v"):
        met[f"{st}_k_rel"] = float(rel_err(got[f"{st}k"], ref[f"{st}k"]).max(initial=0.0))
        met[f"{st}_s_rel"] = float(rel_err(got[f"{st}s"], ref[f"{st}s"]).max(initial=0.0))
        d = code_steps(got[f"{st}q"], ref[f"{st}q"])
        met[f"{st}_code_frac"] = float((d != 0).mean()) if d.size else 0.0
        met[f"{st}_code_maxstep"] = int(d.max(initial=0))
    pg, pr = got["p"].astype(np.float64), ref["p"].astype(np.float64)
    bad_p = ~((np.abs(pg - pr) <= np.maximum(TOL_P_REL * np.abs(pr), TOL_P_ABS)) |
              (np.isnan(pg) & np.isnan(pr)))
    met["p_bad"] = int(bad_p.sum())
    met["p_rel"] = float(rel_err(pg, pr).max(initial=0.0))
    if check_w and got.get("w") is not None:
        # bf16 copy: the RNE of the kernel's own fp32 master, within one bf16 ulp of the oracle's
        own = bf16_bits(torch.from_numpy(got["p"]).to(torch.bfloat16))
        nan = np.isnan(got["p"])
        met["w_own_mismatch"] = int(((own != got["w"]) & ~nan).sum())
        # distance in bf16 ulps on the ordered line (+0 and -0 coincide); values
        # within the absolute tolerance of the master weights also pass
        def ordered(b):
            b = b.astype(np.int32)
            return np.where(b & 0x8000, -(b & 0x7FFF), b)
        wd = np.abs(ordered(got["w"]) - ordered(ref["w"]))
        wval = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).double().numpy()
        close = np.abs(wval(got["w"]) - wval(ref["w"])) <= TOL_P_ABS
        met["w_ulps"] = int(np.where(nan | close, 0, wd).max(initial=0))
    log(f"[parity {label}] " + " ".join(f"{k}={v:.3g}" if isinstance(v, float) else f"{k}={v}"
                                        for k, v in met.items()))
    for st in ("m", "v"):
        assert met[f"{st}_k_rel"] <= TOL_SK, (label, st, "k", met)
        assert met[f"{st}_s_rel"] <= TOL_SK, (label, st, "s", met)
        assert met[f"{st}_code_frac"] <= TOL_CODE_FRAC and met[f"{st}_code_maxstep"] <= 1, (label, st, "codes", met)
    assert met["p_bad"] == 0, (label, "params", met)
    if "w_own_mismatch" in met:
        assert met["w_own_mismatch"] == 0 and met["w_ulps"] <= 1, (label, "bf16", met)
    return met
