"""Seeded synthetic inputs for the FP8-state AdamW step.

This module holds no arithmetic of the method: only parameter-list shapes,
random draws and the sampling of groups for parity checks. Both the oracle
side and the HIP side of the tests take their inputs from here, so it is the
one place the two meet.

Distributions (the workload recipe):
  * fp32 master weights  p ~ N(0, 0.02)                      (standard deviation)
  * bf16 gradients        g = bf16_rne(N(0, 1e-3))
  * prior moments, per group of G elements:
        s_g ~ logUniform(1e-5, 1e-2)
        m_i = random sign * s_g * 10^U(-3, 0)                 (about 1000:1 per group)
        v_i = s_g^2 * 10^U(-1, 0)                             (about 10:1 per group)
    The 1000:1 and 10:1 group ratios are the ones the COAT article reports
    for the first and second moments (section "FP8 optimizer states").
  * hyperparameters lr=1e-4, betas=(0.9, 0.95), eps=1e-8, wd=0.1, step=10.
  * activations (for the FP8 activation codec), a (tokens, channels) bf16
    matrix: N(0, 1) times a per-channel scale 10^U(-3, 1), and one value in a
    thousand 50x larger (outliers), rounded to bf16. Stand-in for the inputs of
    Llama-2-13B's linear layers (channels 5120 or 13824); the article gives no
    activation statistics.

Draws use ``torch.Generator`` on the device the tensors live on, one
generator per (seed, tensor index, stream), so any tensor can be regenerated
on its own. CPU and GPU generators give different numbers for the same seed;
tests always copy one side's inputs to the other rather than regenerating.
"""
from __future__ import annotations

import dataclasses
from typing import List, Tuple

import torch

FMT_E4M3 = 0
FMT_E5M2 = 1

HYPER = dict(lr=1e-4, b1=0.9, b2=0.95, eps=1e-8, wd=0.1, step=10)

# ------------------------------------------------------------------ shapes


def _gpt2_small() -> List[Tuple[str, Tuple[int, ...]]]:
    d, ff, vocab, ctx = 768, 3072, 50257, 1024
    out = [("wte", (vocab, d)), ("wpe", (ctx, d))]
    for i in range(12):
        h = f"h.{i}."
        out += [
            (h + "ln_1.weight", (d,)), (h + "ln_1.bias", (d,)),
            (h + "attn.c_attn.weight", (d, 3 * d)), (h + "attn.c_attn.bias", (3 * d,)),
            (h + "attn.c_proj.weight", (d, d)), (h + "attn.c_proj.bias", (d,)),
            (h + "ln_2.weight", (d,)), (h + "ln_2.bias", (d,)),
            (h + "mlp.c_fc.weight", (d, ff)), (h + "mlp.c_fc.bias", (ff,)),
            (h + "mlp.c_proj.weight", (ff, d)), (h + "mlp.c_proj.bias", (d,)),
        ]
    out += [("ln_f.weight", (d,)), ("ln_f.bias", (d,))]
    return out


def _llama2(d: int, ff: int, layers: int, vocab: int = 32000) -> List[Tuple[str, Tuple[int, ...]]]:
    out = [("embed_tokens", (vocab, d))]
    for i in range(layers):
        h = f"layers.{i}."
        out += [
            (h + "self_attn.q_proj", (d, d)), (h + "self_attn.k_proj", (d, d)),
            (h + "self_attn.v_proj", (d, d)), (h + "self_attn.o_proj", (d, d)),
            (h + "mlp.gate_proj", (ff, d)), (h + "mlp.up_proj", (ff, d)),
            (h + "mlp.down_proj", (d, ff)),
            (h + "input_layernorm", (d,)), (h + "post_attention_layernorm", (d,)),
        ]
    out += [("norm", (d,)), ("lm_head", (vocab, d))]
    return out


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shapes: Tuple[Tuple[str, Tuple[int, ...]], ...]
    group: int
    fmt_m: int
    fmt_v: int
    seed: int
    steps: int = 1

    @property
    def sizes(self) -> List[int]:
        out = []
        for _, shp in self.shapes:
            n = 1
            for d in shp:
                n *= d
            out.append(n)
        return out

    @property
    def n_params(self) -> int:
        return sum(self.sizes)

    def bytes_per_param(self) -> float:
        """Algorithmic HBM bytes per parameter of one step.

        Reads: bf16 grad 2 + fp32 master 4 + two FP8 codes 2; writes: fp32
        master 4 + bf16 copy 2 + two codes 2; per group and per state an fp64
        s and an fp32 k are read and written: 2 * 2 * 12 / G.
        """
        return 16.0 + 48.0 / self.group

    def layer0(self) -> List[int]:
        """Indices of the tensors of the first transformer block."""
        return [i for i, (nm, _) in enumerate(self.shapes)
                if nm.startswith("layers.0.") or nm.startswith("h.0.")]


def _as_shapes(lst):
    return tuple((nm, tuple(s)) for nm, s in lst)


WORKLOADS = {
    "flat1m": Workload("flat1m: one flat tensor of 1,048,576 params, G=128, m E4M3 + v E4M3",
                       (("flat", (1048576,)),), 128, FMT_E4M3, FMT_E4M3, seed=0),
    "gpt2s": Workload("gpt2-small parameter list (124M, 148 tensors), G=128, m E4M3 + v E5M2",
                      _as_shapes(_gpt2_small()), 128, FMT_E4M3, FMT_E5M2, seed=1),
    "llama7b": Workload("llama-2-7b parameter list (6.74B, 291 tensors), G=128, m E4M3 + v E4M3",
                        _as_shapes(_llama2(4096, 11008, 32)), 128, FMT_E4M3, FMT_E4M3, seed=2),
    "llama13b": Workload("llama-2-13b parameter list (13.0B, 363 tensors), G=128, m E4M3 + v E5M2",
                         _as_shapes(_llama2(5120, 13824, 40)), 128, FMT_E4M3, FMT_E5M2, seed=3),
    "llama13b_g32": Workload("llama-2-13b parameter list, G=32, m E4M3 + v E4M3, 10 steps",
                             _as_shapes(_llama2(5120, 13824, 40)), 32, FMT_E4M3, FMT_E4M3, seed=4,
                             steps=10),
}

# ------------------------------------------------------------------ draws

_STREAM_P, _STREAM_G, _STREAM_M, _STREAM_V, _STREAM_SG = 1, 2, 3, 4, 5
_STREAM_ACT = 6


def generator(seed: int, tensor: int, stream: int, device) -> torch.Generator:
    gen = torch.Generator(device=device)
    gen.manual_seed((seed * 1_000_003 + tensor) * 16 + stream)
    return gen


def params(n: int, seed: int, tensor: int = 0, device="cpu", out=None) -> torch.Tensor:
    gen = generator(seed, tensor, _STREAM_P, device)
    t = torch.empty(n, dtype=torch.float32, device=device) if out is None else out
    t.normal_(0.0, 0.02, generator=gen)
    return t


def grads(n: int, seed: int, tensor: int = 0, device="cpu", out=None, step_index: int = 0
          ) -> torch.Tensor:
    """bf16 gradients ~ N(0, 1e-3); ``step_index`` gives fresh grads for later steps."""
    gen = generator(seed, tensor, _STREAM_G + 16 * step_index, device)
    g32 = torch.empty(n, dtype=torch.float32, device=device)
    g32.normal_(0.0, 1e-3, generator=gen)
    if out is None:
        return g32.to(torch.bfloat16)
    out.copy_(g32)
    return out


def activations(tokens: int, channels: int, seed: int, device="cpu") -> torch.Tensor:
    """bf16 activations of shape (tokens, channels), flattened row-major."""
    gen = generator(seed, channels, _STREAM_ACT, device)
    ch = torch.empty(channels, dtype=torch.float32, device=device).uniform_(-3.0, 1.0, generator=gen)
    x = torch.empty(tokens, channels, dtype=torch.float32, device=device).normal_(0.0, 1.0, generator=gen)
    x.mul_(torch.pow(10.0, ch))
    out = torch.empty(tokens, channels, dtype=torch.float32, device=device).uniform_(0.0, 1.0, generator=gen)
    x = torch.where(out < 1e-3, x * 50.0, x)
    return x.to(torch.bfloat16).reshape(-1)


def prior_moments(n: int, G: int, seed: int, tensor: int = 0, device="cpu"):
    """Prior (m, v) as fp32 tensors with the per-group spreads given above."""
    ng = (n + G - 1) // G
    gs = generator(seed, tensor, _STREAM_SG, device)
    log_sg = torch.empty(ng, dtype=torch.float64, device=device).uniform_(-5.0, -2.0, generator=gs)
    sg = torch.pow(10.0, log_sg).repeat_interleave(G)[:n]
    gm = generator(seed, tensor, _STREAM_M, device)
    um = torch.empty(n, dtype=torch.float64, device=device).uniform_(-3.0, 0.0, generator=gm)
    sign = torch.empty(n, dtype=torch.float64, device=device).uniform_(-1.0, 1.0, generator=gm)
    m = torch.where(sign < 0, -1.0, 1.0) * sg * torch.pow(10.0, um)
    gv = generator(seed, tensor, _STREAM_V, device)
    uv = torch.empty(n, dtype=torch.float64, device=device).uniform_(-1.0, 0.0, generator=gv)
    v = sg * sg * torch.pow(10.0, uv)
    return m.to(torch.float32), v.to(torch.float32)


# ------------------------------------------------------------------ sampling


def parity_sample(wl: Workload, every: int = 997, layer0: bool = True) -> List[Tuple[int, List[int]]]:
    """Groups to compare at full size, as (tensor index, sorted group indices).

    Every tensor's first and last group, all groups of the first transformer
    block (when ``layer0``), and every ``every``-th group of the whole list
    counted globally.
    """
    G = wl.group
    out = []
    l0 = set(wl.layer0()) if layer0 else set()
    base = 0
    for ti, n in enumerate(wl.sizes):
        ng = (n + G - 1) // G
        if ti in l0:
            idx = list(range(ng))
        else:
            first = (-base) % every
            idx = sorted(set([0, ng - 1] + list(range(first, ng, every))))
        out.append((ti, idx))
        base += ng
    return out
