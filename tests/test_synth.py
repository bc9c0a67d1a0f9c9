"""The seeded input generator: parameter-list shapes and value distributions (CPU)."""
import numpy as np
import torch

import synth


def test_workload_sizes():
    W = synth.WORKLOADS
    assert W["flat1m"].n_params == 1048576
    assert len(W["gpt2s"].shapes) == 148 and W["gpt2s"].n_params == 124439808
    assert len(W["llama7b"].shapes) == 291 and W["llama7b"].n_params == 6738415616
    assert len(W["llama13b"].shapes) == 363 and W["llama13b"].n_params == 13015864320
    assert W["llama13b"].bytes_per_param() == 16.375
    assert W["llama13b_g32"].bytes_per_param() == 17.5
    assert all(n % 128 == 0 for n in W["llama13b"].sizes)


def test_distributions_and_seeding():
    n, G = 128 * 512, 128
    p = synth.params(n, 0)
    assert abs(p.std().item() - 0.02) < 5e-4 and abs(p.mean().item()) < 5e-4
    g = synth.grads(n, 0)
    assert g.dtype == torch.bfloat16 and abs(g.float().std().item() - 1e-3) < 3e-5
    assert torch.equal(synth.params(n, 0), p) and not torch.equal(synth.params(n, 1), p)
    assert not torch.equal(synth.grads(n, 0, step_index=1), g)
    m, v = synth.prior_moments(n, G, 0)
    am = m.abs().double().view(-1, G)
    ratio_m = (am.max(1).values / am.min(1).values).numpy()
    ratio_v = (v.double().view(-1, G).max(1).values / v.double().view(-1, G).min(1).values).numpy()
    # spreads near the 1000:1 and 10:1 the article reports
    assert 300 < np.median(ratio_m) <= 1000 and 5 < np.median(ratio_v) <= 10
    assert (m < 0).float().mean().item() > 0.45


def test_parity_sample_covers_edges_and_layer0():
    wl = synth.WORKLOADS["llama13b"]
    smp = synth.parity_sample(wl)
    assert len(smp) == 363
    l0 = set(wl.layer0())
    for ti, idx in smp:
        ng = wl.sizes[ti] // wl.group
        assert idx[0] == 0 and idx[-1] == ng - 1
        if ti in l0:
            assert len(idx) == ng
