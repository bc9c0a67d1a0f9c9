"""Checkpoint of a parameter list's optimizer state, host side: the saved file
holds the fp32 masters and the FP8 moments with their per-group scales and
exponents, bit for bit, in 6 + 24/G bytes per parameter; mismatches raise.
(Resuming a run on the GPU is checked in test_gpu_checkpoint.py.)"""
import os

import pytest
import torch

import fp8_optimizer_state_amd as coat

SIZES = [1000, 4113, 131072, 5, 16384]


def _filled(G, seed=0):
    st = coat.ParamListState(SIZES, G, device="cpu")
    g = torch.Generator().manual_seed(seed)
    for name in st.STATE_FIELDS:
        t = getattr(st, name)
        if t.dtype == torch.uint8:
            t.copy_(torch.randint(0, 256, t.shape, generator=g, dtype=torch.uint8))
        else:
            t.copy_(torch.randn(t.shape, generator=g, dtype=torch.float64).to(t.dtype))
    # special values must survive as stored: NaN scale (poisoned group), -0, Inf
    st.m_s[0] = float("nan")
    st.v_s[1] = -0.0
    st.params[2] = float("inf")
    return st


def _bits(t):
    return t.view({torch.float32: torch.int32, torch.float64: torch.int64, torch.uint8: torch.uint8}[t.dtype])


@pytest.mark.parametrize("G", [32, 128])
def test_roundtrip_bit_exact(tmp_path, G):
    st = _filled(G)
    path = os.path.join(tmp_path, "state.safetensors")
    st.save(path, step=14, fmt_m=coat.FMT_E4M3, fmt_v=coat.FMT_E5M2)
    back, meta = coat.ParamListState.load(path, device="cpu")
    assert meta == {"step": 14, "fmt_m": coat.FMT_E4M3, "fmt_v": coat.FMT_E5M2}
    assert back.sizes == SIZES and back.group == G
    for name in st.STATE_FIELDS:
        assert torch.equal(_bits(getattr(back, name)), _bits(getattr(st, name))), name
    # compressed: masters 4 B, codes 2 B, scale 8 B + exponent 4 B per group and moment
    payload = sum(getattr(st, name).numel() * getattr(st, name).element_size() for name in st.STATE_FIELDS)
    assert payload == 6 * st.n_padded + 24 * st.n_groups
    assert payload <= (6 + 24 / G) * st.n_params + 6 * 15 * len(SIZES) + 24 * len(SIZES)
    assert os.path.getsize(path) < payload + 4096


def test_state_dict_is_a_copy():
    st = _filled(128)
    sd = st.state_dict()
    before = sd["m_q"].clone()
    st.m_q.add_(1)
    assert torch.equal(sd["m_q"], before)


def test_mismatches_raise(tmp_path):
    st = _filled(128)
    other = coat.ParamListState(SIZES[:-1], 128, device="cpu")
    with pytest.raises(ValueError):
        other.load_state_dict(st.state_dict())
    bad = st.state_dict()
    bad["m_s"] = bad["m_s"].float()
    with pytest.raises(ValueError):
        st.load_state_dict(bad)
    # a safetensors file of another kind
    from safetensors.torch import save_file
    path = os.path.join(tmp_path, "other.safetensors")
    save_file({"x": torch.zeros(4)}, path, metadata={"format": "something-else"})
    with pytest.raises(ValueError):
        coat.ParamListState.load(path, device="cpu")
