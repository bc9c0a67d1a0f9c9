"""Resume from a checkpoint on the GPU: five steps, save, load into a fresh
state, five more steps equals ten uninterrupted steps bit for bit (every
state buffer and the bf16 copy). Holds at any size; the step itself is
checked against the oracle in the other GPU tests."""
import os

import pytest
import torch

import synth
from _parity import HYPER, log

pytestmark = pytest.mark.gpu
SIZES = [1000, 4113, 131072, 5, 16384, 300000]


@pytest.fixture(scope="module")
def coat():
    import fp8_optimizer_state_amd as c
    assert torch.cuda.is_available()
    c.lib()
    return c


def _init(coat, G, fm, fv, seed):
    st = coat.ParamListState(SIZES, G, device="cuda")
    for i, n in enumerate(SIZES):
        t = st.tensor(i)
        synth.params(n, seed, i, device="cuda", out=t.params)
        m, v = synth.prior_moments(n, G, seed, i, device="cuda")
        coat.quantize(m, t.m_q, t.m_s, t.m_k, group=G, fmt=fm)
        coat.quantize(v, t.v_q, t.v_s, t.v_k, group=G, fmt=fv)
    torch.cuda.synchronize()
    return st


def _steps(coat, st, steps, fm, fv, seed):
    h = HYPER
    for step in steps:
        for i, n in enumerate(SIZES):
            synth.grads(n, seed, i, device="cuda", out=st.tensor(i).grads, step_index=step - 9)
        st.step(fmt_m=fm, fmt_v=fv, lr=h["lr"], beta1=h["b1"], beta2=h["b2"], eps=h["eps"],
                weight_decay=h["wd"], step=step)
    torch.cuda.synchronize()


def _bits(t):
    return t.view({torch.float32: torch.int32, torch.float64: torch.int64, torch.uint8: torch.uint8,
                   torch.bfloat16: torch.int16}[t.dtype])


@pytest.mark.parametrize("G,fm,fv", [(128, 0, 1), (32, 0, 0)])
def test_resume_is_exact(coat, tmp_path, G, fm, fv):
    seed = 21
    log(f"test_resume_is_exact: G={G} fmt {fm}/{fv}, {sum(SIZES)} params")
    whole = _init(coat, G, fm, fv, seed)
    _steps(coat, whole, range(10, 20), fm, fv, seed)

    first = _init(coat, G, fm, fv, seed)
    _steps(coat, first, range(10, 15), fm, fv, seed)
    path = os.path.join(tmp_path, "state.safetensors")
    first.save(path, step=14, fmt_m=fm, fmt_v=fv)
    del first
    resumed, meta = coat.ParamListState.load(path, device="cuda")
    assert meta == {"step": 14, "fmt_m": fm, "fmt_v": fv}
    _steps(coat, resumed, range(meta["step"] + 1, 20), meta["fmt_m"], meta["fmt_v"], seed)

    for name in list(resumed.STATE_FIELDS) + ["params_bf16"]:
        a, b = getattr(whole, name), getattr(resumed, name)
        assert torch.equal(_bits(a), _bits(b)), f"{name} differs after resume"
    # the moments really moved over the last five steps
    assert int((resumed.m_q != _init(coat, G, fm, fv, seed).m_q).sum()) > 0
