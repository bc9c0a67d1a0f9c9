"""The multi-tensor step through the entry point that allocates nothing
(coat_fp8_adamw_step_multi_static, its tables in the library's own device
array) against the workspace entry point (coat_fp8_adamw_step_multi), both
through the C ABI: every output buffer must be bit-identical, on two calls in
a row, the second with a smaller parameter list (the array then still holds
the first call's longer tables past the second call's end)."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
HY = dict(lr=float(np.float32(1e-4)), beta1=float(np.float32(0.9)), beta2=float(np.float32(0.95)),
          eps=float(np.float32(1e-8)), weight_decay=float(np.float32(0.1)))
BUFFERS = ("params", "params_bf16", "m_q", "m_s", "m_k", "v_q", "v_s", "v_k")


@pytest.fixture(scope="module")
def coat():
    import fp8_optimizer_state_amd as c
    assert torch.cuda.is_available()
    c.lib()
    return c


def filled(coat, sizes, G, fm, fv, seed):
    dev = torch.device("cuda")
    st = coat.ParamListState(sizes, G, device=dev)
    for i, n in enumerate(sizes):
        if n == 0:
            continue
        t = st.tensor(i)
        synth.params(n, seed, i, device=dev, out=t.params)
        synth.grads(n, seed, i, device=dev, out=t.grads)
        m, v = synth.prior_moments(n, G, seed, i, device=dev)
        coat.quantize(m, t.m_q, t.m_s, t.m_k, group=G, fmt=fm)
        coat.quantize(v, t.v_q, t.v_s, t.v_k, group=G, fmt=fv)
    torch.cuda.synchronize()
    return st


def twin(coat, st):
    """A second state with the same buffers' contents."""
    other = coat.ParamListState(st.sizes, st.group, device=st.params.device)
    for name in ("params", "params_bf16", "grads") + BUFFERS[2:]:
        getattr(other, name).copy_(getattr(st, name))
    torch.cuda.synchronize()
    return other


def same_bits(a, b):
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


@pytest.mark.parametrize("G,fm,fv", [(128, 0, 1), (32, 0, 0), (256, 1, 0)])
def test_static_entry_point_equals_workspace_entry_point(coat, G, fm, fv):
    first = [3 * 1024 * 1024 + 5, 0, 4096, 777, 1024 * 40, 1, 5120 * 3 + 64, 2048]
    second = [1024 * 9, 300, 0, 1024 * 2 + 17]      # fewer and smaller tensors
    for call, sizes in enumerate((first, second)):
        print(f"no-alloc call {call}: G={G} fm={fm} fv={fv} sizes={sizes}", flush=True)
        a = filled(coat, sizes, G, fm, fv, seed=60 + call + G)
        b = twin(coat, a)
        a.step_static(fmt_m=fm, fmt_v=fv, step=10 + call, **HY)
        b.step_unplanned(fmt_m=fm, fmt_v=fv, step=10 + call, **HY)
        torch.cuda.synchronize()
        for name in BUFFERS:
            assert same_bits(getattr(a, name), getattr(b, name)), (call, name)
        # the step did run: the master weights moved
        assert not torch.equal(a.params, filled(coat, sizes, G, fm, fv, seed=60 + call + G).params)
        del a, b
        torch.cuda.empty_cache()
