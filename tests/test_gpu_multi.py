"""GPU parity of the multi-tensor step (one launch over a parameter list)."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import synth
from _parity import HYPER, bf16_bits, compare, log

pytestmark = pytest.mark.gpu
E4, E5, NOEXP = 0, 1, 0x100


@pytest.fixture(scope="module")
def coat():
    import fp8_optimizer_state_amd as c
    assert torch.cuda.is_available()
    c.lib()
    return c


def build_list(coat, sizes, G, fm, fv, seed, threads=16):
    """Seeded inputs per tensor, prior quantized by the oracle, uploaded into
    the flat buffers of a ParamListState. Returns (state, host inputs)."""
    st = coat.ParamListState(sizes, G)
    host = []

    def one(i):
        n = sizes[i]
        p = synth.params(n, seed, i).numpy()
        g = bf16_bits(synth.grads(n, seed, i))
        m, v = synth.prior_moments(n, G, seed, i)
        mq, ms, mk = oracle.quantize(m.numpy(), G, fm)
        vq, vs, vk = oracle.quantize(v.numpy(), G, fv)
        return dict(p=p, g=g, mq=mq, ms=ms, mk=mk, vq=vq, vs=vs, vk=vk)

    with ThreadPoolExecutor(threads) as ex:
        host = list(ex.map(one, range(len(sizes))))
    for i, h in enumerate(host):
        t = st.tensor(i)
        t.params.copy_(torch.from_numpy(h["p"]))
        t.grads.copy_(torch.from_numpy(h["g"].view(np.int16)).view(torch.bfloat16))
        for key in ("mq", "ms", "mk", "vq", "vs", "vk"):
            getattr(t, key[0] + "_" + key[1]).copy_(torch.from_numpy(h[key]))
    torch.cuda.synchronize()
    return st, host


def oracle_list(host, G, fm, fv, threads=16):
    h = HYPER

    def one(x):
        return oracle.adamw_step(x["p"], x["g"], x["mq"], x["ms"], x["mk"], x["vq"], x["vs"], x["vk"],
                                 G, fm, fv, h["lr"], h["b1"], h["b2"], h["eps"], h["wd"], h["step"])

    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(one, host))


def read_list(st):
    out = []
    for i in range(len(st.sizes)):
        t = st.tensor(i)
        out.append(dict(p=t.params.cpu().numpy(), w=bf16_bits(t.params_bf16.cpu()),
                        mq=t.m_q.cpu().numpy(), ms=t.m_s.cpu().numpy(), mk=t.m_k.cpu().numpy(),
                        vq=t.v_q.cpu().numpy(), vs=t.v_s.cpu().numpy(), vk=t.v_k.cpu().numpy()))
    return out


def concat(lst):
    return {k: np.concatenate([d[k] for d in lst]) for k in lst[0]}


def step_kwargs(fm, fv):
    h = HYPER
    return dict(fmt_m=fm, fmt_v=fv, lr=h["lr"], beta1=h["b1"], beta2=h["b2"], eps=h["eps"],
                weight_decay=h["wd"], step=h["step"])


@pytest.mark.parametrize("G,fm,fv", [(16, E4, E4), (32, E4, E5), (64, E5, E4), (128, E4, E5), (128, E5, E5),
                                     (256, E4, E5), (512, E5, E4), (1024, E4, E4)])
def test_mixed_list_equals_single_calls(coat, G, fm, fv):
    """Tiny, empty, ragged and multi-tile tensors in one launch (the multi-tensor
    kernels specialized for each group size, and the partial tiles' kernel);
    the result is bit-identical to one single-tensor call per tensor and
    matches the oracle."""
    sizes = [768, 0, 1, 17, 2304, 1024 * 5 + 3, 50, 128 * 33, 4096 + 1000, 16, 1024 * 9 + 512 + 7]
    log(f"test_mixed_list_equals_single_calls G={G} fm={fm} fv={fv} sizes={sizes}")
    st, host = build_list(coat, sizes, G, fm, fv, seed=41)
    st2, _ = build_list(coat, sizes, G, fm, fv, seed=41)
    st.step(**step_kwargs(fm, fv))
    for i in range(len(sizes)):
        t = st2.tensor(i)
        if sizes[i]:
            coat.adamw_step(t.params, t.params_bf16, t.grads, t.m_q, t.m_s, t.m_k, t.v_q, t.v_s, t.v_k,
                            group=G, **step_kwargs(fm, fv))
    torch.cuda.synchronize()
    a, b = read_list(st), read_list(st2)
    for x, y in zip(a, b):
        for key in x:
            assert np.array_equal(x[key], y[key], equal_nan=True), key
    ref = oracle_list([h for h, n in zip(host, sizes) if n], G, fm, fv)
    compare(concat([x for x, n in zip(a, sizes) if n]), concat(ref), f"mixed-list G={G}")


@pytest.mark.parametrize("G,fm,fv", [(128, E4 | NOEXP, E5 | NOEXP), (256, E4 | NOEXP, E4 | NOEXP),
                                     (32, E4 | NOEXP, E4 | NOEXP), (64, E4 | NOEXP, E5 | NOEXP),
                                     (128, E4 | NOEXP, E5), (32, E4, E4 | NOEXP)])
def test_mixed_list_without_expansion(coat, G, fm, fv):
    """The multi-tensor kernels specialized for launches without expansion
    (every group stored with k = 1; the table kernel for G >= 128, the direct
    kernel below) and the expanded kernels with one moment at k = 1: the same
    list as above, bit-identical to single-tensor calls, within tolerance of
    the oracle, and each moment without expansion equal to the oracle's in
    every scale and code."""
    sizes = [768, 0, 1, 17, 2304, 1024 * 5 + 3, 50, 128 * 33, 4096 + 1000, 16, 1024 * 9 + 512 + 7]
    log(f"test_mixed_list_without_expansion G={G} fm={fm:#x} fv={fv:#x}")
    st, host = build_list(coat, sizes, G, fm, fv, seed=43)
    st2, _ = build_list(coat, sizes, G, fm, fv, seed=43)
    st.step(**step_kwargs(fm, fv))
    for i in range(len(sizes)):
        t = st2.tensor(i)
        if sizes[i]:
            coat.adamw_step(t.params, t.params_bf16, t.grads, t.m_q, t.m_s, t.m_k, t.v_q, t.v_s, t.v_k,
                            group=G, **step_kwargs(fm, fv))
    torch.cuda.synchronize()
    a, b = read_list(st), read_list(st2)
    for x, y in zip(a, b):
        for key in x:
            assert np.array_equal(x[key], y[key], equal_nan=True), key
    got = concat([x for x, n in zip(a, sizes) if n])
    ref = concat(oracle_list([h for h, n in zip(host, sizes) if n], G, fm, fv))
    compare(got, ref, f"mixed-list no expansion G={G}")
    for mo, f in (("m", fm), ("v", fv)):
        if f & NOEXP:
            assert np.all(got[mo + "k"] == 1.0), mo
            assert np.array_equal(got[mo + "s"], ref[mo + "s"]), mo
            assert np.array_equal(got[mo + "q"], ref[mo + "q"]), mo


def test_unplanned_entry_point(coat):
    sizes = [1000, 128 * 40, 77]
    G, fm, fv = 32, E4, E4
    log("test_unplanned_entry_point")
    st, host = build_list(coat, sizes, G, fm, fv, seed=42)
    st.step_unplanned(**step_kwargs(fm, fv))
    compare(concat(read_list(st)), concat(oracle_list(host, G, fm, fv)), "unplanned")


def test_gpt2_small_workload(coat):
    """The GPT-2-small parameter list (124M params, 148 tensors), every group."""
    wl = synth.WORKLOADS["gpt2s"]
    log(f"test_gpt2_small_workload n={wl.n_params}")
    st, host = build_list(coat, wl.sizes, wl.group, wl.fmt_m, wl.fmt_v, seed=wl.seed)
    log("  inputs ready")
    st.step(**step_kwargs(wl.fmt_m, wl.fmt_v))
    torch.cuda.synchronize()
    got = read_list(st)
    del st
    log("  gpu step done")
    ref = oracle_list(host, wl.group, wl.fmt_m, wl.fmt_v)
    log("  oracle done")
    met = compare(concat(got), concat(ref), "gpt2s")
    assert met["m_k_rel"] < 1e-6


@pytest.mark.parametrize("entry", ["workspace", "static"])
def test_one_call_step_under_graph_capture(coat, entry):
    """The one-call multi-tensor entry points enqueue their table copies (in
    the arguments of small copy launches) and the step without waiting, so
    the whole call can be captured into a HIP graph; every replay equals an
    eager call from the same state, bit for bit, with eager work and
    synchronizations between the replays."""
    sizes = [1000, 128 * 40, 77, 3000, 1024 * 3]
    G, fm, fv = 128, E4, E5
    log(f"test_one_call_step_under_graph_capture entry={entry} sizes={sizes}")
    st_e, _ = build_list(coat, sizes, G, fm, fv, seed=43)  # eager
    st_g, _ = build_list(coat, sizes, G, fm, fv, seed=43)  # replayed graph
    L = coat.lib()
    count = len(sizes)
    nbytes = L.coat_multi_workspace_bytes(count)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    descs = st_g.descriptors()
    h = HYPER
    args = (descs, count, G, fm, fv, h["lr"], h["b1"], h["b2"], h["eps"], h["wd"], h["step"])
    if entry == "static":
        # the library looks up its array on a device's first call: not under capture
        st_tmp, _ = build_list(coat, [1024], G, fm, fv, seed=44)
        st_tmp.step_static(**step_kwargs(fm, fv))
        torch.cuda.synchronize()

    def call():
        s = torch.cuda.current_stream().cuda_stream
        if entry == "workspace":
            rc = L.coat_fp8_adamw_step_multi(*args, ws.data_ptr(), nbytes, s)
        else:
            rc = L.coat_fp8_adamw_step_multi_static(*args, s)
        assert rc == 0, rc

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    before = read_list(st_g)
    for x, y in zip(before, read_list(st_e)):  # capturing ran nothing
        for key in x:
            assert np.array_equal(x[key], y[key], equal_nan=True), key
    for r in range(3):
        if entry == "workspace":
            st_e.step_unplanned(**step_kwargs(fm, fv))
        else:
            st_e.step_static(**step_kwargs(fm, fv))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        a, b = read_list(st_e), read_list(st_g)
        for x, y in zip(a, b):
            for key in x:
                assert np.array_equal(x[key], y[key], equal_nan=True), (r, key)
        log(f"  replay {r}: equal to the eager call")
