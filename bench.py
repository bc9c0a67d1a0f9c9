"""Benchmark of the fused FP8-state AdamW step on one MI355X.

Workload (default): the Llama-2-13B parameter list (13,015,864,320 params in
363 tensors), group 128, first moment E4M3 and second moment E5M2, fp32
master weights, bf16 grads in, bf16 weight copy out; synthetic seeded inputs
resident in HBM (about 133 GB). One step = one multi-tensor launch over the
whole list. Prints one JSON line on stdout; progress goes to stderr.

  python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload llama13b]
                  [--no-cpu-baseline] [--no-reference] [--copy-calibration]
                  [--sweep | --act | --codec | --ceiling]

After the measured steps it also times, unless --no-reference, the same step
without expansion (every group k = 1: the same bytes with the least
arithmetic) on the same box, as a reference for what the box's memory and
clock allow; it is reported beside the measurement, never as `value`.

With --ceiling it measures, in one process and on the same resident
workload, what the step's time is judged against: a plain device copy of
4 GiB (torch copy_), the memory-only floor of the step's access pattern (the
instrument in bench_ceiling.hip: the step's bytes in the step's pattern, no
arithmetic) at the step's residency and at full residency, the step
without expansion (every group k = 1: the same bytes, the least arithmetic)
and the step itself, in interleaved rounds; one JSON line per measurement and
round, a markdown table on stderr.

With --sweep it instead times the step and measures the state codec's
quantization error for every group size in {32, 64, 128, 256}, format pair
{E4M3/E4M3, E4M3/E5M2} and expansion on/off, on the same parameter list:
one JSON line per variant on stdout, a markdown table on stderr.

With --codec it times the FP8 state codec (quantize fp32 moments to codes,
scales and exponents, and dequantize them back; groups of 32 and 128, m in
E4M3 and v in E5M2) on 2^30 values: one JSON line per launch kind.

With --act it times the FP8 activation codec (per tensor and per group of 128,
E4M3 and E5M2) on a 16384 x 13824 bf16 activation matrix (the input of
Llama-2-13B's down projection for 16k tokens): one JSON line per launch kind.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0


def pmc_file(workload: str) -> str:
    """The committed rocprofv3 counter summary (HBM bytes) of a workload's step kernel."""
    return os.path.join(ROOT, "profiles", f"coat_step_multi_{workload}_pmc.json")


# the sources the step kernel is built from (the activation codec is not one)
KERNEL_SRCS = [os.path.join(ROOT, "fp8_optimizer_state_amd", "csrc", f)
               for f in ("coat_common.h", "coat_host.h", "coat_fp8.hip")]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """sha256 over the step kernel's source files, in order."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(workload: str, n_launch_bytes: float):
    """HBM traffic per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    try:
        with open(pmc_file(workload)) as f:
            pmc = json.load(f)
    except (OSError, ValueError):
        return None
    if pmc.get("source_sha256") != kernel_source_hash() or pmc.get("workload") != workload:
        return None
    return pmc.get("hbm_bytes_per_launch")


def quant_error_sums(x, xhat, G: int):
    """Quantization error of one tensor, as sums to pool over tensors:
    (sum over groups with a nonzero norm of ||xhat - x||_2 / ||x||_2, number of
    such groups, sum over nonzero x of |xhat - x| / |x|, number of nonzero x).
    Groups are G consecutive elements; a short last group is padded with zeros,
    which add to neither norm. Accumulated in fp64."""
    import torch

    x = x.reshape(-1).to(torch.float64)
    d = xhat.reshape(-1).to(torch.float64) - x
    pad = (-x.numel()) % G
    if pad:
        x = torch.nn.functional.pad(x, (0, pad))
        d = torch.nn.functional.pad(d, (0, pad))
    nx = x.view(-1, G).pow(2).sum(1).sqrt()
    nd = d.view(-1, G).pow(2).sum(1).sqrt()
    live = nx > 0
    nz = x != 0
    return (float((nd[live] / nx[live]).sum()), int(live.sum()),
            float((d[nz].abs() / x[nz].abs()).sum()), int(nz.sum()))


def sweep(args) -> int:
    """Step time and codec error for each group size x format pair x expansion."""
    import torch

    import fp8_optimizer_state_amd as coat
    import synth

    base = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    coat.lib()
    h = synth.HYPER
    names = {0: "E4M3", 1: "E5M2"}
    rows = []
    for G in (32, 64, 128, 256):
        st = coat.ParamListState(base.sizes, G, device=dev)
        n = st.n_params
        for fm, fv in ((0, 0), (0, 1)):
            for expand in (True, False):
                flag = 0 if expand else coat.FMT_NO_EXPAND
                err = {"m": [0.0, 0, 0.0, 0], "v": [0.0, 0, 0.0, 0]}
                for i, ni in enumerate(base.sizes):
                    t = st.tensor(i)
                    synth.params(ni, base.seed, i, device=dev, out=t.params)
                    synth.grads(ni, base.seed, i, device=dev, out=t.grads)
                    m, v = synth.prior_moments(ni, G, base.seed, i, device=dev)
                    for name, x, q, s_, k_, f in (("m", m, t.m_q, t.m_s, t.m_k, fm), ("v", v, t.v_q, t.v_s, t.v_k, fv)):
                        coat.quantize(x, q, s_, k_, group=G, fmt=f | flag)
                        xh = torch.empty_like(x)
                        coat.dequantize(q, s_, k_, xh, group=G, fmt=f)
                        e = quant_error_sums(x, xh, G)
                        acc = err[name]
                        for j in range(4):
                            acc[j] += e[j]
                        del xh
                    del m, v
                torch.cuda.synchronize()
                hy = dict(fmt_m=fm | flag, fmt_v=fv | flag, lr=h["lr"], beta1=h["b1"], beta2=h["b2"],
                          eps=h["eps"], weight_decay=h["wd"])
                st.plan()
                step = h["step"]
                for _ in range(args.warmup):
                    st.step(step=step, **hy)
                    step += 1
                stream = torch.cuda.current_stream()
                ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                ev0.record(stream)
                for _ in range(args.steps):
                    st.step(step=step, **hy)
                    step += 1
                ev1.record(stream)
                torch.cuda.synchronize()
                ms = ev0.elapsed_time(ev1) / args.steps
                bpp = 16.0 + 48.0 / G
                gbps = bpp * n / (ms * 1e-3) / 1e9
                row = {"sweep": args.workload, "group": G, "fmt_m": names[fm], "fmt_v": names[fv],
                       "expand": expand, "n_params": n, "ms_per_step": ms, "params_per_s": n / (ms * 1e-3),
                       "bytes_per_param": bpp, "achieved_GBps": gbps, "frac_of_8TBps": gbps / PEAK_HBM_GBPS,
                       "m_err_normwise": err["m"][0] / err["m"][1], "m_err_elementwise": err["m"][2] / err["m"][3],
                       "v_err_normwise": err["v"][0] / err["v"][1], "v_err_elementwise": err["v"][2] / err["v"][3]}
                rows.append(row)
                print(json.dumps(row), flush=True)
                log(f"G={G} {names[fm]}/{names[fv]} expand={expand}: {ms:.2f} ms/step, "
                    f"m err {row['m_err_normwise']:.4g}, v err {row['v_err_normwise']:.4g}")
        del st
        torch.cuda.empty_cache()
    log("| G | m / v | expansion | ms/step | params/s | GB/s | % of 8 TB/s | m err (normwise) | m err (elem.) "
        "| v err (normwise) | v err (elem.) |")
    log("|---|---|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        log(f"| {r['group']} | {r['fmt_m']} / {r['fmt_v']} | {'on' if r['expand'] else 'off'} | "
            f"{r['ms_per_step']:.2f} | {r['params_per_s']:.3e} | {r['achieved_GBps']:.0f} | "
            f"{100 * r['frac_of_8TBps']:.1f} | {r['m_err_normwise']:.4g} | {r['m_err_elementwise']:.4g} | "
            f"{r['v_err_normwise']:.4g} | {r['v_err_elementwise']:.4g} |")
    return 0


def act_bench(args) -> int:
    """Throughput of the activation codec's entry points, inputs resident in HBM."""
    import torch

    import fp8_optimizer_state_amd as coat
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    coat.lib()
    tokens, channels = 16384, 13824
    x = synth.activations(tokens, channels, seed=13, device=dev)
    n = x.numel()
    q = torch.empty(n, dtype=torch.uint8, device=dev)
    back = torch.empty(n, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    for fmt, fname in ((0, "E4M3"), (1, "E5M2")):
        for G in (0, 128):
            s = torch.empty(coat.act_nscales(n, G), dtype=torch.float32, device=dev)
            ops = (("quantize", lambda: coat.act_quantize(x, q, s, group=G, fmt=fmt),
                    (2.0 + 2.0 + 1.0) if G == 0 else (2.0 + 1.0 + 4.0 / G)),
                   ("dequantize", lambda: coat.act_dequantize(q, s, back, group=G, fmt=fmt),
                    (1.0 + 2.0) if G == 0 else (1.0 + 4.0 / G + 2.0)))
            for name, fn, bpe in ops:
                for _ in range(args.warmup):
                    fn()
                ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                ev0.record(stream)
                for _ in range(args.steps):
                    fn()
                ev1.record(stream)
                torch.cuda.synchronize()
                ms = ev0.elapsed_time(ev1) / args.steps
                gbps = bpe * n / (ms * 1e-3) / 1e9
                row = {"act_codec": name, "granularity": "tensor" if G == 0 else f"group {G}", "fmt": fname,
                       "n": n, "shape": [tokens, channels], "ms": ms, "elements_per_s": n / (ms * 1e-3),
                       "bytes_per_element": bpe, "achieved_GBps": gbps, "frac_of_8TBps": gbps / PEAK_HBM_GBPS}
                print(json.dumps(row), flush=True)
                log(f"act {name} {row['granularity']} {fname}: {ms:.3f} ms, {gbps:.0f} GB/s")
    return 0


def codec_bench(args) -> int:
    """Throughput of the state codec's entry points (quantize fp32 moments to
    (q, s, k), dequantize back) on 2^30 first- and second-moment-shaped values
    resident in HBM."""
    import torch

    import fp8_optimizer_state_amd as coat
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    coat.lib()
    n = 1 << 30
    stream = torch.cuda.current_stream()
    for G in (32, 128):
        m, v = synth.prior_moments(n, G, 17, 0, device=dev)
        q = torch.empty(n, dtype=torch.uint8, device=dev)
        s = torch.empty(coat.ngroups(n, G), dtype=torch.float64, device=dev)
        k = torch.empty(coat.ngroups(n, G), dtype=torch.float32, device=dev)
        back = torch.empty(n, dtype=torch.float32, device=dev)
        for moment, x, fmt, fname in (("m", m, coat.FMT_E4M3, "E4M3"), ("v", v, coat.FMT_E5M2, "E5M2")):
            bpe = 4.0 + 1.0 + 12.0 / G
            ops = (("quantize", lambda: coat.quantize(x, q, s, k, group=G, fmt=fmt)),
                   ("dequantize", lambda: coat.dequantize(q, s, k, back, group=G, fmt=fmt)))
            for name, fn in ops:
                for _ in range(args.warmup):
                    fn()
                ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                ev0.record(stream)
                for _ in range(args.steps):
                    fn()
                ev1.record(stream)
                torch.cuda.synchronize()
                ms = ev0.elapsed_time(ev1) / args.steps
                gbps = bpe * n / (ms * 1e-3) / 1e9
                row = {"state_codec": name, "moment": moment, "group": G, "fmt": fname, "n": n, "ms": ms,
                       "elements_per_s": n / (ms * 1e-3), "bytes_per_element": bpe, "achieved_GBps": gbps,
                       "frac_of_8TBps": gbps / PEAK_HBM_GBPS}
                print(json.dumps(row), flush=True)
                log(f"state codec {name} {moment} G={G} {fname}: {ms:.3f} ms, {gbps:.0f} GB/s")
        del m, v, q, s, k, back
        torch.cuda.empty_cache()
    return 0


def resident_state(wl, dev):
    """Seeded inputs and prior state of a workload, generated on the device."""
    import torch

    import fp8_optimizer_state_amd as coat
    import synth

    G = wl.group
    st = coat.ParamListState(wl.sizes, G, device=dev)
    for i, n in enumerate(wl.sizes):
        t = st.tensor(i)
        synth.params(n, wl.seed, i, device=dev, out=t.params)
        synth.grads(n, wl.seed, i, device=dev, out=t.grads)
        m, v = synth.prior_moments(n, G, wl.seed, i, device=dev)
        coat.quantize(m, t.m_q, t.m_s, t.m_k, group=G, fmt=wl.fmt_m)
        coat.quantize(v, t.v_q, t.v_s, t.v_k, group=G, fmt=wl.fmt_v)
        del m, v
        if i % 60 == 0:
            log(f"  generated tensor {i}/{len(wl.sizes)}")
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return st


def time_copy(dev, reps: int):
    """Device copy of 2^30 fp32 (4 GiB read + 4 GiB written), HIP events on the
    copy's stream; returns (ms per copy, GB/s over the bytes moved)."""
    import torch

    a = torch.empty(1 << 30, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    a.fill_(1.0)
    stream = torch.cuda.current_stream()
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        b.copy_(a)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    torch.cuda.empty_cache()
    return ms, 2.0 * 4.0 * (1 << 30) / (ms * 1e-3) / 1e9


def ceiling(args) -> int:
    """Plain copy, the memory-only floor of the step's pattern and the step,
    side by side on one resident workload."""
    import ctypes

    import torch

    import fp8_optimizer_state_amd as coat
    import synth

    wl = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    coat.lib()
    path = os.path.join(ROOT, "libbench_ceiling.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run python -c 'import __graft_entry__ as g; g.build()'")
    probe = ctypes.CDLL(path)
    P = ctypes.c_void_p
    probe.ceiling_pattern_pass.argtypes = [P] * 9 + [ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, P]
    probe.ceiling_pattern_pass.restype = ctypes.c_int
    probe.ceiling_copy_pass.argtypes = [P, P, ctypes.c_int64, P]
    probe.ceiling_read_pass.argtypes = [P, ctypes.c_int64, P, P]
    probe.ceiling_write_pass.argtypes = [P, ctypes.c_int64, P]
    for f in (probe.ceiling_copy_pass, probe.ceiling_read_pass, probe.ceiling_write_pass):
        f.restype = ctypes.c_int
    G = wl.group
    lg = G.bit_length() - 1
    log(f"ceiling: workload {wl.name}")
    st = resident_state(wl, dev)
    # the probe walks the flat buffers as one tensor of whole tiles; every group
    # it touches is a group of the list
    n_probe = st.n_padded // 1024 * 1024
    assert n_probe // G <= st.n_groups and n_probe <= st.n_padded
    h = synth.HYPER
    hy = dict(fmt_m=wl.fmt_m, fmt_v=wl.fmt_v, lr=h["lr"], beta1=h["b1"], beta2=h["b2"], eps=h["eps"],
              weight_decay=h["wd"])
    st.plan()
    stream = torch.cuda.current_stream()
    step_lds = 37688  # the table kernel's LDS per block: four blocks per CU
    bpp = wl.bytes_per_param()
    step_no = [h["step"]]

    def probe_pass(layout, lds):
        rc = probe.ceiling_pattern_pass(st.params.data_ptr(), st.params_bf16.data_ptr(), st.grads.data_ptr(),
                                        st.m_q.data_ptr(), st.v_q.data_ptr(), st.m_s.data_ptr(), st.m_k.data_ptr(),
                                        st.v_s.data_ptr(), st.v_k.data_ptr(), n_probe, lg, layout, lds,
                                        stream.cuda_stream)
        assert rc == 0, rc

    def step_once(expand=True):
        flag = 0 if expand else coat.FMT_NO_EXPAND
        st.step(step=step_no[0], **dict(hy, fmt_m=wl.fmt_m | flag, fmt_v=wl.fmt_v | flag))
        step_no[0] += 1

    # plain streams over 4 GiB buffers (copy: 4 GiB read + 4 GiB written)
    bufa = torch.ones(1 << 30, dtype=torch.float32, device=dev)
    bufb = torch.empty_like(bufa)
    word = torch.zeros(4, dtype=torch.int32, device=dev)
    n16 = bufa.numel() // 4
    gib4 = 4.0 * (1 << 30)

    def plain(rc):
        assert rc == 0, rc

    kinds = (("read 4 GiB", lambda: plain(probe.ceiling_read_pass(bufa.data_ptr(), n16, word.data_ptr(),
                                                                  stream.cuda_stream)), gib4),
             ("write 4 GiB", lambda: plain(probe.ceiling_write_pass(bufb.data_ptr(), n16, stream.cuda_stream)), gib4),
             ("copy 4 GiB (probe kernel)", lambda: plain(probe.ceiling_copy_pass(bufa.data_ptr(), bufb.data_ptr(), n16,
                                                                               stream.cuda_stream)), 2 * gib4),
             ("pattern floor, lane-contiguous, step residency", lambda: probe_pass(0, step_lds), bpp * n_probe),
             ("pattern floor, whole-tile (the step's), step residency", lambda: probe_pass(1, step_lds),
              bpp * n_probe),
             ("pattern floor, whole-tile, full residency", lambda: probe_pass(1, 0), bpp * n_probe),
             ("step without expansion (k = 1)", lambda: step_once(False), bpp * wl.n_params),
             ("step", step_once, bpp * wl.n_params))
    # the two step rows leave the state in each other's form (k = 1 or
    # expanded), so each timed batch of a step row follows one untimed launch
    primed = {"step without expansion (k = 1)", "step"}
    for _, fn, _ in kinds:
        for _ in range(args.warmup):
            fn()
    torch.cuda.synchronize()
    rows = {"copy 4 GiB (torch copy_)": []}
    rows.update({name: [] for name, _, _ in kinds})
    rounds = 3
    for r in range(rounds):
        ms, gbps = time_copy(dev, args.steps)
        rows["copy 4 GiB (torch copy_)"].append((ms, gbps))
        print(json.dumps({"ceiling": "copy 4 GiB (torch copy_)", "round": r, "ms": ms, "GBps": gbps,
                          "frac_of_8TBps": gbps / PEAK_HBM_GBPS}), flush=True)
        for name, fn, nbytes in kinds:
            if name in primed:
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.steps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            gbps = nbytes / (ms * 1e-3) / 1e9
            rows[name].append((ms, gbps))
            print(json.dumps({"ceiling": name, "round": r, "workload": wl.name, "ms": ms, "GBps": gbps,
                              "frac_of_8TBps": gbps / PEAK_HBM_GBPS}), flush=True)
        log(f"round {r} done")
    log(f"| measurement ({wl.name}) | ms (mean of {rounds} rounds x {args.steps}) | GB/s | % of 8 TB/s |")
    log("|---|---|---|---|")
    for name, vals in rows.items():
        ms = sum(v[0] for v in vals) / len(vals)
        gb = sum(v[1] for v in vals) / len(vals)
        log(f"| {name} | {ms:.3f} | {gb:.0f} | {100 * gb / PEAK_HBM_GBPS:.1f} |")
    return 0


def cpu_baseline(wl, per_tensor: int = 229376) -> dict:
    """The oracle, single-threaded, on a bounded sample of the workload: the
    first `per_tensor` elements of every tensor (about 65M params for the
    13B list, 10-20 s of CPU work), prior state quantized by the oracle beforehand (untimed)."""
    import numpy as np

    import oracle
    import synth

    F32 = lambda x: float(np.float32(x))
    h = synth.HYPER
    G = wl.group
    chunks = []
    for i, n in enumerate(wl.sizes):
        c = min(n, per_tensor)
        p = synth.params(c, wl.seed, i).numpy()
        g = synth.grads(c, wl.seed, i).view(__import__("torch").int16).numpy().view(np.uint16)
        m, v = synth.prior_moments(c, G, wl.seed, i)
        chunks.append((p, g, m.numpy(), v.numpy()))
    p = np.concatenate([c[0] for c in chunks])
    g = np.concatenate([c[1] for c in chunks])
    # every chunk is a whole number of groups, so concatenation keeps group boundaries
    mq, ms, mk = oracle.quantize_threaded(np.concatenate([c[2] for c in chunks]), G, wl.fmt_m, 8)
    vq, vs, vk = oracle.quantize_threaded(np.concatenate([c[3] for c in chunks]), G, wl.fmt_v, 8)
    n = p.size
    log(f"cpu baseline: oracle on {n} params, 1 thread")
    t0 = time.perf_counter()
    oracle.adamw_step(p, g, mq, ms, mk, vq, vs, vk, G, wl.fmt_m, wl.fmt_v, F32(h["lr"]), F32(h["b1"]),
                      F32(h["b2"]), F32(h["eps"]), F32(h["wd"]), h["step"], threads=1)
    dt = time.perf_counter() - t0
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": n / dt, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": f"first {per_tensor} elements of each of the {len(wl.sizes)} tensors "
                      f"({n} params), one step, single-threaded fp64 C oracle; {dt:.1f} s on {cpu} "
                      f"({os.cpu_count()} hardware threads on the host)",
            "seconds": dt}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama13b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-reference", action="store_true",
                    help="skip the step without expansion timed after the measured steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (for counter calibration)")
    ap.add_argument("--sweep", action="store_true",
                    help="time and measure the codec error of every group size / format / expansion variant")
    ap.add_argument("--act", action="store_true", help="time the FP8 activation codec instead of the step")
    ap.add_argument("--codec", action="store_true",
                    help="time the FP8 state codec (quantize / dequantize of moments) instead of the step")
    ap.add_argument("--ceiling", action="store_true",
                    help="time a plain copy, the memory-only floor of the step's pattern and the step side by side")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0:
        print("bench.py needs --steps >= 1 and --warmup >= 0", file=sys.stderr)
        return 2
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the step shards by whole groups with no exchange between GPUs)",
              file=sys.stderr)
        return 2
    if args.sweep:
        return sweep(args)
    if args.act:
        return act_bench(args)
    if args.codec:
        return codec_bench(args)
    if args.ceiling:
        return ceiling(args)

    import torch

    import fp8_optimizer_state_amd as coat
    import synth

    wl = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    coat.lib()
    G = wl.group
    log(f"workload {wl.name}: {wl.n_params} params, {len(wl.sizes)} tensors")

    # ---- resident state and inputs, generated on the device
    t0 = time.perf_counter()
    st = resident_state(wl, dev)
    log(f"inputs resident in {time.perf_counter() - t0:.1f} s; "
        f"{torch.cuda.memory_allocated() / 1e9:.1f} GB allocated")

    h = synth.HYPER
    hy = dict(fmt_m=wl.fmt_m, fmt_v=wl.fmt_v, lr=h["lr"], beta1=h["b1"], beta2=h["b2"],
              eps=h["eps"], weight_decay=h["wd"])
    st.plan()
    step = h["step"]
    for _ in range(args.warmup):
        st.step(step=step, **hy)
        step += 1
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")

    stream = torch.cuda.current_stream()
    # an event between consecutive launches as well, for the per-step spread
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(args.steps):
        st.step(step=step, **hy)
        step += 1
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    ms_median, ms_min = per_step[len(per_step) // 2], per_step[0]
    log(f"timed {args.steps} steps: {ms:.3f} ms/step (median {ms_median:.3f}, min {ms_min:.3f})")

    n = wl.n_params
    bpp = wl.bytes_per_param()
    launch_bytes = bpp * n

    # the same step without expansion, after the measured steps (which it
    # does not touch): warm-up launches first, the first of which converts the
    # state to k = 1 groups
    ref = None
    if not args.no_reference:
        noexp = dict(hy, fmt_m=wl.fmt_m | coat.FMT_NO_EXPAND, fmt_v=wl.fmt_v | coat.FMT_NO_EXPAND)
        for _ in range(max(args.warmup, 1)):
            st.step(step=step, **noexp)
            step += 1
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        r0.record(stream)
        for _ in range(args.steps):
            st.step(step=step, **noexp)
            step += 1
        r1.record(stream)
        torch.cuda.synchronize()
        ref_ms = r0.elapsed_time(r1) / args.steps
        ref_gbps = launch_bytes / (ref_ms * 1e-3) / 1e9
        ref = {"what": "the same step with COAT_FMT_NO_EXPAND on both moments (every group k = 1: "
                       "the same bytes, no 2^x, no per-group tables), timed after the measured steps",
               "ms_per_step": ref_ms, "GBps": ref_gbps, "frac_of_8TBps": ref_gbps / PEAK_HBM_GBPS,
               "measured_over_reference_time": ms / ref_ms}
        log(f"reference without expansion: {ref_ms:.3f} ms/step ({100 * ref_gbps / PEAK_HBM_GBPS:.1f} % of 8 TB/s)")

    copy = None
    if args.copy_calibration:
        # a device copy of known size, for the counter calibration, timed as well
        copy_ms, copy_gbps = time_copy(dev, 5)
        copy = {"bytes": 2 * 4 * (1 << 30), "ms": copy_ms, "GBps": copy_gbps,
                "frac_of_8TBps": copy_gbps / PEAK_HBM_GBPS}
        log(f"copy calibration: 4 GiB fp32 copy, {copy_ms:.3f} ms, {copy_gbps:.0f} GB/s")

    achieved = launch_bytes / (ms * 1e-3) / 1e9
    traffic = load_traffic(args.workload, launch_bytes)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl)
        log(f"cpu baseline {cpu['value']:.3e} params/s ({cpu['seconds']:.1f} s)")
        cpu.pop("seconds")

    out = {
        "metric": "params/s of fused FP8-state AdamW step; achieved HBM GB/s vs 8 TB/s peak",
        "value": n / (ms * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_median": ms_median,
        "ms_per_step_min": ms_min,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "n_params": n,
            "tensors": len(wl.sizes),
            "group": G,
            "fmt_m": "E4M3", "fmt_v": "E5M2" if wl.fmt_v == 1 else "E4M3",
            "bytes_per_param": bpp,
            "launches_per_step": 1,
            "hyper": {k: v for k, v in h.items()},
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS,
            "traffic": traffic,
            "traffic_source": (f"rocprofv3 FETCH_SIZE and WRITE_SIZE runs committed in "
                               f"{os.path.relpath(pmc_file(args.workload), ROOT)}, taken on kernel source sha256 "
                               f"{kernel_source_hash()[:16]}; not measured in this run")
            if traffic is not None else "null: no committed counter run matches this kernel source and workload",
        },
        "cpu_baseline": cpu,
    }
    if ref is not None:
        out["reference_no_expansion"] = ref
    if copy is not None:
        out["copy_calibration"] = copy
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
