"""GPU parity of the fused FP8-state AdamW step against the oracle (C ABI).

Sizes run from one element to the 1,048,576-parameter flat tensor of the
first workload (G=128, E4M3/E4M3, seed 0), across group sizes, format pairs,
expansion on/off, ragged tails and degenerate groups.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from _parity import (HYPER, StepInputs, bf16_bits, compare, gpu_step, log, make_inputs,
                     oracle_step)

pytestmark = pytest.mark.gpu
E4, E5, NOEXP = 0, 1, 0x100


@pytest.fixture(scope="module", autouse=True)
def coat():
    import fp8_optimizer_state_amd as c
    assert torch.cuda.is_available()
    c.lib()
    return c


def test_flat_1m_workload():
    wl = synth.WORKLOADS["flat1m"]
    n = wl.n_params
    log(f"test_flat_1m_workload n={n} G={wl.group}")
    x = make_inputs(n, wl.group, wl.fmt_m, wl.fmt_v, seed=wl.seed)
    ref = oracle_step(x)
    got = gpu_step(x)
    met = compare(got, ref, "flat1m")
    # the fp64 moment chain keeps k and s far inside the tolerance
    assert met["m_k_rel"] < 1e-6 and met["v_k_rel"] < 1e-6


@pytest.mark.parametrize("fm,fv", [(E4, E4), (E4, E5), (E5, E4), (E5, E5)])
@pytest.mark.parametrize("G", [16, 32, 64, 128, 256, 512, 1024])
def test_groups_and_formats(fm, fv, G):
    n = 1024 * 9 + 5 * G // 2 + 7  # several tiles, a ragged last lane and a short last group
    log(f"test_groups_and_formats fm={fm} fv={fv} G={G} n={n}")
    x = make_inputs(n, G, fm, fv, seed=100 + G + 7 * fm + 3 * fv)
    compare(gpu_step(x), oracle_step(x), f"G={G} fm={fm} fv={fv}")


@pytest.mark.parametrize("fm,fv", [(E4 | NOEXP, E4 | NOEXP), (E4 | NOEXP, E5), (E4, E5 | NOEXP)])
def test_no_expansion(fm, fv):
    n, G = 1024 * 6 + 100, 128
    log(f"test_no_expansion fm={fm:#x} fv={fv:#x}")
    x = make_inputs(n, G, fm, fv, seed=31)
    got, ref = gpu_step(x), oracle_step(x)
    compare(got, ref, "noexp")
    # a moment stored and requantized with k = 1 follows the definition's
    # arithmetic exactly: s = amax / fpmax, |q| s, RN(RN(b x) + RN(c g)), so its
    # scales and codes equal the oracle's bit for bit
    for st, f in (("m", fm), ("v", fv)):
        if f & NOEXP:
            assert np.all(got[st + "k"] == 1.0)
            assert np.array_equal(got[st + "s"], ref[st + "s"]), st
            assert np.array_equal(got[st + "q"], ref[st + "q"]), st


@pytest.mark.parametrize("n", [1, 2, 15, 16, 17, 127, 128, 129, 1023, 1024, 1025, 4096 + 3])
def test_ragged_sizes(n):
    log(f"test_ragged_sizes n={n}")
    x = make_inputs(n, 128, E4, E5, seed=n)
    compare(gpu_step(x), oracle_step(x), f"n={n}")


@pytest.mark.parametrize("step", [1, 2, 1000])
def test_step_counts(step):
    log(f"test_step_counts step={step}")
    x = make_inputs(4096, 128, E4, E5, seed=9)
    compare(gpu_step(x, step=step), oracle_step(x, step=step), f"t={step}")


def test_no_bf16_copy():
    log("test_no_bf16_copy")
    x = make_inputs(5000, 64, E4, E4, seed=10)
    got, ref = gpu_step(x, want_bf16=False), oracle_step(x)
    compare(got, ref, "no-bf16", check_w=False)


# the rare-path tests run with expansion and, through the kernels specialized
# for it, without expansion on both moments
RARE_FMTS = [(E4, E5), (E4 | NOEXP, E5 | NOEXP)]


@pytest.mark.parametrize("fm,fv", RARE_FMTS)
def test_zero_state_and_zero_grads(fm, fv):
    """All-zero groups (zero state, zero grads) next to ordinary ones."""
    n, G = 1024 * 4, 128
    x = make_inputs(n, G, fm, fv, seed=12)
    x.g[: 3 * G] = 0
    for q, s in ((x.mq, x.ms), (x.vq, x.vs)):
        q[: 3 * G] = 0
        s[:3] = 0.0
    x.g[3 * G: 3 * G + 5] = 0x8000  # -0.0 grads in an ordinary group
    log(f"test_zero_state_and_zero_grads fm={fm:#x} fv={fv:#x}")
    got, ref = gpu_step(x), oracle_step(x)
    compare(got, ref, "zeros")
    assert np.all(got["ms"][:3] == 0) and np.all(got["mk"][:3] == 1)


@pytest.mark.parametrize("fm,fv", [(E4, E4), (E4 | NOEXP, E4 | NOEXP)])
def test_nonfinite_grads_poison_their_group_only(fm, fv):
    n, G = 1024 * 3, 128
    x = make_inputs(n, G, fm, fv, seed=13)
    x.g[5] = 0x7FC0            # NaN in group 0
    x.g[G * 7 + 3] = 0x7F80    # +Inf in group 7
    x.g[G * 12 + 100] = 0xFF80  # -Inf in group 12
    log(f"test_nonfinite_grads_poison_their_group_only fm={fm:#x} fv={fv:#x}")
    got, ref = gpu_step(x), oracle_step(x)
    compare(got, ref, "poison")
    for gi in (0, 7, 12):
        assert np.isnan(got["ms"][gi]) and np.all(got["mq"][gi * G:(gi + 1) * G] == 0x7F)
    assert np.isfinite(got["ms"][[1, 2, 6, 8, 11, 13]]).all()


def test_extreme_groups_take_the_exact_path():
    """Groups whose moments leave the fp32 range or are wider than 2^100, and
    narrow tiny groups that trip the range guard."""
    n, G = 32 * 8, 32
    x = make_inputs(n, G, E4, E5, seed=14)
    rng = np.random.default_rng(3)
    x.g[:] = 0  # moments then just decay: m' = b1 m, v' = b2 v
    blocks = [
        1e-200 * (1 + rng.random(G)),                       # tiny, narrow: range guard
        1e-60 * 10.0 ** rng.uniform(-3, 0, G),              # below fp32 range
        np.r_[1.0, 1e-40, 10.0 ** rng.uniform(-30, 0, G - 2)],  # wider than 2^100
        1e30 * (1 + rng.random(G)),                         # large
        1e-3 * (1 + np.linspace(0, 2e-6, G)),               # near-constant, just above 1 + 1e-6
        10.0 ** rng.uniform(-8, -2, G),                     # ordinary
        np.r_[np.zeros(G - 1), 1e-300],                     # a single tiny member
        1e-12 * (1 + rng.random(G)),
    ]
    for b, blk in enumerate(blocks):
        sl = slice(b * G, (b + 1) * G)
        for fmt, (q, s, k) in ((E4, (x.mq, x.ms, x.mk)), (E5, (x.vq, x.vs, x.vk))):
            qq, ss, kk = oracle.quantize(np.abs(blk) if fmt == E5 else blk, G, fmt)
            q[sl], s[b], k[b] = qq, ss[0], kk[0]
    log("test_extreme_groups_take_the_exact_path")
    compare(gpu_step(x), oracle_step(x), "extreme")


def test_repeated_steps_track_the_oracle():
    """Ten consecutive steps with fresh grads, the GPU and the oracle each
    carrying its own state forward; compared after every step."""
    n, G = 1024 * 8, 32
    x = make_inputs(n, G, E4, E4, seed=15)
    xg, xo = x, x
    for t in range(10, 20):
        gbits = bf16_bits(synth.grads(n, 15, step_index=t))
        xg = StepInputs(xg.p, gbits, xg.mq, xg.ms, xg.mk, xg.vq, xg.vs, xg.vk, G, E4, E4)
        xo = StepInputs(xo.p, gbits, xo.mq, xo.ms, xo.mk, xo.vq, xo.vs, xo.vk, G, E4, E4)
        log(f"test_repeated_steps step={t}")
        got, ref = gpu_step(xg, step=t), oracle_step(xo, step=t)
        compare(got, ref, f"t={t}")
        xg = StepInputs(got["p"], gbits, got["mq"], got["ms"], got["mk"], got["vq"], got["vs"],
                        got["vk"], G, E4, E4)
        xo = StepInputs(ref["p"], gbits, ref["mq"], ref["ms"], ref["mk"], ref["vq"], ref["vs"],
                        ref["vk"], G, E4, E4)


def test_deterministic():
    x = make_inputs(1024 * 16, 128, E4, E5, seed=16)
    a, b = gpu_step(x), gpu_step(x)
    for key in a:
        if a[key] is not None:
            assert np.array_equal(a[key], b[key], equal_nan=True), key


def _bf16(x):
    """bf16 rounding (nearest, ties to even) of float values, as float64."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def _bf16_bits(x):
    """bf16 bit patterns of float values by truncation (exact for values that
    already are bf16 numbers)."""
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def threshold_groups():
    """A beta1 and, per offset o in -2..2, the gradients (g_a, g_b) of a group
    whose new first moments have RN(amax / amin) = T + o ulp, T = 1 + 1e-6.

    The group's stored first moment is x = 0.5 in every element (code 0x38,
    the value 1, with s = 0.5 and k = 1), so both the kernel and the oracle
    form m' = RN(b1 x + (1 - b1) g) with one rounding: b1 x and (1 - b1) g are
    exact in fp64 for an fp32 b1 and a bf16 g. One element takes g_a, the
    others g_b: amax = m'_a, amin = m'_b. Found by search over fp32 b1 in
    [0.5, 0.99] (coarse ratio from g_a, then g_b moves m'_b by whole ulps)."""
    T = 1.0 + 1e-6
    U = np.spacing(T)
    b1 = np.arange(np.float32(0.5).view(np.uint32), np.float32(0.99).view(np.uint32),
                   dtype=np.uint32).view(np.float32).astype(np.float64)
    c1 = 1.0 - b1
    X = b1 * 0.5
    ga = _bf16((T - 1.0) * X / c1)
    mA = X + c1 * ga
    uX = np.spacing(X)
    hits = None
    for o in (-2, -1, 0, 1, 2):
        j = np.round((mA / (T + o * U) - X) / uX)
        gb = _bf16(j * uX / c1)
        mB = X + c1 * gb
        good = (np.abs(j) <= 60) & (mB == X + j * uX) & (mA / mB == T + o * U)
        hits = good if hits is None else hits & good
    i = int(np.flatnonzero(hits)[0])
    out = []
    for o in (-2, -1, 0, 1, 2):
        j = np.round((mA[i] / (T + o * U) - X[i]) / uX[i])
        out.append((o, ga[i], _bf16(j * uX[i] / c1[i])))
    return float(np.float32(b1[i])), out


def test_near_constant_threshold():
    """Groups whose max/min quotient rounds to 1 + 1e-6 minus two ulps up to
    plus two ulps: k = 1 up to and including the threshold, expanded above it,
    on the GPU exactly as in the oracle (per-group tables, G = 128)."""
    b1, cases = threshold_groups()
    n, G = 1024, 128
    x = make_inputs(n, G, E4, E4, seed=41)
    for gi, (o, ga, gb) in enumerate(cases):
        sl = slice(gi * G, (gi + 1) * G)
        x.mq[sl] = 0x38           # E4M3 value 1.0
        x.ms[gi], x.mk[gi] = 0.5, 1.0
        x.vq[sl] = np.where(np.arange(G) % 2 == 0, 0x38, 0x40)  # values 1 and 2
        x.vs[gi], x.vk[gi] = 2.0 ** -20, 1.0
        x.g[sl] = _bf16_bits(gb)
        x.g[gi * G] = _bf16_bits(ga)[()]
    log(f"test_near_constant_threshold b1={b1!r} cases={cases}")
    got, ref = gpu_step(x, b1=b1), oracle_step(x, b1=b1)
    # the oracle decides by the rounded quotient: k = 1 up to T, expanded above
    for gi, (o, _, _) in enumerate(cases):
        assert (ref["mk"][gi] == 1.0) == (o <= 0), (o, ref["mk"][gi])
    compare(got, ref, "threshold")
    assert np.array_equal(got["mk"][:5], ref["mk"][:5])


@pytest.mark.parametrize("fm,fv", RARE_FMTS)
@pytest.mark.parametrize("G", [16, 32, 128])
def test_huge_grads_update_in_fp64(G, fm, fv):
    """bf16 grads of 1e20 and up make v' (and, near the bf16 maximum, the
    update's intermediates) exceed the fp32 range while every moment stays
    finite in fp64: the update must still follow the oracle, and no group is
    poisoned."""
    n = 1024 * 3
    x = make_inputs(n, G, fm, fv, seed=42 + G)
    big = np.array([1e20, -3e20, 3e38, -3.3e38, 2e25], np.float32)
    x.g[5:10] = _bf16_bits(big)                # one group with several huge grads
    x.g[G + 17] = _bf16_bits(np.float32(-1e30))[()]
    x.g[1024 + 3 * G: 1024 + 4 * G] = _bf16_bits(np.full(G, 7e21, np.float32))  # a whole group
    log(f"test_huge_grads_update_in_fp64 G={G} fm={fm:#x} fv={fv:#x}")
    got, ref = gpu_step(x), oracle_step(x)
    assert np.isfinite(ref["ms"]).all() and np.isfinite(ref["vs"]).all()
    compare(got, ref, f"huge grads G={G}")


@pytest.mark.parametrize("G", [32, 128, 256])
def test_nan_and_inf_codes_without_expansion(G):
    """A state stored with k = 1 everywhere (both moments without expansion)
    whose finite groups hold an E4M3 NaN code (first moment) or an E5M2 Inf
    or NaN code (second moment) among ordinary codes: each such code decodes
    to NaN or Inf as the oracle's does, in every launch shape (for G >= 128
    the waves whose groups all have k = 1 build only the exact tables)."""
    n = 1024 * 3
    fm, fv = E4 | NOEXP, E5 | NOEXP
    x = make_inputs(n, G, fm, fv, seed=44 + G)
    assert np.all(x.mk == 1.0) and np.all(x.vk == 1.0)
    x.mq[G + 5] = 0x7F                        # E4M3 NaN in group 1
    x.mq[1024 + 2 * G + 9] = 0xFF             # E4M3 -NaN in a later tile
    x.vq[3 * G + 1] = 0x7C                    # E5M2 +Inf in group 3
    x.vq[2048 + 7] = 0x7E                     # E5M2 NaN in the last tile
    log(f"test_nan_and_inf_codes_without_expansion G={G}")
    got, ref = gpu_step(x), oracle_step(x)
    compare(got, ref, f"nan/inf codes G={G}")
    assert np.isnan(ref["p"][G + 5]) and np.isnan(got["p"][G + 5])


@pytest.mark.parametrize("fm,fv", RARE_FMTS)
@pytest.mark.parametrize("G", [16, 32, 128])
def test_poisoned_state_poisons_its_own_moment_only(G, fm, fv):
    """A stored first-moment group that is poisoned (s = NaN, codes 0x7F)
    next to a finite second-moment group: the first moment stays poisoned,
    the second is requantized as usual, and vice versa."""
    n = 1024 * 2
    x = make_inputs(n, G, fm, fv, seed=43 + G)
    x.mq[0:G] = 0x7F
    x.ms[0], x.mk[0] = np.nan, 1.0
    x.vq[3 * G:4 * G] = 0x7F                  # E5M2 NaN code
    x.vs[3], x.vk[3] = np.nan, 1.0
    log(f"test_poisoned_state_poisons_its_own_moment_only G={G} fm={fm:#x} fv={fv:#x}")
    got, ref = gpu_step(x), oracle_step(x)
    assert np.isnan(ref["ms"][0]) and np.isfinite(ref["vs"][0])
    assert np.isnan(ref["vs"][3]) and np.isfinite(ref["ms"][3])
    compare(got, ref, f"poisoned state G={G}")
    assert np.isfinite(got["vs"][0]) and np.isfinite(got["ms"][3])
