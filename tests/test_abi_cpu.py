"""The C ABI library loads and exports every function include/coat_fp8.h
declares; argument checks that return before any device work (CPU only)."""
import ctypes
import os
import re

import pytest

import fp8_optimizer_state_amd as coat

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "coat_fp8.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(coat_\w+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("coat_fp8_adamw_step", "coat_fp8_adamw_step_multi", "coat_multi_plan_init",
                 "coat_fp8_adamw_step_planned", "coat_multi_workspace_bytes", "coat_fp8_quantize",
                 "coat_fp8_dequantize", "coat_fp8_encode", "coat_fp8_decode", "coat_strerror",
                 "coat_abi_version", "coat_fp8_act_quantize", "coat_fp8_act_dequantize"):
        assert want in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(coat.LIB_PATH)
    missing = [nm for nm in declared_functions() if not hasattr(L, nm)]
    assert not missing, missing


def test_static_helpers():
    L = coat.lib()
    assert L.coat_abi_version() == 102
    assert coat.strerror(0) == "ok" and "invalid" in coat.strerror(-1)
    assert L.coat_multi_workspace_bytes(363) >= 363 * 80 + 364 * 8
    assert L.coat_multi_workspace_bytes(363) % 256 == 0


FAKE = 0x7F0000000000  # never dereferenced: every call below fails validation first
HY = (1e-4, 0.9, 0.95, 1e-8, 0.1)


def step(**kw):
    a = dict(p=FAKE, w=None, g=FAKE, mq=FAKE, ms=FAKE, mk=FAKE, vq=FAKE, vs=FAKE, vk=FAKE,
             n=1024, G=128, fm=0, fv=0, hy=HY, t=10)
    a.update(kw)
    return coat.lib().coat_fp8_adamw_step(a["p"], a["w"], a["g"], a["mq"], a["ms"], a["mk"],
                                          a["vq"], a["vs"], a["vk"], a["n"], a["G"], a["fm"],
                                          a["fv"], *a["hy"], a["t"], None)


@pytest.mark.parametrize("G", [0, 8, 15, 100, 2048, -128])
def test_bad_group(G):
    assert step(G=G) == coat.COAT_EINVAL


@pytest.mark.parametrize("fm,fv", [(2, 0), (0, 7), (0x200, 0), (-1, 0)])
def test_bad_format(fm, fv):
    assert step(fm=fm, fv=fv) == coat.COAT_EINVAL


def test_bad_step_and_hyper():
    assert step(t=0) == coat.COAT_EINVAL
    assert step(hy=(float("nan"),) + HY[1:]) == coat.COAT_EINVAL
    assert step(hy=(1e-4, 1.0, 0.95, 1e-8, 0.1)) == coat.COAT_EINVAL  # 1 - b1^t = 0
    assert step(n=-1) == coat.COAT_EINVAL


def test_null_and_alignment():
    assert step(p=None) == coat.COAT_EINVAL
    assert step(mk=None) == coat.COAT_EINVAL
    assert step(p=FAKE + 4) == coat.COAT_EALIGN
    assert step(mq=FAKE + 1) == coat.COAT_EALIGN
    assert step(w=FAKE + 2) == coat.COAT_EALIGN
    assert step(ms=FAKE + 4) == coat.COAT_EALIGN
    assert step(n=0, p=None) == coat.COAT_OK  # nothing to do


def test_codec_argument_checks():
    L = coat.lib()
    assert L.coat_fp8_quantize(FAKE, 100, 96, 0, FAKE, FAKE, FAKE, None) == coat.COAT_EINVAL
    assert L.coat_fp8_quantize(FAKE + 4, 100, 128, 0, FAKE, FAKE, FAKE, None) == coat.COAT_EALIGN
    assert L.coat_fp8_dequantize(FAKE, FAKE, FAKE, 100, 128, 5, FAKE, None) == coat.COAT_EINVAL
    assert L.coat_fp8_encode(FAKE, 10, 0x100, FAKE, None) == coat.COAT_EINVAL
    assert L.coat_fp8_decode(None, 10, 0, FAKE, None) == coat.COAT_EINVAL
    assert L.coat_fp8_encode(FAKE, 0, 0, None, None) == coat.COAT_OK


def test_act_codec_argument_checks():
    L = coat.lib()
    q, d = L.coat_fp8_act_quantize, L.coat_fp8_act_dequantize
    assert q(FAKE, 100, 96, 0, FAKE, FAKE, None) == coat.COAT_EINVAL      # group not a power of two
    assert q(FAKE, 100, 8, 0, FAKE, FAKE, None) == coat.COAT_EINVAL       # group below 16
    assert q(FAKE, 100, 0, 0x100, FAKE, FAKE, None) == coat.COAT_EINVAL   # no flags on activations
    assert q(FAKE, -1, 0, 0, FAKE, FAKE, None) == coat.COAT_EINVAL
    assert q(None, 100, 0, 0, FAKE, FAKE, None) == coat.COAT_EINVAL
    assert q(FAKE + 2, 100, 128, 1, FAKE, FAKE, None) == coat.COAT_EALIGN
    assert q(FAKE, 100, 128, 1, FAKE + 8, FAKE, None) == coat.COAT_EALIGN
    assert q(FAKE, 100, 128, 1, FAKE, FAKE + 2, None) == coat.COAT_EALIGN
    assert q(None, 0, 0, 0, None, None, None) == coat.COAT_OK
    assert d(FAKE, FAKE, 100, 2048, 0, FAKE, None) == coat.COAT_EINVAL
    assert d(FAKE, FAKE, 100, 0, 2, FAKE, None) == coat.COAT_EINVAL
    assert d(FAKE, FAKE, 100, 0, 0, FAKE + 4, None) == coat.COAT_EALIGN
    assert d(FAKE, None, 100, 0, 0, FAKE, None) == coat.COAT_EINVAL


def test_multi_argument_checks():
    L = coat.lib()
    plan = coat._Plan()
    arr = (coat._Tensor * 1)()
    arr[0] = coat._Tensor(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1024)
    need = L.coat_multi_workspace_bytes(1)
    assert L.coat_multi_plan_init(ctypes.byref(plan), arr, 1, None, need, None) == coat.COAT_EINVAL
    assert L.coat_multi_plan_init(ctypes.byref(plan), arr, 1, FAKE, need - 1, None) == coat.COAT_EINVAL
    assert L.coat_multi_plan_init(ctypes.byref(plan), arr, 1, FAKE + 16, need, None) == coat.COAT_EALIGN
    arr[0].params = FAKE + 8
    assert L.coat_multi_plan_init(ctypes.byref(plan), arr, 1, FAKE, need, None) == coat.COAT_EALIGN
    assert L.coat_multi_plan_init(ctypes.byref(plan), arr, -1, FAKE, need, None) == coat.COAT_EINVAL
    assert L.coat_fp8_adamw_step_planned(None, 128, 0, 0, *HY, 10, None) == coat.COAT_EINVAL


def test_static_multi_argument_checks():
    L = coat.lib()
    f = L.coat_fp8_adamw_step_multi_static
    arr = (coat._Tensor * 2)()
    arr[0] = coat._Tensor(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1024)
    arr[1] = coat._Tensor(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0)
    big = (coat._Tensor * (coat.STATIC_MAX_TENSORS + 1))()
    assert f(big, coat.STATIC_MAX_TENSORS + 1, 128, 0, 0, *HY, 10, None) == coat.COAT_ERANGE
    assert "static plan table" in coat.strerror(coat.COAT_ERANGE)
    assert f(arr, -1, 128, 0, 0, *HY, 10, None) == coat.COAT_EINVAL
    assert f(None, 1, 128, 0, 0, *HY, 10, None) == coat.COAT_EINVAL
    assert f(arr, 1, 96, 0, 0, *HY, 10, None) == coat.COAT_EINVAL
    assert f(arr, 1, 128, 0, 0, *HY, 0, None) == coat.COAT_EINVAL
    arr[0].m_q = FAKE + 1
    assert f(arr, 1, 128, 0, 0, *HY, 10, None) == coat.COAT_EALIGN
    # nothing to do: returns before any device call
    assert f(arr, 0, 128, 0, 0, *HY, 10, None) == coat.COAT_OK
    empty = (coat._Tensor * 1)()
    empty[0] = coat._Tensor(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0)
    assert f(empty, 1, 128, 0, 0, *HY, 10, None) == coat.COAT_OK
