"""CPU oracle for the COAT FP8-state AdamW step (ctypes wrapper over coat_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product package never does.

Every function takes and returns numpy arrays and works on host memory. The
C source cites the pages each step follows; see ``coat_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "coat_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FMT_E4M3 = 0
FMT_E5M2 = 1
FMT_NO_EXPAND = 0x100


def build(force: bool = True) -> str:
    """Compile the oracle with gcc: plain C, IEEE fp64, no contraction, no fast-math."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        L.coat_oracle_fp8_decode.argtypes = [ctypes.c_uint8, i32]
        L.coat_oracle_fp8_decode.restype = ctypes.c_double
        L.coat_oracle_fp8_encode.argtypes = [ctypes.c_double, i32]
        L.coat_oracle_fp8_encode.restype = ctypes.c_uint8
        L.coat_oracle_fp8_range.argtypes = [i32]
        L.coat_oracle_fp8_range.restype = ctypes.c_double
        L.coat_oracle_group_k.argtypes = [ctypes.c_double, ctypes.c_double, i32]
        L.coat_oracle_group_k.restype = f32
        L.coat_oracle_fp8_decode_array.argtypes = [P, i64, i32, P]
        L.coat_oracle_fp8_decode_array.restype = None
        L.coat_oracle_fp8_encode_array.argtypes = [P, i64, i32, P]
        L.coat_oracle_fp8_encode_array.restype = None
        L.coat_oracle_quantize.argtypes = [P, i64, i32, i32, P, P, P]
        L.coat_oracle_quantize.restype = ctypes.c_int
        L.coat_oracle_dequantize.argtypes = [P, P, P, i64, i32, i32, P]
        L.coat_oracle_dequantize.restype = ctypes.c_int
        L.coat_oracle_adamw_dense.argtypes = [P, P, P, P, P, i64, f32, f32, f32, f32, f32, i64]
        L.coat_oracle_adamw_dense.restype = ctypes.c_int
        L.coat_oracle_adamw_step.argtypes = [P, P, P, P, P, P, P, P, P, i64, i32, i32, i32,
                                             f32, f32, f32, f32, f32, i64]
        L.coat_oracle_adamw_step.restype = ctypes.c_int
        L.coat_oracle_act_quantize.argtypes = [P, i64, i32, i32, P, P]
        L.coat_oracle_act_quantize.restype = ctypes.c_int
        L.coat_oracle_act_dequantize.argtypes = [P, P, i64, i32, i32, P]
        L.coat_oracle_act_dequantize.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _check(rc: int):
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (status {rc})")


def ngroups(n: int, G: int) -> int:
    return (n + G - 1) // G


# ---------------------------------------------------------------- codec

def fp8_decode(q: np.ndarray, fmt: int) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    out = np.empty(q.shape, np.float64)
    lib().coat_oracle_fp8_decode_array(_ptr(q), q.size, fmt, _ptr(out))
    return out


def fp8_encode(y: np.ndarray, fmt: int) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float64)
    out = np.empty(y.shape, np.uint8)
    lib().coat_oracle_fp8_encode_array(_ptr(y), y.size, fmt, _ptr(out))
    return out


def fp8_range(fmt: int) -> float:
    return lib().coat_oracle_fp8_range(fmt)


def group_k(amax: float, amin: float, fmt: int) -> float:
    return lib().coat_oracle_group_k(amax, amin, fmt)


# ---------------------------------------------------------------- quantize

def quantize(x: np.ndarray, G: int, fmt: int):
    """Per-group quantization with expansion; returns (q uint8, s float64, k float32)."""
    x = np.ascontiguousarray(x, dtype=np.float64).ravel()
    n = x.size
    q = np.empty(n, np.uint8)
    s = np.empty(ngroups(n, G), np.float64)
    k = np.empty(ngroups(n, G), np.float32)
    _check(lib().coat_oracle_quantize(_ptr(x), n, G, fmt, _ptr(q), _ptr(s), _ptr(k)))
    return q, s, k


def dequantize(q: np.ndarray, s: np.ndarray, k: np.ndarray, G: int, fmt: int) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8).ravel()
    s = np.ascontiguousarray(s, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float32)
    assert s.size == ngroups(q.size, G) and k.size == s.size
    x = np.empty(q.size, np.float64)
    _check(lib().coat_oracle_dequantize(_ptr(q), _ptr(s), _ptr(k), q.size, G, fmt, _ptr(x)))
    return x


# ---------------------------------------------------------------- activation codec

def act_quantize(x: np.ndarray, G: int, fmt: int):
    """bf16 values (as uint16 bits) to FP8 codes with absmax scaling, one fp32
    scale per tensor (G = 0) or per group of G; returns (q uint8, s float32)."""
    x = np.ascontiguousarray(x, dtype=np.uint16).ravel()
    n = x.size
    q = np.empty(n, np.uint8)
    s = np.empty(1 if G == 0 else ngroups(n, G), np.float32)
    _check(lib().coat_oracle_act_quantize(_ptr(x), n, G, fmt, _ptr(q), _ptr(s)))
    return q, s


def act_dequantize(q: np.ndarray, s: np.ndarray, G: int, fmt: int) -> np.ndarray:
    """FP8 codes and scales back to bf16 (uint16 bits)."""
    q = np.ascontiguousarray(q, dtype=np.uint8).ravel()
    s = np.ascontiguousarray(s, dtype=np.float32)
    assert s.size == (1 if G == 0 else ngroups(q.size, G))
    x = np.empty(q.size, np.uint16)
    _check(lib().coat_oracle_act_dequantize(_ptr(q), _ptr(s), q.size, G, fmt, _ptr(x)))
    return x


# ---------------------------------------------------------------- AdamW

def adamw_dense(p, g, m, v, lr, b1, b2, eps, wd, step, want_bf16=True):
    """AdamW on dense fp64 moments. Returns (p', w, m', v') as new arrays."""
    p = np.array(p, dtype=np.float32, copy=True).ravel()
    g = np.ascontiguousarray(g, dtype=np.uint16).ravel()
    m = np.array(m, dtype=np.float64, copy=True).ravel()
    v = np.array(v, dtype=np.float64, copy=True).ravel()
    w = np.empty(p.size, np.uint16) if want_bf16 else None
    _check(lib().coat_oracle_adamw_dense(_ptr(p), _ptr(w), _ptr(g), _ptr(m), _ptr(v), p.size,
                                         lr, b1, b2, eps, wd, step))
    return p, w, m, v


def adamw_step(p, g, mq, ms, mk, vq, vs, vk, G, fmt_m, fmt_v, lr, b1, b2, eps, wd, step,
               threads: int = 1):
    """The FP8-state step on host copies; returns a dict of the new state.

    ``threads`` > 1 splits the groups over that many threads (groups are
    independent, so the result is the same as one call over everything).
    """
    p = np.array(p, dtype=np.float32, copy=True).ravel()
    g = np.ascontiguousarray(g, dtype=np.uint16).ravel()
    mq = np.array(mq, dtype=np.uint8, copy=True).ravel()
    vq = np.array(vq, dtype=np.uint8, copy=True).ravel()
    ms = np.array(ms, dtype=np.float64, copy=True).ravel()
    vs = np.array(vs, dtype=np.float64, copy=True).ravel()
    mk = np.array(mk, dtype=np.float32, copy=True).ravel()
    vk = np.array(vk, dtype=np.float32, copy=True).ravel()
    n = p.size
    ng = ngroups(n, G)
    assert g.size == n and mq.size == n and vq.size == n
    assert ms.size == ng and mk.size == ng and vs.size == ng and vk.size == ng
    w = np.empty(n, np.uint16)
    L = lib()

    def run(g0: int, g1: int):
        e0, e1 = g0 * G, min(n, g1 * G)
        if e1 <= e0:
            return 0
        return L.coat_oracle_adamw_step(
            _ptr(p) + 4 * e0, _ptr(w) + 2 * e0, _ptr(g) + 2 * e0,
            _ptr(mq) + e0, _ptr(ms) + 8 * g0, _ptr(mk) + 4 * g0,
            _ptr(vq) + e0, _ptr(vs) + 8 * g0, _ptr(vk) + 4 * g0,
            e1 - e0, G, fmt_m, fmt_v, lr, b1, b2, eps, wd, step)

    if threads <= 1 or ng < 2 * threads:
        _check(run(0, ng))
    else:
        bounds = np.linspace(0, ng, threads + 1).astype(np.int64)
        with ThreadPoolExecutor(threads) as ex:
            for rc in ex.map(run, bounds[:-1].tolist(), bounds[1:].tolist()):
                _check(rc)
    return dict(p=p, w=w, mq=mq, ms=ms, mk=mk, vq=vq, vs=vs, vk=vk)


def quantize_threaded(x: np.ndarray, G: int, fmt: int, threads: int = 1):
    """``quantize`` split over threads on group boundaries (same result)."""
    x = np.ascontiguousarray(x, dtype=np.float64).ravel()
    n = x.size
    ng = ngroups(n, G)
    q = np.empty(n, np.uint8)
    s = np.empty(ng, np.float64)
    k = np.empty(ng, np.float32)
    L = lib()

    def run(g0: int, g1: int):
        e0, e1 = g0 * G, min(n, g1 * G)
        if e1 <= e0:
            return 0
        return L.coat_oracle_quantize(_ptr(x) + 8 * e0, e1 - e0, G, fmt, _ptr(q) + e0,
                                      _ptr(s) + 8 * g0, _ptr(k) + 4 * g0)

    if threads <= 1 or ng < 2 * threads:
        _check(run(0, ng))
    else:
        bounds = np.linspace(0, ng, threads + 1).astype(np.int64)
        with ThreadPoolExecutor(threads) as ex:
            for rc in ex.map(run, bounds[:-1].tolist(), bounds[1:].tolist()):
                _check(rc)
    return q, s, k
