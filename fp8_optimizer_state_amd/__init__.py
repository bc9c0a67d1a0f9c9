"""Python binding of the MI355X FP8-optimizer-state AdamW step.

Argument marshalling only: every call hands raw device pointers of torch
tensors and torch's current HIP stream to ``libcoat_fp8.so`` (the C ABI in
``include/coat_fp8.h``); all arithmetic runs in the HIP kernels. There is no
fallback: if the library is missing or no GPU is present the calls raise.

Method: COAT's optimizer over FP8-compressed Adam state with per-group
dynamic range expansion ("COAT: FP8 training, 40% less memory, 1.4x faster",
blob.wenxiaobai.com, sections "FP8 optimizer states" and "Solution: dynamic
range expansion").
"""
from __future__ import annotations

import ctypes
import json
import os
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import torch

FMT_E4M3 = 0
FMT_E5M2 = 1
FMT_NO_EXPAND = 0x100

COAT_OK, COAT_EINVAL, COAT_EALIGN, COAT_EHIP, COAT_ERANGE = 0, -1, -2, -3, -4
STATIC_MAX_TENSORS = 4096

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcoat_fp8.so")


class CoatError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {strerror(status)} (status {status})")


class _Tensor(ctypes.Structure):
    _fields_ = [("params", ctypes.c_void_p), ("params_bf16", ctypes.c_void_p),
                ("grads", ctypes.c_void_p), ("m_q", ctypes.c_void_p), ("m_s", ctypes.c_void_p),
                ("m_k", ctypes.c_void_p), ("v_q", ctypes.c_void_p), ("v_s", ctypes.c_void_p),
                ("v_k", ctypes.c_void_p), ("n", ctypes.c_int64)]


class _Plan(ctypes.Structure):
    _fields_ = [("workspace", ctypes.c_void_p), ("count", ctypes.c_int32),
                ("tiles", ctypes.c_int64), ("n_total", ctypes.c_int64), ("n_partial", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libcoat_fp8.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run python -m fp8_optimizer_state_amd._build")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    hyper = [f32, f32, f32, f32, f32, i64]
    L.coat_fp8_adamw_step.argtypes = [P, P, P, P, P, P, P, P, P, i64, i32, i32, i32, *hyper, P]
    L.coat_multi_workspace_bytes.argtypes = [i32]
    L.coat_multi_workspace_bytes.restype = ctypes.c_size_t
    L.coat_multi_plan_init.argtypes = [ctypes.POINTER(_Plan), ctypes.POINTER(_Tensor), i32, P,
                                       ctypes.c_size_t, P]
    L.coat_fp8_adamw_step_planned.argtypes = [ctypes.POINTER(_Plan), i32, i32, i32, *hyper, P]
    L.coat_fp8_adamw_step_multi.argtypes = [ctypes.POINTER(_Tensor), i32, i32, i32, i32, *hyper,
                                            P, ctypes.c_size_t, P]
    L.coat_fp8_adamw_step_multi_static.argtypes = [ctypes.POINTER(_Tensor), i32, i32, i32, i32, *hyper, P]
    L.coat_fp8_quantize.argtypes = [P, i64, i32, i32, P, P, P, P]
    L.coat_fp8_dequantize.argtypes = [P, P, P, i64, i32, i32, P, P]
    L.coat_fp8_encode.argtypes = [P, i64, i32, P, P]
    L.coat_fp8_decode.argtypes = [P, i64, i32, P, P]
    L.coat_fp8_act_quantize.argtypes = [P, i64, i32, i32, P, P, P]
    L.coat_fp8_act_dequantize.argtypes = [P, P, i64, i32, i32, P, P]
    L.coat_strerror.argtypes = [ctypes.c_int]
    L.coat_strerror.restype = ctypes.c_char_p
    L.coat_abi_version.restype = ctypes.c_int
    for name in ("coat_fp8_adamw_step", "coat_multi_plan_init", "coat_fp8_adamw_step_planned",
                 "coat_fp8_adamw_step_multi", "coat_fp8_adamw_step_multi_static", "coat_fp8_quantize", "coat_fp8_dequantize",
                 "coat_fp8_encode", "coat_fp8_decode", "coat_fp8_act_quantize",
                 "coat_fp8_act_dequantize"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def strerror(status: int) -> str:
    return lib().coat_strerror(status).decode()


def _check(status: int, what: str):
    if status != COAT_OK:
        raise CoatError(status, what)


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ptr(t: Optional[torch.Tensor], dtype: torch.dtype, numel: int, name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return t.data_ptr()


def ngroups(n: int, group: int) -> int:
    return (n + group - 1) // group


# ---------------------------------------------------------------- single tensor

def adamw_step(params, params_bf16, grads, m_q, m_s, m_k, v_q, v_s, v_k, *, group: int,
               fmt_m: int, fmt_v: int, lr: float, beta1: float, beta2: float, eps: float,
               weight_decay: float, step: int, stream=None) -> None:
    """One FP8-state AdamW step of one tensor, in place (asynchronous)."""
    n = params.numel()
    ng = ngroups(n, group)
    rc = lib().coat_fp8_adamw_step(
        _ptr(params, torch.float32, n, "params"), _ptr(params_bf16, torch.bfloat16, n, "params_bf16"),
        _ptr(grads, torch.bfloat16, n, "grads"),
        _ptr(m_q, torch.uint8, n, "m_q"), _ptr(m_s, torch.float64, ng, "m_s"),
        _ptr(m_k, torch.float32, ng, "m_k"),
        _ptr(v_q, torch.uint8, n, "v_q"), _ptr(v_s, torch.float64, ng, "v_s"),
        _ptr(v_k, torch.float32, ng, "v_k"),
        n, group, fmt_m, fmt_v, lr, beta1, beta2, eps, weight_decay, step, _stream(stream))
    _check(rc, "coat_fp8_adamw_step")


# ---------------------------------------------------------------- codec

def quantize(x, q, s, k, *, group: int, fmt: int, stream=None) -> None:
    n = x.numel()
    ng = ngroups(n, group)
    rc = lib().coat_fp8_quantize(_ptr(x, torch.float32, n, "x"), n, group, fmt,
                                 _ptr(q, torch.uint8, n, "q"), _ptr(s, torch.float64, ng, "s"),
                                 _ptr(k, torch.float32, ng, "k"), _stream(stream))
    _check(rc, "coat_fp8_quantize")


def dequantize(q, s, k, x, *, group: int, fmt: int, stream=None) -> None:
    n = q.numel()
    ng = ngroups(n, group)
    rc = lib().coat_fp8_dequantize(_ptr(q, torch.uint8, n, "q"), _ptr(s, torch.float64, ng, "s"),
                                   _ptr(k, torch.float32, ng, "k"), n, group, fmt,
                                   _ptr(x, torch.float32, n, "x"), _stream(stream))
    _check(rc, "coat_fp8_dequantize")


def encode(y, q, *, fmt: int, stream=None) -> None:
    n = y.numel()
    rc = lib().coat_fp8_encode(_ptr(y, torch.float32, n, "y"), n, fmt,
                               _ptr(q, torch.uint8, n, "q"), _stream(stream))
    _check(rc, "coat_fp8_encode")


def decode(q, y, *, fmt: int, stream=None) -> None:
    n = q.numel()
    rc = lib().coat_fp8_decode(_ptr(q, torch.uint8, n, "q"), n, fmt,
                               _ptr(y, torch.float32, n, "y"), _stream(stream))
    _check(rc, "coat_fp8_decode")


def act_nscales(n: int, group: int) -> int:
    """Scales of an activation tensor: one per tensor (group 0) or per group."""
    return 1 if group == 0 else ngroups(n, group)


def act_quantize(x, q, scale, *, group: int, fmt: int, stream=None) -> None:
    """bf16 activations -> FP8 codes + fp32 scales, per tensor (group 0) or per group."""
    n = x.numel()
    rc = lib().coat_fp8_act_quantize(_ptr(x, torch.bfloat16, n, "x"), n, group, fmt,
                                     _ptr(q, torch.uint8, n, "q"),
                                     _ptr(scale, torch.float32, act_nscales(n, group), "scale"),
                                     _stream(stream))
    _check(rc, "coat_fp8_act_quantize")


def act_dequantize(q, scale, x, *, group: int, fmt: int, stream=None) -> None:
    """FP8 codes + fp32 scales -> bf16 activations."""
    n = q.numel()
    rc = lib().coat_fp8_act_dequantize(_ptr(q, torch.uint8, n, "q"),
                                       _ptr(scale, torch.float32, act_nscales(n, group), "scale"), n,
                                       group, fmt, _ptr(x, torch.bfloat16, n, "x"), _stream(stream))
    _check(rc, "coat_fp8_act_dequantize")


# ---------------------------------------------------------------- parameter lists

def _pad16(n: int) -> int:
    return (n + 15) // 16 * 16


@dataclass
class TensorState:
    """Views of one tensor's slice of the flat buffers of a ``ParamListState``."""
    params: torch.Tensor
    params_bf16: torch.Tensor
    grads: torch.Tensor
    m_q: torch.Tensor
    m_s: torch.Tensor
    m_k: torch.Tensor
    v_q: torch.Tensor
    v_s: torch.Tensor
    v_k: torch.Tensor


class ParamListState:
    """Flat device buffers for a whole parameter list and its FP8 Adam state.

    Each tensor's slice of every element buffer starts on a 16-element
    boundary (16-byte aligned FP8 codes); per-group arrays are packed.
    """

    def __init__(self, sizes: Sequence[int], group: int, device="cuda", with_bf16: bool = True):
        self.sizes = [int(n) for n in sizes]
        self.group = group
        self.offsets, self.goffsets = [], []
        off = goff = 0
        for n in self.sizes:
            self.offsets.append(off)
            self.goffsets.append(goff)
            off += _pad16(n)
            goff += ngroups(n, group)
        self.n_padded, self.n_groups = off, goff
        dev = torch.device(device)
        self.params = torch.zeros(off, dtype=torch.float32, device=dev)
        self.params_bf16 = torch.zeros(off, dtype=torch.bfloat16, device=dev) if with_bf16 else None
        self.grads = torch.zeros(off, dtype=torch.bfloat16, device=dev)
        self.m_q = torch.zeros(off, dtype=torch.uint8, device=dev)
        self.v_q = torch.zeros(off, dtype=torch.uint8, device=dev)
        self.m_s = torch.zeros(goff, dtype=torch.float64, device=dev)
        self.v_s = torch.zeros(goff, dtype=torch.float64, device=dev)
        self.m_k = torch.ones(goff, dtype=torch.float32, device=dev)
        self.v_k = torch.ones(goff, dtype=torch.float32, device=dev)
        self._plan = None
        self._workspace = None

    @property
    def n_params(self) -> int:
        return sum(self.sizes)

    def tensor(self, i: int) -> TensorState:
        o, n, go, ng = self.offsets[i], self.sizes[i], self.goffsets[i], ngroups(self.sizes[i], self.group)
        w = self.params_bf16[o:o + n] if self.params_bf16 is not None else None
        return TensorState(self.params[o:o + n], w, self.grads[o:o + n],
                           self.m_q[o:o + n], self.m_s[go:go + ng], self.m_k[go:go + ng],
                           self.v_q[o:o + n], self.v_s[go:go + ng], self.v_k[go:go + ng])

    def descriptors(self):
        arr = (_Tensor * len(self.sizes))()
        for i, n in enumerate(self.sizes):
            t = self.tensor(i)
            arr[i] = _Tensor(t.params.data_ptr(), t.params_bf16.data_ptr() if t.params_bf16 is not None else None,
                             t.grads.data_ptr(), t.m_q.data_ptr(), t.m_s.data_ptr(), t.m_k.data_ptr(),
                             t.v_q.data_ptr(), t.v_s.data_ptr(), t.v_k.data_ptr(), n)
        return arr

    def plan(self, stream=None) -> _Plan:
        """Upload the descriptor table once; reused by every ``step``."""
        if self._plan is None:
            L = lib()
            count = len(self.sizes)
            nbytes = L.coat_multi_workspace_bytes(count)
            self._workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.params.device)
            plan = _Plan()
            descs = self.descriptors()
            _check(L.coat_multi_plan_init(ctypes.byref(plan), descs, count, self._workspace.data_ptr(),
                                          nbytes, _stream(stream)), "coat_multi_plan_init")
            self._plan = plan
        return self._plan

    def step(self, *, fmt_m: int, fmt_v: int, lr: float, beta1: float, beta2: float, eps: float,
             weight_decay: float, step: int, stream=None) -> None:
        """One FP8-state AdamW step over every tensor, one kernel launch (asynchronous)."""
        plan = self.plan(stream)
        rc = lib().coat_fp8_adamw_step_planned(ctypes.byref(plan), self.group, fmt_m, fmt_v, lr, beta1,
                                               beta2, eps, weight_decay, step, _stream(stream))
        _check(rc, "coat_fp8_adamw_step_planned")

    def step_unplanned(self, *, fmt_m: int, fmt_v: int, lr: float, beta1: float, beta2: float,
                       eps: float, weight_decay: float, step: int, stream=None) -> None:
        """The same step through the one-call entry point (uploads the table each time)."""
        L = lib()
        count = len(self.sizes)
        nbytes = L.coat_multi_workspace_bytes(count)
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.params.device)
        rc = L.coat_fp8_adamw_step_multi(self.descriptors(), count, self.group, fmt_m, fmt_v, lr, beta1,
                                         beta2, eps, weight_decay, step, ws.data_ptr(), nbytes,
                                         _stream(stream))
        _check(rc, "coat_fp8_adamw_step_multi")
        # keep the workspace alive until the launch has run
        torch.cuda.current_stream().synchronize() if stream is None else stream.synchronize()

    def step_static(self, *, fmt_m: int, fmt_v: int, lr: float, beta1: float, beta2: float,
                    eps: float, weight_decay: float, step: int, stream=None) -> None:
        """The same step through the entry point that allocates nothing and
        keeps its tables in the library's own device array (asynchronous)."""
        rc = lib().coat_fp8_adamw_step_multi_static(self.descriptors(), len(self.sizes), self.group, fmt_m,
                                                     fmt_v, lr, beta1, beta2, eps, weight_decay, step,
                                                     _stream(stream))
        _check(rc, "coat_fp8_adamw_step_multi_static")

    # ------------------------------------------------------------ checkpoint
    #
    # The complete optimizer state is the fp32 master weights and the FP8
    # moments with their per-group scales and exponents (plus the step count,
    # which the caller owns). Grads are transient and the bf16 copy is the RNE
    # of the masters, so neither is saved. Stored compressed, as the kernels
    # keep it: 4 + 2 + 24/G bytes per parameter (6.19 at G = 128) against 12
    # for fp32 moments. A resumed run continues bit for bit.

    STATE_FIELDS = ("params", "m_q", "m_s", "m_k", "v_q", "v_s", "v_k")
    CHECKPOINT_FORMAT = "coat-fp8-adamw-state/1"

    def state_dict(self) -> Dict[str, torch.Tensor]:
        """The optimizer state as host tensors (copies of the flat buffers,
        per-tensor padding included). Waits for pending work on the current
        stream."""
        return {name: getattr(self, name).detach().to("cpu", copy=True) for name in self.STATE_FIELDS}

    def load_state_dict(self, sd: Dict[str, torch.Tensor]) -> None:
        """Copy a ``state_dict`` of a list with the same sizes and group size
        into the buffers (the plan stays valid: the buffers do not move)."""
        for name in self.STATE_FIELDS:
            dst = getattr(self, name)
            src = sd[name]
            if src.dtype != dst.dtype or src.shape != dst.shape:
                raise ValueError(f"checkpoint field {name}: {src.dtype} {tuple(src.shape)}, "
                                 f"expected {dst.dtype} {tuple(dst.shape)}")
            dst.copy_(src)

    def save(self, path: str, *, step: int, fmt_m: int, fmt_v: int) -> None:
        """Write the state to a safetensors file; `step` is the last step taken."""
        from safetensors.torch import save_file
        meta = {"format": self.CHECKPOINT_FORMAT, "sizes": json.dumps(self.sizes), "group": str(self.group),
                "step": str(int(step)), "fmt_m": str(int(fmt_m)), "fmt_v": str(int(fmt_v))}
        save_file(self.state_dict(), path, metadata=meta)

    @classmethod
    def load(cls, path: str, device="cuda", with_bf16: bool = True):
        """Rebuild a state from a file written by ``save``. Returns the state
        and the metadata (step, fmt_m, fmt_v as ints). The bf16 copy is not
        stored: it is written again by the next step."""
        from safetensors import safe_open
        with safe_open(path, framework="pt", device="cpu") as f:
            meta = f.metadata() or {}
            if meta.get("format") != cls.CHECKPOINT_FORMAT:
                raise ValueError(f"{path}: not a {cls.CHECKPOINT_FORMAT} checkpoint")
            st = cls(json.loads(meta["sizes"]), int(meta["group"]), device=device, with_bf16=with_bf16)
            st.load_state_dict({name: f.get_tensor(name) for name in cls.STATE_FIELDS})
        return st, {k: int(meta[k]) for k in ("step", "fmt_m", "fmt_v")}

    def quantize_moments(self, m: List[torch.Tensor], v: List[torch.Tensor], *, fmt_m: int, fmt_v: int,
                         stream=None) -> None:
        """Fill the FP8 state from fp32 moments, tensor by tensor."""
        for i in range(len(self.sizes)):
            t = self.tensor(i)
            quantize(m[i], t.m_q, t.m_s, t.m_k, group=self.group, fmt=fmt_m, stream=stream)
            quantize(v[i], t.v_q, t.v_s, t.v_k, group=self.group, fmt=fmt_v, stream=stream)
