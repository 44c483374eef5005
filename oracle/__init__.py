"""Reference oracle for the fused AdamW / AMSGrad step -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (``libradamw.so`` and
``optimizer_step_dl_amd``) never imports or calls it, and it imports nothing
from the product path.

The arithmetic lives in ``radamw_oracle.c`` (plain scalar C, FP32 as the pages
fix it, FP64 host coefficients); this module only marshals numpy arrays into
it.  ``brute64`` is an independent float64 restatement used to pin the C code.

Page abbreviations: FA-ja = RUDA docs page "実験的なデバイス上の融合 AdamW /
AMSGrad"; FA-zh = "实验性融合 AdamW / AMSGrad"; TR-zh = "训练与状态保存".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "radamw_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, F16, BF16 = 0, 1, 2
DTYPE_CODES = {"f32": F32, "f16": F16, "bf16": BF16}

GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
             "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(quiet: bool = True) -> str:
    """Compile radamw_oracle.c into liboracle.so with gcc (no fusion, no fast-math)."""
    cmd = ["gcc", *GCC_FLAGS, "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True, capture_output=quiet)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


class _Options(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double),
                ("beta2", ctypes.c_double), ("eps", ctypes.c_double),
                ("weight_decay", ctypes.c_double),
                ("amsgrad", ctypes.c_int32), ("maximize", ctypes.c_int32)]


class _Coefs(ctypes.Structure):
    _fields_ = [(name, ctypes.c_float) for name in
                ("beta1", "one_minus_beta1", "beta2", "one_minus_beta2",
                 "bc1", "bc2", "lr", "eps", "decay")]


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, u64p = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(ctypes.c_uint64)
    lib.oracle_coefficients.argtypes = [ctypes.POINTER(_Options), ctypes.c_uint64, ctypes.POINTER(_Coefs)]
    lib.oracle_coefficients.restype = None
    lib.oracle_widen.argtypes = [vp, i32, i64]
    lib.oracle_widen.restype = ctypes.c_float
    lib.oracle_adamw_step.argtypes = [vp, vp, i32, i64, vp, vp, vp, u64p,
                                      ctypes.POINTER(_Options), ctypes.c_double, i32]
    lib.oracle_adamw_step.restype = i32
    lib.oracle_grad_stats_accumulate.argtypes = [vp, i32, i64, ctypes.POINTER(ctypes.c_double),
                                                 ctypes.POINTER(ctypes.c_uint32)]
    lib.oracle_grad_stats_accumulate.restype = None
    lib.oracle_stats_plan.argtypes = [i64, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)]
    lib.oracle_stats_plan.restype = i32
    lib.oracle_clip_coefficient.argtypes = [ctypes.c_double] * 3
    lib.oracle_clip_coefficient.restype = ctypes.c_double
    lib.oracle_round_copy.argtypes = [vp, i64, i32, vp]
    lib.oracle_round_copy.restype = None
    _lib = lib
    return lib


@dataclass
class Options:
    """Hyper-parameters of one update.  Defaults follow FA-ja
    "この演算子を使用する理由" (betas, epsilon, weight decay); the pages print
    no learning-rate default, 1e-3 is the value of their usage examples."""
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-5
    weight_decay: float = 1e-4
    amsgrad: bool = False
    maximize: bool = False

    def _c(self) -> _Options:
        return _Options(self.lr, self.beta1, self.beta2, self.eps, self.weight_decay,
                        int(self.amsgrad), int(self.maximize))


def coefficients(opts: Options, t: int) -> dict:
    """FP32 coefficients of update t (FP64 integer power, then cast)."""
    c = _Coefs()
    _load().oracle_coefficients(ctypes.byref(opts._c()), t, ctypes.byref(c))
    return {name: np.float32(getattr(c, name)) for name, _ in _Coefs._fields_}


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _grad_code(grad: np.ndarray, dtype: str | int) -> int:
    code = DTYPE_CODES[dtype] if isinstance(dtype, str) else int(dtype)
    want = np.float32 if code == F32 else np.uint16
    if code == F16 and grad.dtype == np.float16:
        return code
    assert grad.dtype == want, (grad.dtype, dtype)
    return code


class State:
    """Host copy of the optimizer state: the completed-step count and the
    moment arrays (the exposed parts of FA-ja "低レベルの使用")."""

    def __init__(self, n: int, amsgrad: bool):
        self.step = 0
        self.exp_avg = np.zeros(n, np.float32)
        self.exp_avg_sq = np.zeros(n, np.float32)
        self.max_exp_avg_sq = np.zeros(n, np.float32) if amsgrad else None

    def copy(self) -> "State":
        s = State.__new__(State)
        s.step = self.step
        s.exp_avg = self.exp_avg.copy()
        s.exp_avg_sq = self.exp_avg_sq.copy()
        s.max_exp_avg_sq = None if self.max_exp_avg_sq is None else self.max_exp_avg_sq.copy()
        return s


def adamw_step(param: np.ndarray, grad: np.ndarray, gdt, state: State, opts: Options,
               gradient_scale: float = 1.0, skip_update: bool = False) -> bool:
    """One update in place on ``param`` and ``state`` (numpy, C-contiguous).

    ``grad`` is float32 for "f32", float16 or raw uint16 bits for "f16", raw
    uint16 bits for "bf16".  Returns True when the update ran."""
    lib = _load()
    code = _grad_code(grad, gdt)
    n = param.size
    assert param.dtype == np.float32 and grad.size == n
    assert state.exp_avg.size == n and state.exp_avg_sq.size == n
    if opts.amsgrad:
        assert state.max_exp_avg_sq is not None and state.max_exp_avg_sq.size == n
    step = ctypes.c_uint64(state.step)
    ran = lib.oracle_adamw_step(_ptr(param), _ptr(grad), code, n, _ptr(state.exp_avg),
                                _ptr(state.exp_avg_sq),
                                _ptr(state.max_exp_avg_sq) if opts.amsgrad else None,
                                ctypes.byref(step), ctypes.byref(opts._c()),
                                float(gradient_scale), int(bool(skip_update)))
    state.step = step.value
    return bool(ran)


def widen(grad: np.ndarray, gdt) -> np.ndarray:
    """FP32 values of a stored gradient (element by element through the C decoder)."""
    lib = _load()
    code = _grad_code(grad, gdt)
    out = np.empty(grad.size, np.float32)
    p = _ptr(grad)
    for i in range(grad.size):
        out[i] = lib.oracle_widen(p, code, i)
    return out


class StatsAccumulator:
    """Running (sum of squares, non-finite count) over a sequence of tensors."""

    def __init__(self):
        self.sumsq = ctypes.c_double(0.0)
        self.nonfinite = ctypes.c_uint32(0)

    def add(self, grad: np.ndarray, gdt) -> "StatsAccumulator":
        code = _grad_code(grad, gdt)
        _load().oracle_grad_stats_accumulate(_ptr(grad), code, grad.size,
                                             ctypes.byref(self.sumsq), ctypes.byref(self.nonfinite))
        return self

    @property
    def result(self) -> tuple[float, int]:
        return self.sumsq.value, self.nonfinite.value


def grad_stats(grad: np.ndarray, gdt) -> tuple[float, int]:
    """(sum of squares of finite values, non-finite count) of one stored gradient."""
    return StatsAccumulator().add(grad, gdt).result


def stats_plan(rows: int):
    """(scratch_elements, extra_merge_kernels), or None when rows is out of range."""
    se, ex = ctypes.c_int64(), ctypes.c_int32()
    rc = _load().oracle_stats_plan(rows, ctypes.byref(se), ctypes.byref(ex))
    return None if rc != 0 else (se.value, ex.value)


def clip_coefficient(sumsq: float, gradient_scale: float, max_norm: float | None) -> float:
    return _load().oracle_clip_coefficient(sumsq, gradient_scale,
                                           0.0 if max_norm is None else float(max_norm))


def decide(sumsq: float, nonfinite: int, gradient_scale: float, max_norm: float | None):
    """The host decision after the report is read back: (skip, effective_scale).

    A non-finite count above zero skips the whole step (TR-zh "在 ruda:0 上进行
    原生 PyTorch 训练"); otherwise the clip coefficient is folded into the scale."""
    if nonfinite > 0:
        return True, gradient_scale
    return False, gradient_scale / clip_coefficient(sumsq, gradient_scale, max_norm)


def round_copy(p: np.ndarray, dtype) -> np.ndarray:
    """The FP16 / BF16 model copy of FP32 values (raw uint16 bits), rounded to
    nearest even (the FP32-master write-back)."""
    code = DTYPE_CODES[dtype] if isinstance(dtype, str) else int(dtype)
    assert code in (F16, BF16) and p.dtype == np.float32 and p.flags["C_CONTIGUOUS"]
    out = np.empty(p.size, np.uint16)
    _load().oracle_round_copy(_ptr(p), p.size, code, _ptr(out))
    return out
