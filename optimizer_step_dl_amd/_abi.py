"""ctypes binding of libradamw.so -- argument marshalling only.

Every function here has the name of the C entry point it calls.  Torch is
used for device memory and streams: the binding checks what raw pointers
cannot express (tensor device, dtype, contiguity, element count; FA-zh
"增加的实际能力": non-contiguous, broadcast and mismatched device/queue
inputs are errors), passes ``data_ptr()`` and the current HIP stream, and
raises ``RadamwError`` on a non-zero status.  No arithmetic of the method
happens here, and there is no fallback: without the built library every call
raises.

Page abbreviation: FA-zh = RUDA docs page "实验性融合 AdamW / AMSGrad".
"""
from __future__ import annotations

import ctypes
import os
import sys
from dataclasses import dataclass, field
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libradamw.so")

RADAMW_OK = 0
F32, F16, BF16 = 0, 1, 2
_DTYPE_CODE = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}


class RadamwError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = status_string(status) if _lib is not None else str(status)
        extra = ""
        if status == -6 and _lib is not None:
            extra = f" (hipError {_lib.radamw_last_hip_error()})"
        super().__init__(f"{where}: {msg} [{status}]{extra}")


RADAMW_ERR_DECISION = -7


class DecisionMismatch(RadamwError):
    """RADAMW_ERR_DECISION from a fused step: the host's decision differed
    from the device's, and the step ran as the device decided.  ``result``
    and ``step`` (or ``steps``) are what the call reported, so the caller's
    step counts can follow the state that was written."""

    def __init__(self, where: str, result, step=None, steps=None):
        super().__init__(RADAMW_ERR_DECISION, where)
        self.result, self.step, self.steps = result, step, steps


# ----------------------------------------------------------------- structs --

class Options(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double),
                ("amsgrad", ctypes.c_int32), ("maximize", ctypes.c_int32)]


class Control(ctypes.Structure):
    _fields_ = [("gradient_scale", ctypes.c_double), ("skip_update", ctypes.c_int32)]


class _State(ctypes.Structure):
    _fields_ = [("step", ctypes.c_uint64), ("exp_avg", ctypes.c_void_p),
                ("exp_avg_sq", ctypes.c_void_p), ("max_exp_avg_sq", ctypes.c_void_p)]


class _Segment(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("exp_avg", ctypes.c_void_p),
                ("exp_avg_sq", ctypes.c_void_p), ("max_exp_avg_sq", ctypes.c_void_p),
                ("n", ctypes.c_int64)]


class Stats(ctypes.Structure):
    _fields_ = [("w", ctypes.c_uint32 * 3)]

    @property
    def sumsq(self) -> float:
        return ctypes.c_double.from_buffer_copy(
            (ctypes.c_uint32 * 2)(self.w[0], self.w[1])).value

    @property
    def nonfinite(self) -> int:
        return int(self.w[2])


class FusedResult(ctypes.Structure):
    _fields_ = [("updated", ctypes.c_int32), ("found_inf", ctypes.c_int32),
                ("nonfinite", ctypes.c_uint32), ("reserved", ctypes.c_uint32),
                ("sumsq", ctypes.c_double), ("total_norm", ctypes.c_double),
                ("clip_coef", ctypes.c_double)]


def options(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-5, weight_decay=1e-4, amsgrad=False,
            maximize=False) -> Options:
    return Options(lr, beta1, beta2, eps, weight_decay, int(amsgrad), int(maximize))


def control(gradient_scale=1.0, skip_update=False) -> Control:
    return Control(float(gradient_scale), int(bool(skip_update)))


@dataclass
class AdamWState:
    """Host step count + device moment tensors (the exposed parts of the
    pages' optimizer state).  step == 0 means "no state yet"."""
    step: int = 0
    exp_avg: Optional[torch.Tensor] = None
    exp_avg_sq: Optional[torch.Tensor] = None
    max_exp_avg_sq: Optional[torch.Tensor] = None

    def _c(self) -> _State:
        return _State(self.step, _ptr_or_none(self.exp_avg), _ptr_or_none(self.exp_avg_sq),
                      _ptr_or_none(self.max_exp_avg_sq))


@dataclass
class Segment:
    """One tensor of a multi-tensor in-place update."""
    param: torch.Tensor
    grad: torch.Tensor
    exp_avg: torch.Tensor
    exp_avg_sq: torch.Tensor
    max_exp_avg_sq: Optional[torch.Tensor] = None


# ----------------------------------------------------------------- loading --

_lib = None


def load(path: str = LIB_PATH):
    """Load libradamw.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m optimizer_step_dl_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, u64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_double
    P = ctypes.POINTER
    sig = {
        "radamw_options_default": ([], Options),
        "radamw_step": ([vp, vp, i32, i64, P(_State), vp, P(_State), P(Options), P(Control), vp, P(i32)], ctypes.c_int),
        "radamw_step_inplace": ([vp, vp, i32, i64, P(_State), P(Options), P(Control), vp, P(i32)], ctypes.c_int),
        "radamw_step_multi": ([P(_Segment), i32, i32, P(u64), P(Options), P(Control), vp, P(i32)], ctypes.c_int),
        "radamw_step_staged_inplace": ([vp, vp, i32, i64, P(_State), vp, P(Options), P(Control), vp, P(i32)],
                                       ctypes.c_int),
        "radamw_stream_probe": ([P(vp), i32, P(vp), i32, i64, i32, vp], ctypes.c_int),
        "radamw_bucket_layout": ([i64, P(i32), i32, P(i64), P(i64)], ctypes.c_int),
        "radamw_step_multi_writeback": ([P(_Segment), P(vp), i32, i32, i32, P(u64), P(Options), P(Control), vp,
                                         P(i32)], ctypes.c_int),
        "radamw_stats_plan": ([i64, P(i64), P(i32)], ctypes.c_int),
        "radamw_grad_stats_rows": ([i64, i32], i64),
        "radamw_grad_stats": ([vp, i32, i64, vp, i64, P(i64), vp], ctypes.c_int),
        "radamw_merge_stats": ([vp, i64, vp, i64, vp, i32, vp], ctypes.c_int),
        "radamw_read_report": ([vp, P(Stats), vp], ctypes.c_int),
        "radamw_decide": ([P(Stats), dbl, dbl, P(Control), P(FusedResult)], ctypes.c_int),
        "radamw_check_decision": ([P(Stats), P(ctypes.c_uint32), dbl, dbl, P(FusedResult)], ctypes.c_int),
        "radamw_fused_workspace_bytes": ([P(_Segment), i32, i32], i64),
        "radamw_fused_step_multi": ([P(_Segment), i32, i32, P(u64), P(Options), dbl, dbl, i32, vp, i64, vp,
                                     P(FusedResult)], ctypes.c_int),
        "radamw_fused_step_multi_noalloc": ([P(_Segment), i32, i32, P(u64), P(Options), dbl, dbl, i32, vp,
                                             P(FusedResult)], ctypes.c_int),
        "radamw_host_coefficients": ([P(Options), u64, dbl, P(ctypes.c_float)], ctypes.c_int),
        "radamw_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "radamw_last_hip_error": ([], ctypes.c_int),
        "radamw_launch_count": ([], u64),
        "radamw_time_next_update": ([vp, vp], ctypes.c_int),
        "radamw_list_create": ([P(_Segment), i32, i32, i32, P(vp), i32, vp, P(vp)], ctypes.c_int),
        "radamw_list_step": ([vp, P(u64), P(Options), P(Control), vp, P(i32)], ctypes.c_int),
        "radamw_list_fused_step": ([vp, P(u64), P(Options), dbl, dbl, i32, vp, P(FusedResult)], ctypes.c_int),
        "radamw_list_destroy": ([vp], ctypes.c_int),
        "radamw_lists_fused_step": ([P(vp), i32, P(u64), P(Options), dbl, dbl, i32, vp, P(FusedResult)],
                                    ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


EXPORTS = ("radamw_options_default", "radamw_step", "radamw_step_inplace", "radamw_step_multi",
           "radamw_step_staged_inplace", "radamw_stream_probe", "radamw_bucket_layout", "radamw_step_multi_writeback",
           "radamw_stats_plan", "radamw_grad_stats_rows", "radamw_grad_stats", "radamw_merge_stats",
           "radamw_read_report", "radamw_decide", "radamw_check_decision", "radamw_fused_workspace_bytes",
           "radamw_fused_step_multi", "radamw_fused_step_multi_noalloc", "radamw_host_coefficients", "radamw_status_string",
           "radamw_last_hip_error", "radamw_launch_count", "radamw_time_next_update",
           "radamw_list_create", "radamw_list_step", "radamw_list_fused_step", "radamw_list_destroy",
           "radamw_lists_fused_step")


# ----------------------------------------------------------------- helpers --

def _ptr_or_none(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _check(rc: int, where: str):
    if rc != RADAMW_OK:
        raise RadamwError(rc, where)


def _stream(device: torch.device):
    return torch.cuda.current_stream(device).cuda_stream


def _dense(t: torch.Tensor, what: str, dtype=None, numel=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{what} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{what} must be {dtype} (got {t.dtype})")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{what} has {t.numel()} elements, expected {numel}")
    if device is not None and t.device != device:
        raise ValueError(f"{what} is on {t.device}, expected {device}")
    return t


def _grad_code(g: torch.Tensor) -> int:
    if g.dtype not in _DTYPE_CODE:
        raise ValueError(f"gradient dtype {g.dtype} is not float32/float16/bfloat16")
    return _DTYPE_CODE[g.dtype]


def _check_fast(t: torch.Tensor, what: str, dev_index: int, numel: int, dtype=None):
    """Cheap form of _dense for long tensor lists (same checks)."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if t.get_device() != dev_index:
        raise ValueError(f"{what} is on device {t.get_device()}, expected {dev_index}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{what} has {t.numel()} elements, expected {numel}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{what} must be {dtype} (got {t.dtype})")


def _segments(segs: Sequence[Segment], amsgrad: bool):
    arr = (_Segment * max(1, len(segs)))()
    code = None
    dev_index = None
    f32 = torch.float32
    for i, s in enumerate(segs):
        p = s.param
        if dev_index is None:
            if not isinstance(p, torch.Tensor) or not p.is_cuda:
                raise ValueError(f"segment {i} param must be a device tensor")
            dev_index = p.get_device()
        n = p.numel()
        _check_fast(p, f"segment {i} param", dev_index, n, f32)
        _check_fast(s.grad, f"segment {i} grad", dev_index, n)
        c = _grad_code(s.grad)
        if code is not None and c != code:
            raise ValueError("all gradients of one call must share a dtype")
        code = c
        _check_fast(s.exp_avg, f"segment {i} exp_avg", dev_index, n, f32)
        _check_fast(s.exp_avg_sq, f"segment {i} exp_avg_sq", dev_index, n, f32)
        if s.max_exp_avg_sq is not None:
            _check_fast(s.max_exp_avg_sq, f"segment {i} max_exp_avg_sq", dev_index, n, f32)
        arr[i] = _Segment(p.data_ptr(), s.grad.data_ptr(), s.exp_avg.data_ptr(),
                          s.exp_avg_sq.data_ptr(), _ptr_or_none(s.max_exp_avg_sq), n)
    device = torch.device("cuda", torch.cuda.current_device() if dev_index is None else dev_index)
    return arr, (F32 if code is None else code), device


class SegmentList:
    """A tensor list marshalled once, for repeated multi-tensor steps over
    the same tensors (optimizer state and parameters normally keep their
    storage for a whole run).  Holds references to the tensors; the C entry
    points still validate every pointer on each call."""

    def __init__(self, segments: Sequence[Segment]):
        self.segments = list(segments)
        self.array, self.code, self.device = _segments(self.segments, False)

    def __len__(self):
        return len(self.segments)


def _marshal(segments):
    if isinstance(segments, SegmentList):
        return segments.array, segments.code, segments.device, len(segments)
    arr, code, dev = _segments(segments, False)
    return arr, code, dev, len(segments)


# ------------------------------------------------------------- entry points --

def radamw_options_default() -> Options:
    return load().radamw_options_default()


def radamw_step(param: torch.Tensor, grad: torch.Tensor, state: AdamWState, opts: Options,
                ctrl: Control, out_param: torch.Tensor, out_state: AdamWState) -> bool:
    """Out-of-place update: writes out_param/out_state, never the inputs.
    Returns True when launched (then out_state.step = state.step + 1)."""
    lib = load()
    dev = param.device
    n = param.numel()
    _dense(param, "param", torch.float32)
    _dense(grad, "grad", numel=n, device=dev)
    _dense(out_param, "out_param", torch.float32, n, dev)
    for name in ("exp_avg", "exp_avg_sq", "max_exp_avg_sq"):
        t = getattr(out_state, name)
        if t is not None:
            _dense(t, f"out_state.{name}", torch.float32, n, dev)
        t = getattr(state, name)
        if t is not None and state.step > 0:
            _dense(t, f"state.{name}", torch.float32, n, dev)
    cin, cout = state._c(), out_state._c()
    updated = ctypes.c_int32(0)
    with torch.cuda.device(dev):
        rc = lib.radamw_step(param.data_ptr(), grad.data_ptr(), _grad_code(grad), n, ctypes.byref(cin),
                             out_param.data_ptr(), ctypes.byref(cout), ctypes.byref(opts), ctypes.byref(ctrl),
                             _stream(dev), ctypes.byref(updated))
    _check(rc, "radamw_step")
    if updated.value:
        out_state.step = cout.step
    return bool(updated.value)


def radamw_step_inplace(param: torch.Tensor, grad: torch.Tensor, state: AdamWState, opts: Options,
                        ctrl: Control) -> bool:
    """In-place update of param and state; state.step advances on launch."""
    lib = load()
    dev = param.device
    n = param.numel()
    _dense(param, "param", torch.float32)
    _dense(grad, "grad", numel=n, device=dev)
    for name in ("exp_avg", "exp_avg_sq", "max_exp_avg_sq"):
        t = getattr(state, name)
        if t is not None:
            _dense(t, f"state.{name}", torch.float32, n, dev)
    cst = state._c()
    updated = ctypes.c_int32(0)
    with torch.cuda.device(dev):
        rc = lib.radamw_step_inplace(param.data_ptr(), grad.data_ptr(), _grad_code(grad), n,
                                     ctypes.byref(cst), ctypes.byref(opts), ctypes.byref(ctrl),
                                     _stream(dev), ctypes.byref(updated))
    _check(rc, "radamw_step_inplace")
    state.step = cst.step
    return bool(updated.value)


def radamw_step_staged_inplace(param: torch.Tensor, grad: torch.Tensor, state: AdamWState, delta: torch.Tensor,
                               opts: Options, ctrl: Control) -> bool:
    """The staged (unfused, 4 or 5 launches) baseline, in place; delta is an
    FP32 scratch tensor of the same size.  For measurement."""
    lib = load()
    dev = param.device
    n = param.numel()
    _dense(param, "param", torch.float32)
    _dense(grad, "grad", numel=n, device=dev)
    _dense(delta, "delta", torch.float32, n, dev)
    for name in ("exp_avg", "exp_avg_sq", "max_exp_avg_sq"):
        t = getattr(state, name)
        if t is not None:
            _dense(t, f"state.{name}", torch.float32, n, dev)
    cst = state._c()
    updated = ctypes.c_int32(0)
    with torch.cuda.device(dev):
        rc = lib.radamw_step_staged_inplace(param.data_ptr(), grad.data_ptr(), _grad_code(grad), n,
                                            ctypes.byref(cst), delta.data_ptr(), ctypes.byref(opts),
                                            ctypes.byref(ctrl), _stream(dev), ctypes.byref(updated))
    _check(rc, "radamw_step_staged_inplace")
    state.step = cst.step
    return bool(updated.value)


def radamw_stream_probe(ins: Sequence[torch.Tensor], outs: Sequence[torch.Tensor], cap_per_cu: int = 0,
                        sink: Optional[torch.Tensor] = None) -> None:
    """Streaming ceiling (measurement only): len(ins) FP32 read streams and
    len(outs) write streams with the update kernel's geometry;
    outs[w] = sum(ins) + w.  With no output, ``sink`` (an FP32 tensor of the
    streams' size) is the never-written sink."""
    lib = load()
    tensors = list(ins) + list(outs) + ([] if sink is None else [sink])
    if not tensors:
        raise ValueError("at least one stream")
    dev = tensors[0].device
    n = tensors[0].numel()
    for i, t in enumerate(tensors):
        _dense(t, f"stream {i}", torch.float32, n, dev)
    # an output given as one of the inputs is updated in place
    if not outs and sink is None:
        raise ValueError("a read-only probe needs a sink tensor")
    pin = (ctypes.c_void_p * max(1, len(ins)))(*[t.data_ptr() for t in ins])
    wr = list(outs) if outs else [sink]
    pout = (ctypes.c_void_p * len(wr))(*[t.data_ptr() for t in wr])
    with torch.cuda.device(dev):
        rc = lib.radamw_stream_probe(pin, len(ins), pout, len(outs), n, int(cap_per_cu), _stream(dev))
    _check(rc, "radamw_stream_probe")


def radamw_bucket_layout(n: int, element_bytes: Sequence[int]):
    """(byte offsets, arena bytes) of the library's placement for the
    streams of one flattened bucket in a single allocation."""
    k = len(element_bytes)
    eb = (ctypes.c_int32 * max(1, k))(*[int(x) for x in element_bytes])
    offs = (ctypes.c_int64 * max(1, k))()
    total = ctypes.c_int64()
    _check(load().radamw_bucket_layout(int(n), eb, k, offs, ctypes.byref(total)), "radamw_bucket_layout")
    return [int(offs[i]) for i in range(k)], int(total.value)


_PITCH_ALIGN = 2 << 20


def bucket_arena(n: int, dtypes: Sequence[torch.dtype], device=None):
    """One device allocation holding len(dtypes) streams of n elements, placed
    by radamw_bucket_layout (from a 2 MiB-aligned start).  Returns the views,
    in order; each keeps the allocation alive."""
    device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    sizes = [torch.empty(0, dtype=d).element_size() for d in dtypes]
    offs, total = radamw_bucket_layout(n, sizes)
    raw = torch.empty(total + _PITCH_ALIGN, dtype=torch.uint8, device=device)
    lead = (-raw.data_ptr()) % _PITCH_ALIGN
    return [raw[lead + o:lead + o + n * es].view(d) for o, es, d in zip(offs, sizes, dtypes)]


def bucket_segment(n: int, grad_dtype: torch.dtype = torch.float32, amsgrad: bool = False, device=None) -> Segment:
    """A flattened bucket's p, gradient, m, v (and v_max) as one allocation
    in the library's placement (bucket_arena); contents uninitialised."""
    f32 = torch.float32
    dts = [f32, grad_dtype, f32, f32] + ([f32] if amsgrad else [])
    views = bucket_arena(n, dts, device)
    return Segment(views[0], views[1], views[2], views[3], views[4] if amsgrad else None)


def radamw_step_multi(segments, step: int, opts: Options, ctrl: Control):
    """In-place update of a tensor list (a sequence of Segment or a
    SegmentList) sharing options and step count.  Returns (updated, new_step)."""
    lib = load()
    arr, code, dev, count = _marshal(segments)
    st = ctypes.c_uint64(step)
    updated = ctypes.c_int32(0)
    with torch.cuda.device(dev):
        rc = lib.radamw_step_multi(arr, count, code, ctypes.byref(st), ctypes.byref(opts),
                                   ctypes.byref(ctrl), _stream(dev), ctypes.byref(updated))
    _check(rc, "radamw_step_multi")
    return bool(updated.value), int(st.value)


def _models(models, segs, dev):
    """Host array of model-copy pointers (None entries stay NULL) and their
    shared dtype."""
    mdt = None
    ptrs = (ctypes.c_void_p * max(1, len(segs)))()
    for i, (m, s) in enumerate(zip(models, segs)):
        if m is None:
            continue
        _dense(m, f"model copy {i}", numel=s.param.numel(), device=dev)
        if m.dtype not in (torch.float16, torch.bfloat16) or (mdt is not None and m.dtype != mdt):
            raise ValueError("model copies must all be float16 or all bfloat16")
        mdt = m.dtype
        ptrs[i] = m.data_ptr()
    return ptrs, mdt


def radamw_step_multi_writeback(segments, models: Sequence[Optional[torch.Tensor]], step: int, opts: Options,
                                ctrl: Control):
    """radamw_step_multi plus a 16-bit model copy per tensor, written in the
    same pass.  models[i] is a float16 / bfloat16 tensor of segments[i]'s
    size, or None; all copies share one dtype.  Returns (updated, new_step)."""
    lib = load()
    arr, code, dev, count = _marshal(segments)
    if len(models) != count:
        raise ValueError("one model entry (tensor or None) per segment")
    segs = segments.segments if isinstance(segments, SegmentList) else segments
    ptrs, mdt = _models(models, segs, dev)
    st = ctypes.c_uint64(step)
    updated = ctypes.c_int32(0)
    with torch.cuda.device(dev):
        rc = lib.radamw_step_multi_writeback(arr, ptrs, count, code, _DTYPE_CODE[mdt or torch.bfloat16],
                                             ctypes.byref(st), ctypes.byref(opts), ctypes.byref(ctrl), _stream(dev),
                                             ctypes.byref(updated))
    _check(rc, "radamw_step_multi_writeback")
    return bool(updated.value), int(st.value)


def radamw_stats_plan(rows: int):
    """(scratch_elements, extra_merge_kernels) for ``rows`` records."""
    se, ex = ctypes.c_int64(), ctypes.c_int32()
    _check(load().radamw_stats_plan(rows, ctypes.byref(se), ctypes.byref(ex)), "radamw_stats_plan")
    return se.value, ex.value


def radamw_grad_stats_rows(n: int, dtype: torch.dtype) -> int:
    r = load().radamw_grad_stats_rows(n, _DTYPE_CODE[dtype])
    if r < 0:
        raise RadamwError(int(r), "radamw_grad_stats_rows")
    return int(r)


def radamw_grad_stats(grad: torch.Tensor, rows: torch.Tensor, row_offset: int = 0) -> int:
    """Analyse ``grad`` into records rows[row_offset:]; ``rows`` is an int32
    tensor of 3 * capacity words.  Returns the number of records written."""
    lib = load()
    dev = grad.device
    _dense(grad, "grad")
    _dense(rows, "rows", torch.int32, device=dev)
    cap = rows.numel() // 3 - row_offset
    written = ctypes.c_int64(0)
    with torch.cuda.device(dev):
        rc = lib.radamw_grad_stats(grad.data_ptr(), _grad_code(grad), grad.numel(),
                                   rows.data_ptr() + 12 * row_offset, cap, ctypes.byref(written),
                                   _stream(dev))
    _check(rc, "radamw_grad_stats")
    return int(written.value)


def radamw_merge_stats(rows: torch.Tensor, nrows: int, scratch: Optional[torch.Tensor],
                       report: torch.Tensor, hierarchical: bool = True) -> None:
    lib = load()
    dev = rows.device
    _dense(rows, "rows", torch.int32)
    _dense(report, "report", torch.int32, 3, dev)
    if scratch is not None:
        _dense(scratch, "scratch", torch.float32, device=dev)
    with torch.cuda.device(dev):
        rc = lib.radamw_merge_stats(rows.data_ptr(), nrows, _ptr_or_none(scratch),
                                    0 if scratch is None else scratch.numel(), report.data_ptr(),
                                    int(bool(hierarchical)), _stream(dev))
    _check(rc, "radamw_merge_stats")


def radamw_read_report(report: torch.Tensor) -> Stats:
    lib = load()
    _dense(report, "report", torch.int32, 3)
    out = Stats()
    with torch.cuda.device(report.device):
        rc = lib.radamw_read_report(report.data_ptr(), ctypes.byref(out), _stream(report.device))
    _check(rc, "radamw_read_report")
    return out


def radamw_decide(host_report: Stats, gradient_scale: float, max_grad_norm: Optional[float]):
    """(Control, FusedResult) of the host decision for a read-back report."""
    ctrl, res = Control(), FusedResult()
    rc = load().radamw_decide(ctypes.byref(host_report), float(gradient_scale),
                              0.0 if max_grad_norm is None else float(max_grad_norm),
                              ctypes.byref(ctrl), ctypes.byref(res))
    _check(rc, "radamw_decide")
    return ctrl, res


def radamw_check_decision(host_report: Stats, device_skip: int, device_inv_scale_bits: int,
                          gradient_scale: float, max_grad_norm: Optional[float]):
    """(agree, FusedResult): the host's decision from ``host_report`` against
    a device decision {skip, bits of the FP32 unscale factor}; the result's
    ``updated`` follows the device's."""
    dec = (ctypes.c_uint32 * 2)(int(device_skip) & 0xffffffff, int(device_inv_scale_bits) & 0xffffffff)
    res = FusedResult()
    rc = load().radamw_check_decision(ctypes.byref(host_report), dec, float(gradient_scale),
                                      0.0 if max_grad_norm is None else float(max_grad_norm), ctypes.byref(res))
    if rc not in (RADAMW_OK, RADAMW_ERR_DECISION):
        _check(rc, "radamw_check_decision")
    return rc == RADAMW_OK, res


def radamw_fused_workspace_bytes(segments) -> int:
    arr, code, _, count = _marshal(segments)
    r = load().radamw_fused_workspace_bytes(arr, count, code)
    if r < 0:
        raise RadamwError(int(r), "radamw_fused_workspace_bytes")
    return int(r)


def radamw_fused_step_multi(segments, step: int, opts: Options,
                            gradient_scale: float, max_grad_norm: Optional[float],
                            hierarchical: bool, workspace: Optional[torch.Tensor]):
    """Statistics -> merge -> read-back -> decision -> one update launch.
    Returns (FusedResult, new_step)."""
    lib = load()
    arr, code, dev, count = _marshal(segments)
    if workspace is not None:
        _dense(workspace, "workspace", device=dev)
    st = ctypes.c_uint64(step)
    res = FusedResult()
    with torch.cuda.device(dev):
        rc = lib.radamw_fused_step_multi(
            arr, count, code, ctypes.byref(st), ctypes.byref(opts), float(gradient_scale),
            0.0 if max_grad_norm is None else float(max_grad_norm), int(bool(hierarchical)),
            _ptr_or_none(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
            _stream(dev), ctypes.byref(res))
    if rc == RADAMW_ERR_DECISION:
        raise DecisionMismatch("radamw_fused_step_multi", res, step=int(st.value))
    _check(rc, "radamw_fused_step_multi")
    return res, int(st.value)


def radamw_fused_step_multi_noalloc(segments, step: int, opts: Options, gradient_scale: float,
                                    max_grad_norm: Optional[float], hierarchical: bool):
    """radamw_fused_step_multi over one flattened bucket (at most one
    segment) with no workspace: the library's static device scratch holds
    the statistics, so the call allocates nothing.  Returns when the step has
    completed.  Returns (FusedResult, new_step)."""
    lib = load()
    arr, code, dev, count = _marshal(segments)
    st = ctypes.c_uint64(step)
    res = FusedResult()
    with torch.cuda.device(dev):
        rc = lib.radamw_fused_step_multi_noalloc(
            arr, count, code, ctypes.byref(st), ctypes.byref(opts), float(gradient_scale),
            0.0 if max_grad_norm is None else float(max_grad_norm), int(bool(hierarchical)), _stream(dev),
            ctypes.byref(res))
    if rc == RADAMW_ERR_DECISION:
        raise DecisionMismatch("radamw_fused_step_multi_noalloc", res, step=int(st.value))
    _check(rc, "radamw_fused_step_multi_noalloc")
    return res, int(st.value)


class TensorList:
    """A persistent tensor list (radamw_list_create): the segments are
    validated once and their launch tables kept in device memory, so each
    step only launches.  The list holds a reference to every tensor it was
    built from, so their storage stays allocated while it lives; a gradient
    that moves to a new tensor needs a new list.  ``models`` optionally
    gives a float16 / bfloat16 model copy per segment (or None), rewritten
    by every update.  Free it with close() (or a ``with`` block)."""

    def __init__(self, segments, amsgrad: bool, models: Optional[Sequence[Optional[torch.Tensor]]] = None):
        lib = load()
        self.segments = list(segments.segments if isinstance(segments, SegmentList) else segments)
        arr, code, dev = _segments(self.segments, False)
        self.device, self.code, self.amsgrad = dev, code, bool(amsgrad)
        self.models = None if models is None else list(models)
        ptrs, mdt = None, None
        if self.models is not None:
            if len(self.models) != len(self.segments):
                raise ValueError("one model entry (tensor or None) per segment")
            ptrs, mdt = _models(self.models, self.segments, dev)
        handle = ctypes.c_void_p()
        with torch.cuda.device(dev):
            rc = lib.radamw_list_create(arr, len(self.segments), code, int(self.amsgrad), ptrs,
                                        _DTYPE_CODE[mdt or torch.bfloat16], _stream(dev), ctypes.byref(handle))
        _check(rc, "radamw_list_create")
        self._handle = handle

    def _live(self):
        if self._handle is None:
            raise RuntimeError("the tensor list was closed")
        return self._handle

    def step(self, step: int, opts: Options, ctrl: Control):
        """radamw_step_multi over the list.  Returns (updated, new_step)."""
        st = ctypes.c_uint64(step)
        updated = ctypes.c_int32(0)
        with torch.cuda.device(self.device):
            rc = load().radamw_list_step(self._live(), ctypes.byref(st), ctypes.byref(opts), ctypes.byref(ctrl),
                                         _stream(self.device), ctypes.byref(updated))
        _check(rc, "radamw_list_step")
        return bool(updated.value), int(st.value)

    def fused_step(self, step: int, opts: Options, gradient_scale: float, max_grad_norm: Optional[float],
                   hierarchical: bool):
        """radamw_fused_step_multi over the list.  Returns (FusedResult, new_step)."""
        st = ctypes.c_uint64(step)
        res = FusedResult()
        with torch.cuda.device(self.device):
            rc = load().radamw_list_fused_step(self._live(), ctypes.byref(st), ctypes.byref(opts),
                                               float(gradient_scale),
                                               0.0 if max_grad_norm is None else float(max_grad_norm),
                                               int(bool(hierarchical)), _stream(self.device), ctypes.byref(res))
        if rc == RADAMW_ERR_DECISION:
            raise DecisionMismatch("radamw_list_fused_step", res, step=int(st.value))
        _check(rc, "radamw_list_fused_step")
        return res, int(st.value)

    def close(self):
        if getattr(self, "_handle", None) is not None:
            h, self._handle = self._handle, None
            _check(load().radamw_list_destroy(h), "radamw_list_destroy")

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        if getattr(self, "_handle", None) is not None and not sys.is_finalizing():
            try:
                self.close()
            except Exception:
                pass

    def __len__(self):
        return len(self.segments)


def radamw_list_create(segments, amsgrad: bool, models=None) -> TensorList:
    return TensorList(segments, amsgrad, models)


def radamw_list_step(lst: TensorList, step: int, opts: Options, ctrl: Control):
    return lst.step(step, opts, ctrl)


def radamw_list_fused_step(lst: TensorList, step: int, opts: Options, gradient_scale: float,
                           max_grad_norm: Optional[float], hierarchical: bool):
    return lst.fused_step(step, opts, gradient_scale, max_grad_norm, hierarchical)


def radamw_list_destroy(lst: TensorList) -> None:
    lst.close()


def radamw_lists_fused_step(lists: Sequence[TensorList], steps: Sequence[int], opts: Sequence[Options],
                            gradient_scale: float, max_grad_norm: Optional[float], hierarchical: bool):
    """One fused step over several lists (parameter groups): one statistics
    reduction and one decision, then each list's update with its own options
    and step count.  Returns (FusedResult, new_steps)."""
    k = len(lists)
    if len(steps) != k or len(opts) != k or k == 0:
        raise ValueError("one step count and one options struct per list")
    dev = lists[0].device
    handles = (ctypes.c_void_p * k)(*[lst._live().value for lst in lists])
    st = (ctypes.c_uint64 * k)(*[int(x) for x in steps])
    op = (Options * k)(*opts)
    res = FusedResult()
    with torch.cuda.device(dev):
        rc = load().radamw_lists_fused_step(handles, k, st, op, float(gradient_scale),
                                            0.0 if max_grad_norm is None else float(max_grad_norm),
                                            int(bool(hierarchical)), _stream(dev), ctypes.byref(res))
    if rc == RADAMW_ERR_DECISION:
        raise DecisionMismatch("radamw_lists_fused_step", res, steps=[int(x) for x in st])
    _check(rc, "radamw_lists_fused_step")
    return res, [int(x) for x in st]


def radamw_host_coefficients(opts: Options, t: int, gradient_scale: float = 1.0) -> list[float]:
    out = (ctypes.c_float * 9)()
    _check(load().radamw_host_coefficients(ctypes.byref(opts), t, float(gradient_scale), out),
           "radamw_host_coefficients")
    return list(out)


def radamw_status_string(status: int) -> str:
    return load().radamw_status_string(status).decode()


status_string = radamw_status_string


def radamw_last_hip_error() -> int:
    return load().radamw_last_hip_error()


def radamw_launch_count() -> int:
    return int(load().radamw_launch_count())


def radamw_time_next_update(start: Optional["torch.cuda.Event"], stop: Optional["torch.cuda.Event"]) -> None:
    """Record torch events at the first update kernel's start and the last
    one's end in the next launching update call on this thread.  The events
    must already exist on the device (recorded once)."""
    load().radamw_time_next_update(None if start is None else start.cuda_event,
                                   None if stop is None else stop.cuda_event)
