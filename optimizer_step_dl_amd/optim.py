"""FusedAdamW -- a torch.optim.Optimizer over libradamw.so.

Page abbreviations: TR-zh = RUDA docs page "训练与状态保存" (section
"在 ruda:0 上进行原生 PyTorch 训练" describes the native-PyTorch optimizer this
mirrors); FA-ja = "実験的なデバイス上の融合 AdamW / AMSGrad".

Behaviour (TR-zh):
  * ``fused_step=True`` turns on the read-only gradient analysis: before any
    parameter is updated, the statistics of every active gradient are
    reduced to one 12-byte report that is read back to the host; a
    non-finite value anywhere skips the whole step (no update, no step
    increment).  ``hierarchical_stats=True`` reduces the statistics with the
    fan-in-1024 merge levels; ``max_grad_norm`` clips the global L2 norm of
    the unscaled gradients of all active groups and requires
    ``fused_step=True``.  Both booleans default to False, clipping to None.
  * ``.grad`` is kept (the caller clears it before the next accumulation
    window); master parameters and moments are FP32.  ``model_copies`` maps
    master parameters to float16 / bfloat16 model tensors that the update
    rewrites in the same pass (the low-precision write-back an FP32-master
    optimizer performs).
  * ``state_dict()`` records the step options; with hierarchical statistics
    the options carry version 2.  An archive without step options restores
    with the fused and hierarchical modes off.

All arithmetic runs in the library's kernels; this class only groups
tensors (by parameter group and by step count, since one launch shares one
step count) and sequences the C entry points.  Parameters must be FP32
device tensors; gradients FP32, FP16 or BF16 of the same shape.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional

import torch

from . import _abi

STEP_OPTIONS_VERSION_FLAT = 1
STEP_OPTIONS_VERSION_HIERARCHICAL = 2


class FusedAdamW(torch.optim.Optimizer):
    def __init__(self, params: Iterable, lr: float = 1e-3, betas=(0.9, 0.999), eps: float = 1e-5,
                 weight_decay: float = 1e-4, amsgrad: bool = False, *, maximize: bool = False,
                 fused_step: bool = False, max_grad_norm: Optional[float] = None,
                 hierarchical_stats: bool = False, model_copies: Optional[dict] = None):
        if max_grad_norm is not None and not fused_step:
            raise ValueError("max_grad_norm requires fused_step=True")
        if max_grad_norm is not None and not (math.isfinite(max_grad_norm) and max_grad_norm > 0):
            raise ValueError("max_grad_norm must be a positive finite number")
        defaults = dict(lr=lr, betas=tuple(betas), eps=eps, weight_decay=weight_decay, amsgrad=amsgrad,
                        maximize=maximize)
        super().__init__(params, defaults)
        self.fused_step = bool(fused_step)
        self.max_grad_norm = max_grad_norm
        self.hierarchical_stats = bool(hierarchical_stats)
        self._workspace: Optional[torch.Tensor] = None
        self.last_result: Optional[_abi.FusedResult] = None
        self._copies: dict = {}
        for master, copy in (model_copies or {}).items():
            self.attach_model_copy(master, copy)

    def attach_model_copy(self, master: torch.Tensor, copy: torch.Tensor) -> None:
        """Keep a float16 / bfloat16 model copy of an FP32 master parameter:
        every update rewrites it (rounded to nearest even) in the same pass."""
        if copy.dtype not in (torch.float16, torch.bfloat16) or copy.shape != master.shape:
            raise ValueError("a model copy is a float16 / bfloat16 tensor of the master's shape")
        self._copies[master] = copy

    # ------------------------------------------------------------ state --
    def _state_for(self, p: torch.Tensor, amsgrad: bool):
        st = self.state[p]
        if not st:
            st["step"] = 0
            st["exp_avg"] = torch.empty_like(p, memory_format=torch.contiguous_format)
            st["exp_avg_sq"] = torch.empty_like(p, memory_format=torch.contiguous_format)
            if amsgrad:
                st["max_exp_avg_sq"] = torch.empty_like(p, memory_format=torch.contiguous_format)
        elif amsgrad and "max_exp_avg_sq" not in st:
            raise RuntimeError("amsgrad was switched on after the first step; the running max has no history")
        return st

    def _active(self):
        """[(group, [(param, state), ...])] for parameters that have a gradient."""
        out = []
        for group in self.param_groups:
            items = []
            for p in group["params"]:
                if p.grad is None:
                    continue
                if p.dtype != torch.float32:
                    raise ValueError("FusedAdamW keeps FP32 master parameters")
                if p.grad.is_sparse:
                    raise ValueError("sparse gradients are not supported")
                items.append((p, self._state_for(p, group["amsgrad"])))
            if items:
                out.append((group, items))
        return out

    @staticmethod
    def _options(group) -> _abi.Options:
        b1, b2 = group["betas"]
        return _abi.options(group["lr"], b1, b2, group["eps"], group["weight_decay"], group["amsgrad"],
                            group["maximize"])

    @staticmethod
    def _segment(p, st) -> _abi.Segment:
        return _abi.Segment(p, p.grad, st["exp_avg"], st["exp_avg_sq"], st.get("max_exp_avg_sq"))

    # ------------------------------------------------------------- step --
    @torch.no_grad()
    def step(self, closure=None, gradient_scale: float = 1.0):
        """One update of every parameter with a gradient.  ``gradient_scale``
        divides the stored gradients (a loss scale).  Returns the closure's
        loss, if any."""
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        active = self._active()
        if not active:
            return loss
        ctrl = _abi.control(gradient_scale, False)
        self.last_result = None
        if self.fused_step:
            ctrl = self._fused_decision(active, gradient_scale)
            if ctrl is None:
                return loss  # whole step skipped: non-finite gradient
        for group, items in active:
            opts = self._options(group)
            by_step = {}  # one launch set per (step count, model-copy dtype)
            for p, st in items:
                copy = self._copies.get(p)
                key = (st["step"], None if copy is None else copy.dtype)
                by_step.setdefault(key, []).append((p, st))
            for (step, copy_dtype), members in by_step.items():
                segs = [self._segment(p, st) for p, st in members]
                if copy_dtype is None:
                    _, new_step = _abi.radamw_step_multi(segs, step, opts, ctrl)
                else:
                    copies = [self._copies[p] for p, _ in members]
                    _, new_step = _abi.radamw_step_multi_writeback(segs, copies, step, opts, ctrl)
                for _, st in members:
                    st["step"] = new_step
        return loss

    def _fused_decision(self, active, gradient_scale: float):
        """Statistics of every active gradient -> merge -> 12-byte read-back ->
        decision.  Returns the control for the update, or None to skip."""
        grads = [p.grad for _, items in active for p, _ in items]
        dev = grads[0].device
        rows_total = sum(_abi.radamw_grad_stats_rows(g.numel(), g.dtype) for g in grads)
        scratch_elems = _abi.radamw_stats_plan(rows_total)[0] if rows_total else 0
        words = 3 * rows_total + scratch_elems + 3
        if self._workspace is None or self._workspace.numel() < words or self._workspace.device != dev:
            self._workspace = torch.empty(words, dtype=torch.int32, device=dev)
        ws = self._workspace
        rows = ws[:3 * rows_total]
        off = 0
        for g in grads:
            off += _abi.radamw_grad_stats(g.contiguous() if not g.is_contiguous() else g, rows, off)
        scratch = ws[3 * rows_total:3 * rows_total + scratch_elems].view(torch.float32) if scratch_elems else None
        report = ws[3 * rows_total + scratch_elems:3 * rows_total + scratch_elems + 3]
        _abi.radamw_merge_stats(rows, rows_total, scratch, report, self.hierarchical_stats)
        host = _abi.radamw_read_report(report)
        ctrl, result = _abi.radamw_decide(host, gradient_scale, self.max_grad_norm)
        self.last_result = result
        return None if ctrl.skip_update else ctrl

    # ------------------------------------------------------- checkpoints --
    def step_options(self) -> dict:
        return {
            "version": STEP_OPTIONS_VERSION_HIERARCHICAL if self.hierarchical_stats else STEP_OPTIONS_VERSION_FLAT,
            "fused_step": self.fused_step,
            "max_grad_norm": self.max_grad_norm,
            "hierarchical_stats": self.hierarchical_stats,
        }

    def state_dict(self):
        sd = super().state_dict()
        sd["step_options"] = self.step_options()
        return sd

    def load_state_dict(self, state_dict):
        state_dict = dict(state_dict)
        opts = state_dict.pop("step_options", None)
        super().load_state_dict(state_dict)
        for st in self.state.values():
            if "step" in st:
                st["step"] = int(st["step"])
        if opts is None:
            # an archive written without step options: fused and hierarchical modes off
            self.fused_step, self.max_grad_norm, self.hierarchical_stats = False, None, False
        else:
            version = int(opts.get("version", STEP_OPTIONS_VERSION_FLAT))
            if version not in (STEP_OPTIONS_VERSION_FLAT, STEP_OPTIONS_VERSION_HIERARCHICAL):
                raise ValueError(f"unknown step-options version {version}")
            self.fused_step = bool(opts.get("fused_step", False))
            self.max_grad_norm = opts.get("max_grad_norm")
            self.hierarchical_stats = version == STEP_OPTIONS_VERSION_HIERARCHICAL and bool(
                opts.get("hierarchical_stats", False))
            if self.max_grad_norm is not None and not self.fused_step:
                raise ValueError("archive has max_grad_norm without fused_step")
