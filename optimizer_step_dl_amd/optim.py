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

``flatten=True`` moves every parameter group into one flattened bucket
(FA-ja "サポートされている契約": a pre-flattened bucket shares the options
and the step count): the parameters, their gradients and the moments of a
group become views of one device allocation in the library's stream
placement (radamw_bucket_layout), so a group's step is one analysis and one
update launch over the whole bucket, and for groups of up to about 2^28
parameters the placement itself moves HBM 3-4.5% faster than separate
allocations (larger groups gain the launches, not the placement).  In that mode every parameter of a
group is updated at every step (a parameter that received no gradient is
updated with a zero gradient), ``zero_grad`` zeroes the gradient bucket in
place whatever ``set_to_none`` says, and a ``.grad`` replaced by another
tensor is copied back into its place in the bucket before the step.  The
gradient dtype of a group is ``flatten_grad_dtype``, else the dtype of the
parameters' current ``.grad`` (or their ``grad_dtype``), else FP32.

All arithmetic runs in the library's kernels; this class only groups
tensors into launch buckets (parameter group, gradient dtype, model-copy
dtype, step count: one launch shares one options struct, one dtype and one
step count) and calls the C entry points.  Each bucket is a persistent
tensor list, validated once and reused while its tensors keep their
storage, and a fused step is one radamw_lists_fused_step call over all of
them.  A cached list holds references to the tensors it was built from
(including the gradients of the last step) until it is rebuilt or freed.
Parameters must be FP32 device tensors; gradients FP32, FP16 or BF16 of the
same shape.  Torch versions that check a gradient's dtype against its
parameter's need ``param.grad_dtype`` set (to the 16-bit dtype, or None)
before a 16-bit ``.grad`` is assigned to an FP32 master parameter.
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
                 hierarchical_stats: bool = False, model_copies: Optional[dict] = None,
                 flatten: bool = False, flatten_grad_dtype: Optional[torch.dtype] = None):
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
        self._cache: dict = {}  # bucket -> (storage signature, TensorList)
        self.last_result: Optional[_abi.FusedResult] = None
        self._copies: dict = {}
        for master, copy in (model_copies or {}).items():
            self.attach_model_copy(master, copy)
        self._flat: list = []  # flattened buckets, one per parameter group
        self._flat_ids: set = set()
        if flatten:
            if self._copies:
                raise ValueError("flatten does not keep model copies")
            self._flatten(flatten_grad_dtype)

    def attach_model_copy(self, master: torch.Tensor, copy: torch.Tensor) -> None:
        """Keep a float16 / bfloat16 model copy of an FP32 master parameter:
        every update rewrites it (rounded to nearest even) in the same pass."""
        if id(master) in getattr(self, "_flat_ids", ()):
            raise ValueError("a flattened parameter keeps no model copy")
        if copy.dtype not in (torch.float16, torch.bfloat16) or copy.shape != master.shape:
            raise ValueError("a model copy is a float16 / bfloat16 tensor of the master's shape")
        self._copies[master] = copy

    # ------------------------------------------------------ flattening --
    def _flatten(self, grad_dtype):
        """Move each parameter group into one bucket allocation (see the
        module docstring): parameters, gradients and moments become views."""
        f32 = torch.float32
        for gi, group in enumerate(self.param_groups):
            params = list(group["params"])
            if not params:
                continue
            dev = params[0].device
            gds = set()
            for p in params:
                if p.dtype != f32 or p.device != dev or p.device.type != "cuda" or p.is_sparse:
                    raise ValueError("flatten needs dense FP32 device parameters of one device per group")
                gd = grad_dtype or (p.grad.dtype if p.grad is not None else None) or \
                    getattr(p, "grad_dtype", None) or f32
                gds.add(gd)
            if len(gds) != 1:
                raise ValueError("the parameters of a flattened group need one gradient dtype")
            gd = gds.pop()
            if gd not in (f32, torch.float16, torch.bfloat16):
                raise ValueError(f"gradient dtype {gd} is not float32 / float16 / bfloat16")
            ams = bool(group["amsgrad"])
            total = sum(p.numel() for p in params)
            streams = _abi.bucket_arena(total, [f32, gd, f32, f32] + ([f32] if ams else []), dev)
            members, off = [], 0
            with torch.no_grad():
                for p in params:
                    n = p.numel()
                    pv = streams[0][off:off + n].view(p.shape)
                    pv.copy_(p.detach())
                    p.data = pv
                    gv = streams[1][off:off + n].view(p.shape)
                    if p.grad is not None:
                        gv.copy_(p.grad)
                    else:
                        gv.zero_()
                    if gd != p.dtype:
                        if not hasattr(p, "grad_dtype"):
                            raise ValueError("this torch cannot keep a 16-bit .grad on an FP32 parameter")
                        p.grad_dtype = gd
                    p.grad = gv
                    st = self.state[p]
                    st.clear()
                    st["step"] = 0
                    st["exp_avg"] = streams[2][off:off + n].view(p.shape)
                    st["exp_avg_sq"] = streams[3][off:off + n].view(p.shape)
                    if ams:
                        st["max_exp_avg_sq"] = streams[4][off:off + n].view(p.shape)
                    members.append((p, off, n))
                    self._flat_ids.add(id(p))
                    off += n
            # the group is found by its index at every step: load_state_dict
            # replaces the group dicts, and schedulers edit the current ones
            self._flat.append({"group_index": gi, "amsgrad": ams, "grad_dtype": gd, "streams": streams,
                               "members": members, "list": None})

    def _flat_lists(self):
        """[(TensorList, group, members)] of the flattened buckets: each
        gradient is put back in its place in the bucket first (a parameter
        without one gets a zero gradient), and every bucket is one
        single-segment persistent list."""
        out = []
        for b in self._flat:
            group = self.param_groups[b["group_index"]]
            if bool(group["amsgrad"]) != b["amsgrad"]:
                raise RuntimeError("amsgrad of a flattened group cannot change")
            g_arena = b["streams"][1]
            with torch.no_grad():
                for p, off, n in b["members"]:
                    gv = g_arena[off:off + n]
                    if p.grad is None:
                        gv.zero_()
                        p.grad = gv.view(p.shape)
                    elif p.grad.data_ptr() != gv.data_ptr() or p.grad.dtype != g_arena.dtype:
                        gv.copy_(p.grad.reshape(-1))
                        p.grad = gv.view(p.shape)
            steps = {self.state[p]["step"] for p, _, _ in b["members"]}
            if len(steps) != 1:
                raise RuntimeError("the parameters of a flattened group share one step count")
            if b["list"] is None:
                b["list"] = _abi.TensorList([_abi.Segment(*b["streams"])], b["amsgrad"])
            out.append((b["list"], group, [(p, self.state[p]) for p, _, _ in b["members"]]))
        return out

    @torch.no_grad()
    def zero_grad(self, set_to_none: bool = True):
        """As torch's, except that a flattened group's gradients are zeroed
        in place (one fill of the gradient bucket) and stay its views."""
        for b in self._flat:
            b["streams"][1].zero_()
            for p, off, n in b["members"]:
                gv = b["streams"][1][off:off + n]
                if p.grad is None or p.grad.data_ptr() != gv.data_ptr():
                    p.grad = gv.view(p.shape)
        for group in self.param_groups:
            for p in group["params"]:
                if id(p) in self._flat_ids or p.grad is None:
                    continue
                if set_to_none:
                    p.grad = None
                else:
                    if p.grad.grad_fn is not None:
                        p.grad.detach_()
                    else:
                        p.grad.requires_grad_(False)
                    p.grad.zero_()

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
                if p.grad is None or id(p) in self._flat_ids:
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
    def _lists(self, active):
        """Launch buckets -- (parameter group, gradient dtype, model-copy
        dtype, step count), since one launch shares one options struct, one
        gradient dtype and one step count -- each as a persistent tensor list
        [(TensorList, group, members)].  A cached list is reused while its
        tensors keep their storage; a list whose tensors moved (a new
        ``.grad`` tensor, a loaded state) is rebuilt, and lists no bucket
        uses any more are freed."""
        buckets = {}
        for group, items in active:
            for p, st in items:
                copy = self._copies.get(p)
                key = (id(group), bool(group["amsgrad"]), p.grad.dtype, None if copy is None else copy.dtype,
                       st["step"])
                buckets.setdefault(key, (group, []))[1].append((p, st))
        out, used = [], set()
        for key, (group, members) in buckets.items():
            ident = key[:4] + (tuple(id(p) for p, _ in members),)
            sig = tuple((p.data_ptr(), p.grad.data_ptr(), st["exp_avg"].data_ptr(), st["exp_avg_sq"].data_ptr(),
                         st["max_exp_avg_sq"].data_ptr() if "max_exp_avg_sq" in st else 0,
                         self._copies[p].data_ptr() if p in self._copies else 0, p.numel())
                        for p, st in members)
            cached = self._cache.get(ident)
            if cached is None or cached[0] != sig:
                if cached is not None:
                    cached[1].close()
                segs = [self._segment(p, st) for p, st in members]
                copies = None if key[3] is None else [self._copies[p] for p, _ in members]
                cached = (sig, _abi.TensorList(segs, group["amsgrad"], copies))
                self._cache[ident] = cached
            used.add(ident)
            out.append((cached[1], group, members))
        for ident in [k for k in self._cache if k not in used]:
            self._cache.pop(ident)[1].close()
        return out

    def _release_lists(self):
        for _, lst in self._cache.values():
            lst.close()
        self._cache.clear()
        for b in self._flat:
            if b["list"] is not None:
                b["list"].close()
                b["list"] = None

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
        self.last_result = None
        if not active and not self._flat:
            return loss
        lists = self._lists(active) + self._flat_lists()
        if self.fused_step:
            # statistics of every active gradient -> one 12-byte report ->
            # one decision for all buckets -> each bucket's update
            try:
                res, steps = _abi.radamw_lists_fused_step(
                    [lst for lst, _, _ in lists], [members[0][1]["step"] for _, _, members in lists],
                    [self._options(group) for _, group, _ in lists], gradient_scale, self.max_grad_norm,
                    self.hierarchical_stats)
            except _abi.DecisionMismatch as e:
                # the step ran as the device decided: keep the step counts
                # consistent with the state it wrote, then report the fault
                self.last_result = e.result
                for (_, _, members), new_step in zip(lists, e.steps):
                    for _, st in members:
                        st["step"] = new_step
                raise
            self.last_result = res
        else:
            ctrl = _abi.control(gradient_scale, False)
            steps = [lst.step(members[0][1]["step"], self._options(group), ctrl)[1]
                     for lst, group, members in lists]
        for (_, _, members), new_step in zip(lists, steps):
            for _, st in members:
                st["step"] = new_step
        return loss

    # ------------------------------------------------------- checkpoints --
    def step_options(self) -> dict:
        return {
            "version": STEP_OPTIONS_VERSION_HIERARCHICAL if self.hierarchical_stats else STEP_OPTIONS_VERSION_FLAT,
            "fused_step": self.fused_step,
            "max_grad_norm": self.max_grad_norm,
            "hierarchical_stats": self.hierarchical_stats,
        }

    def _param_index(self):
        """id(param) -> its index in a state_dict (torch numbers parameters
        across groups in order)."""
        idx, k = {}, 0
        for group in self.param_groups:
            for p in group["params"]:
                idx.setdefault(id(p), k)
                k += 1
        return idx

    def state_dict(self):
        sd = super().state_dict()
        sd["step_options"] = self.step_options()
        if self._flat:
            # a flattened parameter's state is a view of its group's bucket:
            # store compact copies, not the whole allocation behind them
            index = self._param_index()
            sd["state"] = dict(sd["state"])
            for b in self._flat:
                for p, _, _ in b["members"]:
                    k = index[id(p)]
                    if k in sd["state"]:
                        sd["state"][k] = {name: (v.clone() if torch.is_tensor(v) else v)
                                          for name, v in sd["state"][k].items()}
        return sd

    def load_state_dict(self, state_dict):
        self._release_lists()
        state_dict = dict(state_dict)
        opts = state_dict.pop("step_options", None)
        super().load_state_dict(state_dict)
        for st in self.state.values():
            if "step" in st:
                st["step"] = int(st["step"])
        for b in self._flat:
            # the loaded state goes back into the bucket, whose views it keeps
            s_arena = b["streams"]
            names = ["exp_avg", "exp_avg_sq"] + (["max_exp_avg_sq"] if b["amsgrad"] else [])
            steps = set()
            with torch.no_grad():
                for p, off, n in b["members"]:
                    st = self.state[p]
                    steps.add(int(st.get("step", 0)))
                    for j, name in enumerate(names):
                        view = s_arena[2 + j][off:off + n].view(p.shape)
                        if name in st:
                            view.copy_(st[name])
                        else:
                            view.zero_()
                        st[name] = view
                    st["step"] = int(st.get("step", 0))
            if len(steps) != 1:
                raise ValueError("the parameters of a flattened group share one step count")
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
