"""Shared pieces of the GPU parity tests: device placement, oracle mirrors
and the comparison bars.

The bars (floating point):
  - after one update, per element: |gpu - oracle| <= 1e-6 * (1 + |oracle|)
    for p, m, v, v_max (the stated contract);
  - after many updates: max |gpu - oracle| / max |oracle| <= 1e-5 per array
    (normwise; per-element relative error is unbounded where m crosses 0);
  - diagnostic on the moments (the absolute bar above is vacuous at 1e-6
    scale): |gpu - oracle| <= k ulps of the magnitude of the terms summed.
Step counts, skip decisions and non-finite counts are compared exactly.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth
import optimizer_step_dl_amd as ra

DEV = torch.device("cuda", 0)
TORCH_GDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def announce(msg: str):
    """Name the GPU case before it runs (a fault may end the process)."""
    sys.stdout.write(f"\n[gpu-case] {msg}\n")
    sys.stdout.flush()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").numpy().copy()


def grad_host(g: torch.Tensor) -> np.ndarray:
    return synth.grad_numpy(g)


def oracle_opts(o: ra.Options) -> oracle.Options:
    return oracle.Options(lr=o.lr, beta1=o.beta1, beta2=o.beta2, eps=o.eps,
                          weight_decay=o.weight_decay, amsgrad=bool(o.amsgrad),
                          maximize=bool(o.maximize))


def new_gpu_state(n: int, amsgrad: bool, fill=float("nan")) -> ra.AdamWState:
    """Moment buffers for a step-0 state, filled with NaN: the first update
    must initialise them without reading (any read would leak NaN)."""
    mk = lambda: torch.full((n,), fill, dtype=torch.float32, device=DEV)
    return ra.AdamWState(0, mk(), mk(), mk() if amsgrad else None)


def contract_one_step(gpu: np.ndarray, ref: np.ndarray, what: str):
    err = np.abs(gpu.astype(np.float64) - ref.astype(np.float64))
    bound = 1e-6 * (1.0 + np.abs(ref.astype(np.float64)))
    bad = np.flatnonzero(~(err <= bound))
    assert bad.size == 0, f"{what}: {bad.size} elements over 1e-6(1+|ref|), first {bad[:5]}, max err {err.max()}"


def normwise(gpu: np.ndarray, ref: np.ndarray, what: str, tol: float = 1e-5):
    ref64 = ref.astype(np.float64)
    denom = np.abs(ref64).max()
    err = np.abs(gpu.astype(np.float64) - ref64).max()
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    assert err <= tol * denom, f"{what}: normwise {err / max(denom, 1e-300):.3e} > {tol}"


def ulps_of(gpu: np.ndarray, ref: np.ndarray, scale: np.ndarray, k: float, what: str):
    """|gpu - ref| <= k ulps of ``scale`` (the magnitude of the summed terms)."""
    err = np.abs(gpu.astype(np.float64) - ref.astype(np.float64))
    ulp = np.spacing(np.abs(scale).astype(np.float32)).astype(np.float64)
    bad = np.flatnonzero(~(err <= k * ulp + 1e-30))
    assert bad.size == 0, f"{what}: {bad.size} elements over {k} ulps, first {bad[:5]}"


def bits_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def snapshot(*ts):
    return [None if t is None else t.clone() for t in ts]


def unchanged(before, after) -> bool:
    return all((a is None and b is None) or bits_equal(a, b) for a, b in zip(before, after))


# --------------------------------------------------- whole-array parity --
#
# At full size the oracle runs on every element: each tensor's pre-step
# state is staged through pinned host memory, the oracle updates it there
# (split over threads into contiguous slices: the update is elementwise, so
# the slices compute exactly what one call would), and the GPU's result is
# compared with it element by element on the device, in float64, chunk by
# chunk.
#
# Bars for one update from the same state:
#   p, m, v, v_max : |gpu - oracle| <= 1e-6 (1 + |oracle|)        (contract)
#   m              : |gpu - oracle| <= K_M ulp(|b1 m_old| + |(1-b1) g|)
#   v, v_max       : |gpu - oracle| <= K_V ulp(b2 v_old + (1-b2) g^2)
# with g the unscaled gradient.  Derivation: the GPU forms g = x * fl(1/s)
# and fuses b1 m_old (b2 v_old) into the sum with an FMA, the oracle forms
# g = fl(x / s) and rounds every product; with a power-of-two scale both g
# are exact and the two results differ by at most ~2 roundings of the
# terms (K = 4 leaves room); with any other scale the two g differ by up to
# 3 units of 2^-24 |g|, which (1-b1) g and (1-b2) g^2 carry into the sum,
# up to ~7.3 ulps of the terms (K = 8).  v_max is max(v_max_old, v): equal
# branches give v's error or none, and a different branch means v and
# v_max_old lie within v's error of each other.

import os as _os
from concurrent.futures import ThreadPoolExecutor as _Pool

ORACLE_THREADS = max(1, min(16, len(_os.sched_getaffinity(0))))


def oracle_step_threaded(p, g, gdt, state, opts, scale, skip=False, threads=ORACLE_THREADS):
    """oracle.adamw_step over ``threads`` contiguous slices at once (numpy,
    in place).  Returns whether the update ran."""
    n = p.size
    if n < (1 << 20) or threads <= 1:
        return oracle.adamw_step(p, g, gdt, state, opts, scale, skip)
    bounds = [(n * k // threads, n * (k + 1) // threads) for k in range(threads)]

    def run(b):
        lo, hi = b
        s = oracle.State.__new__(oracle.State)
        s.step = state.step
        s.exp_avg, s.exp_avg_sq = state.exp_avg[lo:hi], state.exp_avg_sq[lo:hi]
        s.max_exp_avg_sq = None if state.max_exp_avg_sq is None else state.max_exp_avg_sq[lo:hi]
        ran = oracle.adamw_step(p[lo:hi], g[lo:hi], gdt, s, opts, scale, skip)
        return ran, s.step

    with _Pool(threads) as pool:
        outs = list(pool.map(run, bounds))
    assert len({o for o in outs}) == 1
    state.step = outs[0][1]
    return outs[0][0]


class PinnedStage:
    """Reusable pinned host buffers, one per (role, dtype), grown on demand."""

    def __init__(self):
        self.bufs = {}

    def host(self, t: torch.Tensor, role: str) -> torch.Tensor:
        key = (role, t.dtype)
        b = self.bufs.get(key)
        if b is None or b.numel() < t.numel():
            b = torch.empty(max(t.numel(), 1), dtype=t.dtype, pin_memory=t.numel() >= (1 << 20))
            self.bufs[key] = b
        b = b[:t.numel()]
        b.copy_(t.reshape(-1))
        return b


def _np_of(t: torch.Tensor) -> np.ndarray:
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def oracle_one_step_pinned(stage, pre, g, gdt, opts, scale, step, amsgrad, skip=False):
    """Run the oracle one step from device pre-state ``pre`` = (p, m, v,
    v_max or None) at completed-step count ``step``; returns pinned host
    tensors (p, m, v, v_max or None) holding the oracle's result."""
    hp = stage.host(pre[0], "p")
    hm, hv = stage.host(pre[1], "m"), stage.host(pre[2], "v")
    hx = stage.host(pre[3], "x") if amsgrad else None
    hg = stage.host(g, "g")
    st = oracle.State.__new__(oracle.State)
    st.step = step
    st.exp_avg, st.exp_avg_sq = hm.numpy(), hv.numpy()
    st.max_exp_avg_sq = None if hx is None else hx.numpy()
    if step == 0:  # "no state": the moments start from zero, whatever the buffers hold
        st.exp_avg[:] = 0
        st.exp_avg_sq[:] = 0
        if hx is not None:
            st.max_exp_avg_sq[:] = 0
    oracle_step_threaded(hp.numpy(), _np_of(hg), gdt, st, opts, scale, skip)
    return hp, hm, hv, hx


def _ulp32(x64: torch.Tensor) -> torch.Tensor:
    x = x64.abs().float()
    return (torch.nextafter(x, torch.full_like(x, float("inf"))) - x).double()


def compare_one_step_full(what, after, ref, pre, g, eff_scale, b1, b2, first, power_of_two,
                          chunk=1 << 25, stats=None, finite_only=False):
    """Every element of ``after`` (device p, m, v, v_max or None) against the
    oracle's ``ref`` (host) under the bars above.  ``pre`` holds the device
    m, v (unused on a first step) the update started from; ``g`` the device
    gradient.  ``stats`` (a dict), if given, receives the largest error in
    units of each ulp bar."""
    k_m, k_v = (4.0, 4.0) if power_of_two else (8.0, 8.0)
    n = after[0].numel()
    names = ("p", "m", "v", "vmax")
    worst = {"m": 0.0, "v": 0.0, "vmax": 0.0}
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        gg = g[lo:hi].double() / eff_scale
        m_old = torch.zeros_like(gg) if first else pre[1][lo:hi].double()
        v_old = torch.zeros_like(gg) if first else pre[2][lo:hi].double()
        m_ulp = _ulp32((b1 * m_old).abs() + ((1.0 - b1) * gg).abs())
        v_ulp = _ulp32(b2 * v_old + (1.0 - b2) * gg * gg)
        keep = torch.isfinite(gg) if finite_only else None
        for name, a, r in zip(names, after, ref):
            if a is None:
                continue
            got = a[lo:hi].double()
            want = r[lo:hi].to(a.device, non_blocking=False).double()
            err = (got - want).abs()
            bad = ~(err <= 1e-6 * (1.0 + want.abs()))
            if name != "p":
                ulp = m_ulp if name == "m" else v_ulp
                k = k_m if name == "m" else k_v
                bad |= ~(err <= k * ulp + 1e-45)
                ratio = err / (ulp + 1e-45)
                if keep is not None:
                    ratio = torch.where(keep, ratio, torch.zeros_like(ratio))
                worst[name] = max(worst[name], float(ratio.max()))
            if keep is not None:
                bad &= keep
            nbad = int(bad.sum())
            if nbad:
                idx = torch.nonzero(bad).flatten()[:5] + lo
                raise AssertionError(f"{what} {name}: {nbad} of elements [{lo}, {hi}) over the bar, first {idx.tolist()}, "
                                     f"gpu {a[idx].tolist()} oracle {r[idx.cpu()].tolist()}")
    if stats is not None:
        for k, val in worst.items():
            stats[k] = max(stats.get(k, 0.0), val)


def is_power_of_two(x: float) -> bool:
    m, _ = np.frexp(x)
    return m == 0.5


def clone_state(p, st):
    """Device copies of (p, m, v, v_max) before a step."""
    return tuple(None if t is None else t.clone() for t in (p, st.exp_avg, st.exp_avg_sq, st.max_exp_avg_sq))


def check_step_from(pre, after, g_dev, gdt, opts, scale, step_before, what, stats=None, stage=None):
    """The oracle run one update from the GPU's own pre-step state ``pre``
    (device copies of p, m, v, v_max) with the device gradient ``g_dev``,
    compared with every element of ``after`` (device p, m, v, v_max) under
    the contract and the moments' ulp bars (compare_one_step_full)."""
    amsgrad = bool(opts.amsgrad)
    ref = oracle_one_step_pinned(stage or PinnedStage(), pre, g_dev, gdt, oracle_opts(opts), scale, step_before,
                                 amsgrad)
    compare_one_step_full(what, after, ref, pre, g_dev, scale, opts.beta1, opts.beta2, first=step_before == 0,
                          power_of_two=is_power_of_two(scale), stats=stats)
