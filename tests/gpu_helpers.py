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
