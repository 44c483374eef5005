"""GPU check of radamw_fused_step_multi_noalloc, the fused step that
allocates nothing (its statistics rows, merge scratch, decision and report
live in a static device array of the library): through the C ABI, several
calls in a row -- a large first step with the clip active, then smaller
inputs, a flat merge and a skipped step -- each equal, bit for bit, the same
step through radamw_fused_step_multi with a caller workspace.  The name
sorts last so that the suite's other tests run first."""
import ctypes

import pytest
import torch

import synth
import optimizer_step_dl_amd as ra
from optimizer_step_dl_amd import _abi
from gpu_helpers import DEV, announce, bits_equal

pytestmark = pytest.mark.gpu


def _noalloc(segs, step, opts, scale, max_norm, hierarchical):
    """The entry point through the C ABI: (status, result, new step)."""
    lib = ra.load()
    arr, code, dev, count = _abi._marshal(segs)
    st = ctypes.c_uint64(step)
    res = _abi.FusedResult()
    with torch.cuda.device(dev):
        rc = lib.radamw_fused_step_multi_noalloc(arr, count, code, ctypes.byref(st), ctypes.byref(opts),
                                                 float(scale), float(max_norm), int(hierarchical),
                                                 _abi._stream(dev), ctypes.byref(res))
    return rc, res, int(st.value)


def _bucket(n, gdt, scale, amsgrad, key):
    p = synth.normal(n, 0.02, key + ("p",), DEV)
    g = synth.stored_grad(n, 1e-3, scale, gdt, key + ("g",), DEV)
    m, v, vmax = synth.steady_state(n, key, amsgrad, DEV)
    return ra.Segment(p, g, m, v, vmax)


def _twin(s):
    c = lambda t: None if t is None else t.clone()
    return ra.Segment(c(s.param), s.grad, c(s.exp_avg), c(s.exp_avg_sq), c(s.max_exp_avg_sq))


CASES = [  # n, grad dtype, scale, AMSGrad, completed steps, max_norm, hierarchical, inject inf
    (5_000_003, "bf16", 1.0, True, 0, 1.0, True, False),
    (70_001, "f32", 1.0, False, 7, 0.0, False, False),
    (70_001, "f16", 1024.0, True, 3, 1.0, True, True),
    ((1 << 22) + 5, "f16", 1024.0, False, 41, 0.5, True, False),
    (1029, "bf16", 1.0, False, 0, 1.0, False, False),
]


def test_noalloc_fused_step_equals_fused_step_with_workspace():
    announce("noalloc fused step vs workspace fused step")
    for k, (n, gdt, scale, ams, step, max_norm, hier, inject) in enumerate(CASES):
        announce(f"noalloc case {k}: n={n} {gdt} ams={ams} step={step} clip={max_norm} hier={hier} inf={inject}")
        a = _bucket(n, gdt, scale, ams, (0, "noalloc", k))
        if inject:
            a.grad[n // 3] = float("inf")
        b = _twin(a)
        opts = ra.options(lr=1e-3, weight_decay=0.01, amsgrad=ams)
        ws = torch.empty(ra.radamw_fused_workspace_bytes([b]), dtype=torch.uint8, device=DEV)
        want, want_step = ra.radamw_fused_step_multi([b], step, opts, scale, max_norm, hier, ws)
        rc, got, got_step = _noalloc([a], step, opts, scale, max_norm, hier)
        torch.cuda.synchronize()
        assert rc == 0, rc
        assert got_step == want_step == step + (0 if inject else 1)
        for f in ("updated", "found_inf", "nonfinite", "sumsq", "total_norm", "clip_coef"):
            assert getattr(got, f) == getattr(want, f), (k, f)
        assert bool(got.updated) == (not inject)
        for x, y in ((a.param, b.param), (a.exp_avg, b.exp_avg), (a.exp_avg_sq, b.exp_avg_sq)):
            assert bits_equal(x, y), k
        if ams:
            assert bits_equal(a.max_exp_avg_sq, b.max_exp_avg_sq), k


def test_noalloc_allocates_no_device_memory_and_rejects_lists():
    announce("noalloc memory and rejections")
    s = _bucket(300_000, "f32", 1.0, False, (0, "noalloc-mem"))
    opts = ra.options()
    rc, _, step = _noalloc([s], 5, opts, 1.0, 1.0, True)
    assert rc == 0 and step == 6
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info(DEV)[0]
    for k in range(5):
        rc, res, step = _noalloc([s], step, opts, 1.0, 1.0, True)
        assert rc == 0 and res.updated
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info(DEV)[0] == free0
    launches = ra.radamw_launch_count()
    rc, _, st = _noalloc([s, s], step, opts, 1.0, 1.0, True)  # two segments: beyond what it takes
    assert rc == -5 and st == step and ra.radamw_launch_count() == launches
    e = torch.empty(0, device=DEV)
    rc, res, st = _noalloc([ra.Segment(e, e, e, e)], step, opts, 1.0, 1.0, True)  # empty: nothing to do
    assert rc == 0 and st == step and not res.updated and ra.radamw_launch_count() == launches
    # the Python binding of the same entry point
    res, st = ra.radamw_fused_step_multi_noalloc([s], step, opts, 1.0, 1.0, True)
    assert res.updated and st == step + 1
