"""GPU parity of the gradient statistics (radamw_grad_stats, radamw_merge_stats,
radamw_read_report) and of the fused step (radamw_fused_step_multi) against the
CPU oracle.  Counts and skip decisions are compared exactly; sums of squares
against math.fsum-exact values within FP64 rounding.

Page abbreviations: FA-ja = "実験的なデバイス上の融合 AdamW / AMSGrad",
TR-zh = "训练与状态保存"."""
import math


import numpy as np
import pytest
import torch

import oracle
import synth
import optimizer_step_dl_amd as ra
from gpu_helpers import DEV, TORCH_GDT, announce, contract_one_step, grad_host, host, new_gpu_state, oracle_opts

pytestmark = pytest.mark.gpu


def _inject(g: torch.Tensor, k: int, key) -> np.ndarray:
    pos = synth.nonfinite_positions(g.numel(), k, key)
    vals = torch.tensor(synth.nonfinite_values(k), dtype=g.dtype, device=g.device)
    g[torch.from_numpy(pos).to(g.device)] = vals
    return pos


def _exact_sumsq(g_host: np.ndarray, gdt: str) -> float:
    x = oracle.widen(g_host, gdt).astype(np.float64) if g_host.size < 300000 else None
    if x is None:
        t = torch.from_numpy(g_host.view(np.int16) if gdt != "f32" else g_host)
        if gdt != "f32":
            t = t.view(TORCH_GDT[gdt])
        x = t.double().numpy()
    x = x[np.isfinite(x)]
    return math.fsum((x * x).tolist())


def _stats_gpu(grads, hierarchical=True):
    rows_total = sum(ra.radamw_grad_stats_rows(g.numel(), g.dtype) for g in grads)
    rows = torch.zeros(3 * max(rows_total, 1), dtype=torch.int32, device=DEV)
    off = 0
    for g in grads:
        off += ra.radamw_grad_stats(g, rows, off)
    assert off == rows_total
    se, _ = ra.radamw_stats_plan(rows_total)
    scratch = torch.zeros(max(se, 1), dtype=torch.float32, device=DEV)
    report = torch.zeros(3, dtype=torch.int32, device=DEV)
    ra.radamw_merge_stats(rows, rows_total, scratch if se else None, report, hierarchical)
    rep = ra.radamw_read_report(report)
    return rep.sumsq, rep.nonfinite, rows_total


def sequential_bound(n: int) -> float:
    """A-priori relative error bound of a left-to-right FP64 sum of n
    non-negative terms (the oracle's order): (n - 1) * 2^-53."""
    return max(n - 1, 1) * 2.0**-53


@pytest.mark.parametrize("gdt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("n", [1, 7, 8, 9, 4096, 8193, 100003, 3_000_001, 70_000_003])
def test_grad_stats_single_tensor(gdt, n):
    """Counts bit-exact against the oracle; the GPU's sum within 1e-12 of the
    exactly rounded sum (math.fsum); the oracle's sequential sum within its
    own rounding bound.  70,000,003 elements put every analysis workgroup on
    several passes (rows capped at 8192) with a ragged tail."""
    announce(f"stats {gdt} n={n}")
    g = synth.stored_grad(n, 1e-2, 64.0, gdt, (0, "st", gdt, n)).to(DEV)
    k = min(n // 3, 11)
    if k:
        _inject(g, k, (0, "st", gdt, n, "pos"))
    gh = grad_host(g)
    s_ref, c_ref = oracle.grad_stats(gh, gdt)
    s_gpu, c_gpu, rows = _stats_gpu([g])
    assert c_gpu == c_ref == k
    exact = _exact_sumsq(gh, gdt)
    assert abs(s_gpu - exact) <= 1e-12 * exact
    assert abs(s_ref - exact) <= sequential_bound(n) * exact
    if n > 8192 * (4096 if gdt == "f32" else 8192):
        assert rows == 8192


def test_grad_stats_list_hierarchical_vs_flat_and_deterministic():
    announce("stats list hierarchical/flat")
    sizes = [5, 4096, 2047, 2049, 9_000_001, 17, 4_000_000, 640_001]
    grads = [synth.stored_grad(n, 1e-4, 1.0, "bf16", (0, "sl", i)).to(DEV) for i, n in enumerate(sizes)]
    _inject(grads[4], 5, (0, "sl", "pos"))
    acc = oracle.StatsAccumulator()
    for g in grads:
        acc.add(grad_host(g), "bf16")
    s_ref, c_ref = acc.result
    s_h, c_h, rows = _stats_gpu(grads, True)
    s_f, c_f, _ = _stats_gpu(grads, False)
    s_h2, c_h2, _ = _stats_gpu(grads, True)
    assert rows > 1024  # at least one intermediate merge level
    assert c_h == c_f == c_ref == 5
    assert s_h == s_h2 and c_h2 == c_h  # bit-identical repeat
    tol = sequential_bound(sum(sizes)) + 1e-12
    assert abs(s_h - s_ref) <= tol * s_ref and abs(s_f - s_ref) <= tol * s_ref


@pytest.mark.parametrize("nrows", [1, 1024, 1025, 1048576, 1048577, 4194304])
def test_merge_levels_on_synthetic_rows(nrows):
    """Rows with dyadic sums and known counts: the merged report is exact."""
    announce(f"merge rows={nrows}")
    r = torch.arange(nrows, device=DEV, dtype=torch.int64)
    vals = ((r % 7) + 1).double() * 0.25          # dyadic: every partial sum exact
    bits = vals.view(torch.int64)
    rows = torch.stack([(bits & 0xFFFFFFFF).to(torch.int64), (bits >> 32) & 0xFFFFFFFF, r % 3], dim=1)
    rows = rows.to(torch.int32).contiguous().view(-1)
    se, extra = ra.radamw_stats_plan(nrows)
    scratch = torch.zeros(max(se, 1), dtype=torch.float32, device=DEV)
    report = torch.zeros(3, dtype=torch.int32, device=DEV)
    before = ra.radamw_launch_count()
    ra.radamw_merge_stats(rows, nrows, scratch if se else None, report, True)
    assert ra.radamw_launch_count() == before + extra + 1
    rep = ra.radamw_read_report(report)
    assert rep.sumsq == float(vals.sum().item())
    assert rep.nonfinite == int((r % 3).sum().item())


def test_merge_count_saturates():
    nrows = 3000
    rows = torch.zeros(nrows, 3, dtype=torch.int64)
    rows[:, 2] = 0xFFFFFFF0
    rows = rows.to(torch.int32).view(-1).to(DEV)  # wraps to the same bit pattern
    report = torch.zeros(3, dtype=torch.int32, device=DEV)
    scratch = torch.zeros(ra.radamw_stats_plan(nrows)[0], device=DEV)
    ra.radamw_merge_stats(rows, nrows, scratch, report, True)
    assert ra.radamw_read_report(report).nonfinite == 2**32 - 1


def _fused_case(sizes, gdt, inject, max_norm, key, step0=0, amsgrad=False, hierarchical=True):
    opts = ra.options(lr=1e-3, weight_decay=1e-4, amsgrad=amsgrad)
    scale = 1.0
    segs, refs = [], []
    for i, n in enumerate(sizes):
        p0 = synth.normal(n, 0.02, key + (i, "p"))
        g = synth.stored_grad(n, 1e-4, 1.0, gdt, key + (i, "g")).to(DEV)
        st = new_gpu_state(n, amsgrad)
        segs.append(ra.Segment(p0.to(DEV), g, st.exp_avg, st.exp_avg_sq, st.max_exp_avg_sq))
        refs.append((p0.numpy().copy(), oracle.State(n, amsgrad)))
    if inject:
        _inject(segs[len(segs) // 2].grad, inject, key + ("pos",))
    acc = oracle.StatsAccumulator()
    for s in segs:
        acc.add(grad_host(s.grad), gdt)
    s_ref, c_ref = acc.result
    skip_ref, eff_ref = oracle.decide(s_ref, c_ref, scale, max_norm)
    ws = torch.zeros(ra.radamw_fused_workspace_bytes(segs), dtype=torch.uint8, device=DEV)
    before = ra.radamw_launch_count()
    snap = [s.param.clone() for s in segs]
    res, step = ra.radamw_fused_step_multi(segs, step0, opts, scale, max_norm, hierarchical, ws)
    torch.cuda.synchronize()
    assert res.nonfinite == c_ref and bool(res.found_inf) == skip_ref
    assert abs(res.sumsq - s_ref) <= (sequential_bound(sum(sizes)) + 1e-12) * max(s_ref, 1e-300)
    launched = ra.radamw_launch_count() - before
    nstats = len([n for n in sizes if n])
    if skip_ref:
        assert not res.updated and step == step0
        assert all(torch.equal(a, s.param) for a, s in zip(snap, segs))
        # one analysis launch for the whole list, the merge levels, the final merge, and the update
        # launches queued behind it, which read the device's skip decision and write nothing
        extra = ra.radamw_stats_plan(sum(ra.radamw_grad_stats_rows(n, TORCH_GDT[gdt]) for n in sizes))[1]
        solo = sum(1 for n in sizes if n >= 1 << 22)
        shared = sum(1 for n in sizes if 0 < n < 1 << 22)
        assert nstats > 1 and launched == 1 + extra + 1 + solo + (1 if shared else 0)
    else:
        assert res.updated and step == step0 + 1
        for (p_ref, st_ref), s in zip(refs, segs):
            oracle.adamw_step(p_ref, grad_host(s.grad), gdt, st_ref, oracle_opts(opts), eff_ref)
            contract_one_step(host(s.param), p_ref, "fused p")
            contract_one_step(host(s.exp_avg), st_ref.exp_avg, "fused m")
    return res


def test_fused_step_clips_when_norm_exceeds_max():
    announce("fused clip")
    res = _fused_case([4096, 1_000_000, 2049, 300_000], "bf16", 0, 0.05, (0, "fc"))
    assert res.clip_coef < 1.0 and res.total_norm > 0.05


def test_fused_step_without_clip_is_plain_update():
    announce("fused no clip")
    res = _fused_case([4096, 50_000], "f32", 0, 1e6, (0, "fn"))
    assert res.clip_coef == 1.0


def test_fused_step_decision_slot_with_odd_rows_and_workspace_alignment():
    """Three statistics rows (36 bytes): the decision moves to the last 8
    bytes of the workspace to stay 8-byte aligned, and the clipped step
    still matches the oracle.  A workspace that is only 4-byte aligned is
    rejected (RADAMW_ERR_ALIGN) before anything is launched."""
    announce("fused odd rows / workspace alignment")
    res = _fused_case([4096, 8192], "f32", 0, 1e-3, (0, "fodd"))
    assert res.clip_coef < 1.0
    segs = [ra.Segment(torch.zeros(n, device=DEV), torch.zeros(n, device=DEV), torch.zeros(n, device=DEV),
                       torch.zeros(n, device=DEV)) for n in (4096, 8192)]
    need = ra.radamw_fused_workspace_bytes(segs)
    assert need == 3 * 12 + 12
    ws = torch.zeros(need + 16, dtype=torch.uint8, device=DEV)
    before = ra.radamw_launch_count()
    with pytest.raises(ra.RadamwError) as e:
        ra.radamw_fused_step_multi(segs, 5, ra.options(), 1.0, 1.0, True, ws[4:4 + need])
    assert e.value.status == -4 and ra.radamw_launch_count() == before


def test_fused_step_behind_queued_work():
    """A fused step queued behind tens of milliseconds of other work on its
    stream (torch's bounded busy kernel): the host spins, then yields, then
    checks the stream now and then until the final merge writes this call's
    completion word, and the step still returns the oracle's result.  Two
    such steps in a row each wait for their own word."""
    announce("fused step behind queued work")
    for k in range(2):
        torch.cuda._sleep(50_000_000)
        res = _fused_case([4096, 300_000], "f32", 0, 0.05, (0, "fq", k))
        assert res.updated and res.clip_coef < 1.0


def test_fused_step_found_inf_skips_everything():
    announce("fused found_inf")
    res = _fused_case([4096, 1_000_000, 2049], "bf16", 3, 1.0, (0, "fi"), step0=4)
    assert res.found_inf and res.nonfinite == 3


@pytest.mark.parametrize("gdt", ["bf16", "f32"])
def test_fused_statistics_launch_equals_per_tensor_launches(gdt):
    """radamw_fused_step_multi analyses all gradients in one launch; its
    report is bit-identical to per-tensor radamw_grad_stats launches
    followed by the same merge (same rows, same order)."""
    announce(f"fused stats table {gdt}")
    sizes = [4096, 3, 9_000_001, 2047, 1_000_000, 8193, 65536]
    grads = [synth.stored_grad(n, 1e-3, 1.0, gdt, (0, "fst", gdt, i)).to(DEV) for i, n in enumerate(sizes)]
    _inject(grads[2], 4, (0, "fst", gdt, "pos"))
    s_ref, c_ref, rows = _stats_gpu(grads, True)
    assert rows > 1024
    segs = []
    for i, g in enumerate(grads):
        n = g.numel()
        segs.append(ra.Segment(torch.zeros(n, device=DEV), g, torch.zeros(n, device=DEV), torch.zeros(n, device=DEV)))
    ws = torch.empty(ra.radamw_fused_workspace_bytes(segs), dtype=torch.uint8, device=DEV)
    before = ra.radamw_launch_count()
    res, step = ra.radamw_fused_step_multi(segs, 3, ra.options(), 1.0, 1.0, True, ws)
    torch.cuda.synchronize()
    assert res.found_inf and not res.updated and step == 3
    assert res.nonfinite == c_ref == 4 and res.sumsq == s_ref
    extra = ra.radamw_stats_plan(rows)[1]
    # one analysis launch, merges, final merge, and the queued updates (9,000,001 alone, the rest shared)
    assert ra.radamw_launch_count() - before == 1 + extra + 1 + 2


def _norm_of(grads, gdt, scale):
    acc = oracle.StatsAccumulator()
    for g in grads:
        acc.add(grad_host(g), gdt)
    return math.sqrt(acc.result[0]) / scale


@pytest.mark.parametrize("gdt,scale,clip_at,maximize", [
    ("f32", 1.0, None, False),      # no clipping
    ("f32", 3.0, 0.5, False),       # clip active, non-power-of-two scale
    ("bf16", 1000.0, 2.0, True),    # maximize: the device takes the sign from the launch
    ("f16", 0.37, 1.0, False),      # scale below one
    ("bf16", 1.0, "at", False),     # max_norm equal to the norm: clip within rounding of 1
    ("f32", 7.0, 1e9, True),        # bound far above the norm: clip == 1
])
def test_device_decision_matches_host_decision(gdt, scale, clip_at, maximize):
    """The fused step decides on the device (the final merge writes skip and
    the clipped FP32 unscale factor; the queued update kernels read them);
    the same step composed from separate calls decides on the host
    (radamw_read_report + radamw_decide + radamw_step_multi).  Over five
    steps, every output bit agrees."""
    announce(f"device decision {gdt} scale={scale} clip={clip_at} max={maximize}")
    key = (0, "devdec", gdt, str(scale), str(clip_at), maximize)
    sizes = [3, 4096, 2049, 1_000_001, 5_000_000]
    opts = ra.options(lr=1e-3, weight_decay=1e-2, maximize=maximize)
    a, b = [], []
    for i, n in enumerate(sizes):
        p = synth.normal(n, 0.02, key + (i, "p")).to(DEV)
        mk = lambda: torch.zeros(n, device=DEV)
        a.append(ra.Segment(p, torch.empty(n, device=DEV, dtype=TORCH_GDT[gdt]), mk(), mk()))
        b.append(ra.Segment(p.clone(), a[-1].grad, mk(), mk()))
    ws = torch.empty(ra.radamw_fused_workspace_bytes(a), dtype=torch.uint8, device=DEV)
    rows_total = sum(ra.radamw_grad_stats_rows(n, TORCH_GDT[gdt]) for n in sizes)
    rows = torch.empty(3 * rows_total, dtype=torch.int32, device=DEV)
    scratch = torch.empty(max(1, ra.radamw_stats_plan(rows_total)[0]), device=DEV)
    report = torch.empty(3, dtype=torch.int32, device=DEV)
    sa = sb = 0
    for t in range(1, 6):
        for i, s in enumerate(a):
            s.grad.copy_(synth.stored_grad(sizes[i], 1e-3, scale, gdt, key + (i, "g", t)).to(DEV))
        max_norm = clip_at
        if clip_at == "at":
            max_norm = _norm_of([s.grad for s in a], gdt, scale)
        res, sa = ra.radamw_fused_step_multi(a, sa, opts, scale, max_norm, True, ws)
        off = 0
        for s in b:
            off += ra.radamw_grad_stats(s.grad, rows, off)
        ra.radamw_merge_stats(rows, rows_total, scratch, report, True)
        host = ra.radamw_read_report(report)
        ctrl, hres = ra.radamw_decide(host, scale, max_norm)
        updated, sb = ra.radamw_step_multi(b, sb, opts, ctrl)
        torch.cuda.synchronize()
        assert (res.sumsq, res.nonfinite, res.clip_coef, res.total_norm) == \
            (hres.sumsq, hres.nonfinite, hres.clip_coef, hres.total_norm)
        assert res.updated and updated and sa == sb == t
        if clip_at not in (None, 1e9):
            assert res.clip_coef <= 1.0
        for i, (x, y) in enumerate(zip(a, b)):
            for u, w, what in ((x.param, y.param, "p"), (x.exp_avg, y.exp_avg, "m"), (x.exp_avg_sq, y.exp_avg_sq, "v")):
                assert torch.equal(u.view(torch.int32), w.view(torch.int32)), f"step {t} tensor {i} {what}"
