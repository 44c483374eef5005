"""Full-size GPU parity: the 2^28 bucket (every update variant bench.py
times, the first step, the write-back of a BF16 model copy and the fused
step), the 1.1B-parameter 201-tensor list
(as separate tensors and as one flattened bucket), the 6.7B-parameter
291-tensor list with statistics, clipping and an injected non-finite step,
and one tensor beyond 32-bit indexing.

Every element of every output is compared with the oracle: each tensor's
pre-step state is kept on the device, staged through pinned host memory,
updated there by the C oracle (threads over contiguous slices), and the GPU's
result is compared with it on the device (gpu_helpers.compare_one_step_full:
the 1e-6 (1 + |ref|) contract on p, m, v, v_max and ulp bars on the
moments).  Statistics are checked over every gradient element.

Page abbreviations: FA-ja = "実験的なデバイス上の融合 AdamW / AMSGrad",
FA-zh = "实验性融合 AdamW / AMSGrad", TR-zh = "训练与状态保存"."""
import numpy as np
import pytest
import torch

import oracle
import synth
import optimizer_step_dl_amd as ra
from gpu_helpers import (DEV, PinnedStage, announce, bits_equal, compare_one_step_full, grad_host,
                         oracle_one_step_pinned, oracle_opts)

pytestmark = pytest.mark.gpu


def _bit_sum(t):
    """Sum of a tensor's 32-bit words as integers: an exact fingerprint of
    whether any word changed (up to a collision no bug produces)."""
    return int(t.view(torch.int32).sum(dtype=torch.int64))


def _clone(ts):
    return [None if t is None else t.clone() for t in ts]


@pytest.mark.parametrize("variant,gdt,mode", [
    ("adamw", "f32", "inplace"), ("adamw", "f32", "outofplace"), ("amsgrad", "f32", "inplace"),
    ("amsgrad", "f32", "outofplace"), ("adamw", "bf16", "inplace"), ("amsgrad", "f16", "inplace")])
def test_bucket_2pow28_steady_state(variant, gdt, mode):
    """The 268,435,456-element bucket at t = 1000 as bench.py builds it,
    updated the way bench.py's update-only variants launch it (one-segment
    radamw_step_multi in place, radamw_step out of place); every element of
    p, m, v (and v_max) against the oracle."""
    n = 1 << 28
    announce(f"bucket 2^28 {variant} {gdt} {mode}")
    amsgrad = variant == "amsgrad"
    key = (0, "bucket", n)
    p = synth.normal(n, 0.02, key + ("p",), DEV)
    g = synth.stored_grad(n, 1e-3, 1.0, gdt, key + ("g",), DEV)
    m, v, vmax = synth.steady_state(n, key, amsgrad, DEV, m_std=1e-4, v_root_std=1e-3)
    opts = ra.options(lr=1e-3, weight_decay=1e-4, amsgrad=amsgrad)
    if mode == "inplace":
        pre = _clone((p, m, v, vmax))
        updated, step = ra.radamw_step_multi([ra.Segment(p, g, m, v, vmax)], 999, opts, ra.control(1.0))
        assert updated and step == 1000
        outs = (p, m, v, vmax)
    else:
        pre = (p, m, v, vmax)
        sums = [_bit_sum(t) for t in pre if t is not None]
        outs = (torch.empty_like(p), torch.empty_like(m), torch.empty_like(v),
                torch.empty_like(vmax) if amsgrad else None)
        st_out = ra.AdamWState(0, outs[1], outs[2], outs[3])
        assert ra.radamw_step(p, g, ra.AdamWState(999, m, v, vmax), opts, ra.control(1.0), outs[0], st_out)
        assert st_out.step == 1000
        torch.cuda.synchronize()
        assert [_bit_sum(t) for t in pre if t is not None] == sums  # inputs untouched
    torch.cuda.synchronize()
    stage = PinnedStage()
    ref = oracle_one_step_pinned(stage, pre, g, gdt, oracle_opts(opts), 1.0, 999, amsgrad)
    stats = {}
    compare_one_step_full(f"bucket {variant} {gdt} {mode}", outs, ref, pre, g, 1.0, 0.9, 0.999,
                          first=False, power_of_two=True, stats=stats)
    announce(f"largest moment errors in units of their ulp bars: {stats}")
    if amsgrad:
        assert bool(torch.all(outs[3] >= outs[2]))


def test_bucket_2pow28_first_step():
    """The bucket's first step (no state: FA-zh "增加的实际能力"), as bench.py's
    first-step variant launches it: m and v start as NaN-filled buffers, so
    any read of them would poison the result; every element of p, m and v
    against the oracle's first step."""
    n = 1 << 28
    announce("bucket 2^28 first step")
    key = (0, "bucket", n)
    p = synth.normal(n, 0.02, key + ("p",), DEV)
    g = synth.stored_grad(n, 1e-3, 1.0, "f32", key + ("g",), DEV)
    m = torch.full((n,), float("nan"), device=DEV)
    v = torch.full((n,), float("nan"), device=DEV)
    opts = ra.options(lr=1e-3, weight_decay=1e-4)
    pre = (p.clone(), m.clone(), v.clone(), None)
    st = ra.AdamWState(0, m, v, None)
    assert ra.radamw_step_inplace(p, g, st, opts, ra.control(1.0)) and st.step == 1
    torch.cuda.synchronize()
    stage = PinnedStage()
    ref = oracle_one_step_pinned(stage, pre, g, "f32", oracle_opts(opts), 1.0, 0, False)
    stats = {}
    compare_one_step_full("bucket first step", (p, m, v, None), ref, pre, g, 1.0, 0.9, 0.999,
                          first=True, power_of_two=True, stats=stats)
    announce(f"largest moment errors in units of their ulp bars: {stats}")


def test_bucket_2pow28_bf16_model_copy():
    """The bucket's update with the BF16 model copy written in the same pass
    (bench.py's write-back variant): p, m, v against the oracle element by
    element; the copy equals torch's round-to-nearest-even conversion of the
    updated p bit for bit, and the oracle's rounding of its own p within the
    contract on p plus one BF16 unit."""
    n = 1 << 28
    announce("bucket 2^28 with BF16 model copy")
    key = (0, "bucket", n)
    p = synth.normal(n, 0.02, key + ("p",), DEV)
    g = synth.stored_grad(n, 1e-3, 1.0, "f32", key + ("g",), DEV)
    m, v, _ = synth.steady_state(n, key, False, DEV, m_std=1e-4, v_root_std=1e-3)
    opts = ra.options(lr=1e-3, weight_decay=1e-4)
    pre = _clone((p, m, v, None))
    model = torch.full((n,), 7.0, dtype=torch.bfloat16, device=DEV)
    updated, step = ra.radamw_step_multi_writeback([ra.Segment(p, g, m, v, None)], [model], 999, opts,
                                                   ra.control(1.0))
    assert updated and step == 1000
    torch.cuda.synchronize()
    assert torch.equal(model.view(torch.int16), p.to(torch.bfloat16).view(torch.int16))
    stage = PinnedStage()
    ref = oracle_one_step_pinned(stage, pre, g, "f32", oracle_opts(opts), 1.0, 999, False)
    compare_one_step_full("bucket with model copy", (p, m, v, None), ref, pre, g, 1.0, 0.9, 0.999,
                          first=False, power_of_two=True)
    ref_bits = torch.from_numpy(oracle.round_copy(ref[0].numpy(), "bf16").view(np.int16))
    chunk = 1 << 25
    same = 0
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        ours = model[lo:hi].double()
        want = ref_bits[lo:hi].to(DEV).view(torch.bfloat16).double()
        p_ref = ref[0][lo:hi].to(DEV).double()
        bound = 1e-6 * (1 + p_ref.abs()) + 2.0**-7 * p_ref.abs() + 2.0**-24
        assert bool(torch.all((ours - want).abs() <= bound)), f"model copy, elements {lo}..{hi}"
        same += int(torch.count_nonzero(ours == want))
    assert same > 0.99 * n


def test_bucket_2pow28_fused_step_as_benched():
    """The headline step exactly as bench.py times it: one
    radamw_fused_step_multi call over the one-segment 2^28 bucket (FP32
    grads, AdamW, t = 1000) with hierarchical statistics and a clip at
    max_grad_norm = 1.0 (the norm is ~16.4, so the clip is active).  The
    report's count is the oracle's over all 2^28 gradients bit for bit and its
    sum lies within the oracle's sequential FP64 bound; the clip coefficient
    is the oracle's rule applied to the report, bit for bit; every element
    matches the oracle run at the clipped scale."""
    n = 1 << 28
    announce("bucket 2^28 fused step as benched")
    key = (0, "bucket", n)
    p = synth.normal(n, 0.02, key + ("p",), DEV)
    g = synth.stored_grad(n, 1e-3, 1.0, "f32", key + ("g",), DEV)
    m, v, _ = synth.steady_state(n, key, False, DEV, m_std=1e-4, v_root_std=1e-3)
    opts = ra.options(lr=1e-3, weight_decay=1e-4)
    seglist = ra.SegmentList([ra.Segment(p, g, m, v, None)])
    ws = torch.empty(ra.radamw_fused_workspace_bytes(seglist), dtype=torch.uint8, device=DEV)
    pre = _clone((p, m, v, None))
    sumsq, count = oracle.grad_stats(grad_host(g), "f32")
    res, step = ra.radamw_fused_step_multi(seglist, 999, opts, 1.0, 1.0, True, ws)
    torch.cuda.synchronize()
    assert res.updated and not res.found_inf and step == 1000
    assert res.nonfinite == count == 0
    assert abs(res.sumsq - sumsq) <= (n - 1) * 2.0**-53 * sumsq
    clip = oracle.clip_coefficient(res.sumsq, 1.0, 1.0)
    assert res.clip_coef == clip and 0.0 < clip < 1.0
    skip, eff = oracle.decide(res.sumsq, res.nonfinite, 1.0, 1.0)
    assert not skip
    ref = oracle_one_step_pinned(PinnedStage(), pre, g, "f32", oracle_opts(opts), eff, 999, False)
    stats = {}
    compare_one_step_full("fused bucket", (p, m, v, None), ref, pre, g, eff, 0.9, 0.999, first=False,
                          power_of_two=False, stats=stats)
    announce(f"largest moment errors in units of their ulp bars: {stats}")


def _decoder_segments(shapes, gdt, scale, amsgrad, step, key, std):
    """Pre-warmed state for t = step + 1: m ~ N(0, 0.1 sigma), v = N(0, sigma)^2,
    v_max = v * U(1, 1.5), sigma the unscaled gradient's standard deviation."""
    segs = []
    for i, (name, n) in enumerate(shapes):
        p = synth.normal(n, 0.02, key + (i, "p"), DEV)
        g = synth.stored_grad(n, std, scale, gdt, key + (i, "g"), DEV)
        if step > 0:
            m, v, vmax = synth.steady_state(n, key + (i,), amsgrad, DEV, m_std=0.1 * std, v_root_std=std)
        else:
            m, v = torch.empty(n, device=DEV), torch.empty(n, device=DEV)
            vmax = torch.empty(n, device=DEV) if amsgrad else None
        segs.append(ra.Segment(p, g, m, v, vmax))
    return segs


def _seg_state(s):
    return (s.param, s.exp_avg, s.exp_avg_sq, s.max_exp_avg_sq)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("odd", [False, True])
def test_decoder_1b_list_multi_call_vs_per_tensor(odd):
    """201 tensors shaped like a 1.1B decoder (odd variant: norms 2047/2049),
    FP16 grads N(0,1e-4)*1024 with scale 1024, AMSGrad, t = 50: one
    radamw_step_multi call (the 156 tensors of >= 2^22 elements launched
    alone, the 45 norm vectors in one shared launch) equals 201
    radamw_step_inplace launches bit for bit, and every element of every
    tensor matches the oracle."""
    shapes = synth.decoder_1b_shapes(odd)
    announce(f"decoder 1.1B list odd={odd}")
    opts = ra.options(lr=1e-3, weight_decay=1e-4, amsgrad=True)
    oo = oracle_opts(opts)
    scale = 1024.0
    segs = _decoder_segments(shapes, "f16", scale, True, 49, (0, "dec1b", odd), 1e-4)
    twins = [ra.Segment(s.param.clone(), s.grad, s.exp_avg.clone(), s.exp_avg_sq.clone(), s.max_exp_avg_sq.clone())
             for s in segs]
    launches = ra.radamw_launch_count()
    updated, step = ra.radamw_step_multi(segs, 49, opts, ra.control(scale))
    solo = sum(1 for _, n in shapes if n >= 1 << 22)
    shared = sum(1 for _, n in shapes if n < 1 << 22)
    assert (solo, shared) == (156, 45)
    assert updated and step == 50 and ra.radamw_launch_count() == launches + solo + 1
    torch.cuda.synchronize()
    stage, stats = PinnedStage(), {}
    for i, (s, tw) in enumerate(zip(segs, twins)):
        # the twin still holds the pre-step state: the oracle starts from it
        ref = oracle_one_step_pinned(stage, _seg_state(tw), tw.grad, "f16", oo, scale, 49, True)
        compare_one_step_full(shapes[i][0], _seg_state(s), ref, _seg_state(tw), s.grad, scale, 0.9, 0.999,
                              first=False, power_of_two=True, stats=stats)
        assert ra.radamw_step_inplace(tw.param, tw.grad, ra.AdamWState(49, tw.exp_avg, tw.exp_avg_sq,
                                                                       tw.max_exp_avg_sq), opts, ra.control(scale))
        torch.cuda.synchronize()
        assert bits_equal(s.param, tw.param) and bits_equal(s.exp_avg, tw.exp_avg), shapes[i][0]
        assert bits_equal(s.exp_avg_sq, tw.exp_avg_sq) and bits_equal(s.max_exp_avg_sq, tw.max_exp_avg_sq)
    announce(f"largest moment errors in units of their ulp bars: {stats}")


@pytest.mark.timeout(600)
def test_decoder_1b_flattened_bucket():
    """The 1.1B decoder's state as one flattened bucket (FA-ja
    "サポートされている契約": a pre-flattened bucket, sharing options and the
    step count): p, the FP16 gradient, m, v and v_max each one contiguous
    allocation of 1,261,529,088 elements, updated by one radamw_step_multi
    call over a single segment, i.e. one launch.  Every element matches the
    oracle, and each tensor's slice equals a per-tensor launch over the same
    slice of a twin arena bit for bit."""
    shapes = synth.decoder_1b_shapes()
    total = synth.total(shapes)
    announce(f"decoder 1.1B flattened bucket ({total} params)")
    opts = ra.options(lr=1e-3, weight_decay=1e-4, amsgrad=True)
    oo = oracle_opts(opts)
    scale = 1024.0
    arena = [torch.empty(total, device=DEV), torch.empty(total, dtype=torch.float16, device=DEV)] + \
        [torch.empty(total, device=DEV) for _ in range(3)]
    spans, off = [], 0
    for i, (_, n) in enumerate(shapes):
        key = (0, "dec1b-flat", i)
        arena[0][off:off + n] = synth.normal(n, 0.02, key + ("p",), DEV)
        arena[1][off:off + n] = synth.stored_grad(n, 1e-4, scale, "f16", key + ("g",), DEV)
        m, v, vmax = synth.steady_state(n, key, True, DEV, m_std=1e-5, v_root_std=1e-4)
        arena[2][off:off + n], arena[3][off:off + n], arena[4][off:off + n] = m, v, vmax
        spans.append((off, n))
        off += n
    twin = [t.clone() if k != 1 else t for k, t in enumerate(arena)]
    launches = ra.radamw_launch_count()
    updated, step = ra.radamw_step_multi([ra.Segment(*arena)], 49, opts, ra.control(scale))
    assert updated and step == 50 and ra.radamw_launch_count() == launches + 1
    torch.cuda.synchronize()
    stage, stats = PinnedStage(), {}
    for i, (o, n) in enumerate(spans):
        a = [t[o:o + n] for t in arena]
        b = [t[o:o + n] for t in twin]
        pre = (b[0], b[2], b[3], b[4])
        ref = oracle_one_step_pinned(stage, pre, b[1], "f16", oo, scale, 49, True)
        compare_one_step_full(f"flat {shapes[i][0]}", (a[0], a[2], a[3], a[4]), ref, pre, a[1], scale, 0.9, 0.999,
                              first=False, power_of_two=True, stats=stats)
        assert ra.radamw_step_inplace(b[0], b[1], ra.AdamWState(49, b[2], b[3], b[4]), opts, ra.control(scale))
    torch.cuda.synchronize()
    for k in (0, 2, 3, 4):
        assert bits_equal(arena[k], twin[k])
    announce(f"largest moment errors in units of their ulp bars: {stats}")


def _oracle_stats(segs):
    acc = oracle.StatsAccumulator()
    for s in segs:
        acc.add(grad_host(s.grad), "bf16")
    return acc.result


@pytest.mark.timeout(900)
def test_decoder_7b_list_stats_clip_skip_sequence():
    """291 tensors shaped like a 6.7B decoder, BF16 grads N(0,1e-4), scale 1,
    in-place AdamW from no state: fused step (stats -> hierarchical merge ->
    12-byte read-back -> clip at 1.0 -> update) at t = 1; then a step with
    round(1e-6 * N) = 6,738 injected +inf/NaN values, which must report
    exactly that count and skip; then a clean step at t = 2.  Statistics are
    checked against the oracle over every element; each update over every
    element, as one step from the state it started from."""
    shapes = synth.decoder_7b_shapes()
    total = synth.total(shapes)
    announce(f"decoder 6.7B list ({total} params)")
    opts = ra.options(lr=1e-3, weight_decay=1e-4)
    oo = oracle_opts(opts)
    segs = _decoder_segments(shapes, "bf16", 1.0, False, 0, (0, "dec7b"), 1e-4)
    ws = torch.empty(ra.radamw_fused_workspace_bytes(segs), dtype=torch.uint8, device=DEV)
    offsets = np.cumsum([0] + [n for _, n in shapes])
    stage, stats = PinnedStage(), {}

    def fused(step, call):
        announce(f"decoder 6.7B fused call {call}")
        sumsq, count = _oracle_stats(segs)
        skip, eff = oracle.decide(sumsq, count, 1.0, 1.0)
        pre = [_clone(_seg_state(s)) for s in segs] if not skip else None
        res, new_step = ra.radamw_fused_step_multi(segs, step, opts, 1.0, 1.0, True, ws)
        torch.cuda.synchronize()
        assert res.nonfinite == count and bool(res.found_inf) == skip
        # The oracle sums 6.7e9 squares left to right in FP64; its a-priori
        # rounding bound is (n - 1) * 2^-53 ~ 7.5e-7 relative, and with bf16
        # squares its rounding is one-sided (odd squares are 1 mod 8), so it
        # drifts low by ~5e-9 here.  The GPU's tree sums are exact to ~1e-15
        # (pinned against fsum-exact sums in the statistics tests).
        assert abs(res.sumsq - sumsq) <= (total - 1) * 2.0**-53 * sumsq
        assert bool(res.updated) == (not skip) and new_step == step + (0 if skip else 1)
        if not skip:
            # the device decided with the report's own sum: the clip it applied
            _, eff_dev = oracle.decide(res.sumsq, res.nonfinite, 1.0, 1.0)
            for i, s in enumerate(segs):
                ref = oracle_one_step_pinned(stage, pre[i], s.grad, "bf16", oo, eff_dev, step, False)
                compare_one_step_full(f"{shapes[i][0]} call {call}", _seg_state(s), ref, pre[i], s.grad, eff_dev,
                                      0.9, 0.999, first=step == 0, power_of_two=False, stats=stats)
                pre[i] = None
        return res, new_step

    res, step = fused(0, 1)
    assert step == 1 and 0.0 < res.clip_coef < 1.0  # norm ~ sqrt(N) * 1e-4 ~ 8.2 > 1
    # injected step: fresh grads with 6,738 non-finite values at seeded global positions
    k = round(1e-6 * total)
    pos = synth.nonfinite_positions(total, k, (0, "dec7b", "inject"))
    vals = synth.nonfinite_values(k)
    for i, s in enumerate(segs):
        s.grad.copy_(synth.stored_grad(s.grad.numel(), 1e-4, 1.0, "bf16", (0, "dec7b", i, "g2"), DEV))
        lo, hi = np.searchsorted(pos, [offsets[i], offsets[i + 1]])
        if hi > lo:
            local = torch.from_numpy(pos[lo:hi] - offsets[i]).to(DEV)
            s.grad[local] = torch.tensor(vals[lo:hi], dtype=torch.bfloat16, device=DEV)
    launches = ra.radamw_launch_count()
    sums = [tuple(_bit_sum(t) for t in (s.param, s.exp_avg, s.exp_avg_sq)) for s in segs]
    res, step = fused(step, 2)
    assert res.found_inf and res.nonfinite == k == 6738 and step == 1 and not res.updated
    # statistics ran and the update kernels queued behind them read the skip and wrote nothing
    assert ra.radamw_launch_count() > launches
    assert [tuple(_bit_sum(t) for t in (s.param, s.exp_avg, s.exp_avg_sq)) for s in segs] == sums
    # clean step at t = 2
    for i, s in enumerate(segs):
        s.grad.copy_(synth.stored_grad(s.grad.numel(), 1e-4, 1.0, "bf16", (0, "dec7b", i, "g3"), DEV))
    res, step = fused(step, 3)
    assert step == 2 and res.updated and not res.found_inf
    announce(f"largest moment errors in units of their ulp bars: {stats}")


@pytest.mark.timeout(600)
def test_single_tensor_beyond_32_bit_indexing():
    """One tensor of 2^32 + 1029 elements (64-bit indexing in every kernel):
    in-place AdamW with BF16 grads at t = 3 and its statistics, with one inf
    past 2^32 and one NaN below 2^31.  Every element with a finite gradient
    matches the oracle (a non-finite gradient is outside the formula's
    contract); statistics over every element (count exact, sum within the
    sequential bound)."""
    n = (1 << 32) + 1029
    announce(f"single tensor n={n}")
    p = synth.normal(n, 0.02, (0, "huge", "p"), DEV)
    g = synth.stored_grad(n, 1e-3, 1.0, "bf16", (0, "huge", "g"), DEV)
    m, v, _ = synth.steady_state(n, (0, "huge"), False, DEV)
    g[(1 << 32) + 17] = float("inf")
    g[(1 << 31) - 1] = float("nan")
    opts = ra.options(lr=1e-3, weight_decay=0.01)
    # statistics over everything
    rows = ra.radamw_grad_stats_rows(n, torch.bfloat16)
    rows_buf = torch.zeros(3 * rows, dtype=torch.int32, device=DEV)
    assert ra.radamw_grad_stats(g, rows_buf) == rows
    se, _ = ra.radamw_stats_plan(rows)
    report = torch.zeros(3, dtype=torch.int32, device=DEV)
    ra.radamw_merge_stats(rows_buf, rows, torch.zeros(max(se, 1), device=DEV) if se else None, report, True)
    rep = ra.radamw_read_report(report)
    acc = oracle.StatsAccumulator()
    chunk = 1 << 28
    for lo in range(0, n, chunk):
        acc.add(grad_host(g[lo:lo + chunk]), "bf16")
    s_ref, c_ref = acc.result
    assert rep.nonfinite == c_ref == 2
    assert abs(rep.sumsq - s_ref) <= (n - 1) * 2.0**-53 * s_ref
    pre = _clone((p, m, v, None))
    updated, step = ra.radamw_step_multi([ra.Segment(p, g, m, v)], 2, opts, ra.control(1.0))
    assert updated and step == 3
    torch.cuda.synchronize()
    # the update is elementwise: the oracle takes the tensor in 2^28-element slices
    stage = PinnedStage()
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        pre_c = tuple(None if t is None else t[lo:hi] for t in pre)
        ref = oracle_one_step_pinned(stage, pre_c, g[lo:hi], "bf16", oracle_opts(opts), 1.0, 2, False)
        compare_one_step_full(f"n = 2^32 + 1029, [{lo}, {hi})", (p[lo:hi], m[lo:hi], v[lo:hi], None), ref, pre_c,
                              g[lo:hi], 1.0, 0.9, 0.999, first=False, power_of_two=True, finite_only=True)
    assert int(torch.isfinite(g).logical_not().sum()) == 2
