"""Persistent tensor lists (radamw_list_*): a list validated once and stepped
many times gives the bits of the per-call entry points (radamw_step_multi,
radamw_step_multi_writeback, radamw_fused_step_multi) on the same tensors,
and the oracle's values within the one-step contract bar."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
import optimizer_step_dl_amd as ra
from gpu_helpers import (DEV, TORCH_GDT, announce, bits_equal, check_step_from, clone_state, contract_one_step,
                         grad_host, host, new_gpu_state, normwise, oracle_opts)

pytestmark = pytest.mark.gpu

SOLO = 1 << 22  # tensors this large get a launch of their own
# empty, single and ragged tensors share one launch; two large tensors go alone
SIZES = [0, 1, 5, 4096, 4097, 2047, 2049, 100_000, 3, 70_001, SOLO, SOLO + 5]


def _make(sizes, gdt, amsgrad, key, misaligned=True):
    """Segments with step-0 (NaN-filled) state and the oracle's twins.  With
    `misaligned`, segment 3's parameter is a view one element into a larger
    buffer, so its streams sit at different 16-byte phases (scalar path)."""
    segs, refs = [], []
    for i, n in enumerate(sizes):
        p0 = synth.normal(n, 0.02, key + (i, "p"))
        if misaligned and i == 3:
            buf = torch.empty(n + 1, device=DEV)
            p = buf[1:]
            p.copy_(p0.to(DEV))
        else:
            p = p0.to(DEV)
        st = new_gpu_state(n, amsgrad)
        segs.append(ra.Segment(p, torch.empty(n, device=DEV, dtype=TORCH_GDT[gdt]), st.exp_avg, st.exp_avg_sq,
                               st.max_exp_avg_sq))
        refs.append((p0.numpy().copy(), oracle.State(n, amsgrad)))
    return segs, refs


def _fill_grads(segs, twins, sizes, gdt, scale, key, t):
    for i, (s, tw) in enumerate(zip(segs, twins)):
        g = synth.stored_grad(sizes[i], 1e-4, scale, gdt, key + (i, "g", t))
        s.grad.copy_(g.to(DEV))
        tw.grad.copy_(s.grad)


def _pre(segs):
    return [clone_state(s.param, ra.AdamWState(0, s.exp_avg, s.exp_avg_sq, s.max_exp_avg_sq)) for s in segs]


def _one_step_checks(segs, pres, sizes, gdt, opts, scale, step_before, what):
    """Every element of every non-empty segment against the oracle run one
    update from the segment's own pre-step state (contract + moment ulps)."""
    for i, (s, pre) in enumerate(zip(segs, pres)):
        if sizes[i]:
            check_step_from(pre, (s.param, s.exp_avg, s.exp_avg_sq, s.max_exp_avg_sq), s.grad, gdt, opts, scale,
                            step_before, f"{what} segment {i} n={sizes[i]}")


def _same_bits(a: ra.Segment, b: ra.Segment, amsgrad: bool, what: str):
    assert bits_equal(a.param, b.param), f"{what}: param"
    assert bits_equal(a.exp_avg, b.exp_avg), f"{what}: exp_avg"
    assert bits_equal(a.exp_avg_sq, b.exp_avg_sq), f"{what}: exp_avg_sq"
    if amsgrad:
        assert bits_equal(a.max_exp_avg_sq, b.max_exp_avg_sq), f"{what}: max_exp_avg_sq"


@pytest.mark.parametrize("gdt,amsgrad", [("bf16", True), ("f32", False), ("f16", False)])
def test_list_step_matches_step_multi_and_oracle(gdt, amsgrad):
    announce(f"list step {gdt} ams={amsgrad}")
    key = (0, "list", gdt, amsgrad)
    opts = ra.options(lr=1e-3, weight_decay=0.01, amsgrad=amsgrad)
    scale = 128.0
    segs, refs = _make(SIZES, gdt, amsgrad, key)
    twins, _ = _make(SIZES, gdt, amsgrad, key)
    solo = sum(1 for n in SIZES if n >= SOLO)
    with ra.TensorList(segs, amsgrad) as lst:
        step = tstep = 0
        for t in range(1, 4):
            _fill_grads(segs, twins, SIZES, gdt, scale, key, t)
            for i, s in enumerate(segs):
                if SIZES[i]:
                    oracle.adamw_step(refs[i][0], grad_host(s.grad), gdt, refs[i][1], oracle_opts(opts), scale)
            pres = _pre(segs)
            before = ra.radamw_launch_count()
            updated, step = lst.step(step, opts, ra.control(scale))
            assert updated and step == t
            assert ra.radamw_launch_count() - before == solo + 1  # no table staging: launches only
            _, tstep = ra.radamw_step_multi(twins, tstep, opts, ra.control(scale))
            torch.cuda.synchronize()
            _one_step_checks(segs, pres, SIZES, gdt, opts, scale, t - 1, f"list step {t}")
            for i, (s, tw) in enumerate(zip(segs, twins)):
                _same_bits(s, tw, amsgrad, f"step {t} segment {i} n={SIZES[i]}")
                if t == 1 and SIZES[i]:
                    contract_one_step(host(s.param), refs[i][0], f"segment {i} p")
                    contract_one_step(host(s.exp_avg), refs[i][1].exp_avg, f"segment {i} m")
                    contract_one_step(host(s.exp_avg_sq), refs[i][1].exp_avg_sq, f"segment {i} v")
        for i, s in enumerate(segs):
            if SIZES[i]:
                normwise(host(s.param), refs[i][0], f"segment {i} p after 3 steps")
                normwise(host(s.exp_avg_sq), refs[i][1].exp_avg_sq, f"segment {i} v after 3 steps")
        # skip_update: nothing launched, nothing written, step unchanged
        snap = [s.param.clone() for s in segs]
        before = ra.radamw_launch_count()
        updated, step2 = lst.step(step, opts, ra.control(scale, True))
        assert not updated and step2 == step and ra.radamw_launch_count() == before
        torch.cuda.synchronize()
        assert all(torch.equal(a, s.param) for a, s in zip(snap, segs))


def test_list_fused_step_matches_fused_multi_and_oracle():
    """Statistics -> merge -> read-back -> clip -> update through a list,
    step by step against radamw_fused_step_multi: identical reports and
    states, including an injected non-finite step that skips everything."""
    announce("list fused step bf16")
    gdt, key, max_norm = "bf16", (0, "listf"), 0.05
    opts = ra.options(lr=1e-3, weight_decay=1e-4)
    segs, refs = _make(SIZES, gdt, False, key)
    twins, _ = _make(SIZES, gdt, False, key)
    ws = torch.empty(ra.radamw_fused_workspace_bytes(twins), dtype=torch.uint8, device=DEV)
    with ra.TensorList(segs, False) as lst:
        step = tstep = 0
        for t in range(1, 6):
            _fill_grads(segs, twins, SIZES, gdt, 1.0, key, t)
            if t == 4:  # one +inf in the largest gradient: the whole step is skipped
                segs[-1].grad[12345] = float("inf")
                twins[-1].grad[12345] = float("inf")
            if t == 1:
                acc = oracle.StatsAccumulator()
                for s in segs:
                    acc.add(grad_host(s.grad), gdt)
                skip_ref, eff_ref = oracle.decide(*acc.result, 1.0, max_norm)
                assert not skip_ref
            pres, step_before = _pre(segs), step
            res, step = lst.fused_step(step, opts, 1.0, max_norm, True)
            tres, tstep = ra.radamw_fused_step_multi(twins, tstep, opts, 1.0, max_norm, True, ws)
            torch.cuda.synchronize()
            if res.updated:  # one update at the clip the report decided
                _, eff = oracle.decide(res.sumsq, res.nonfinite, 1.0, max_norm)
                _one_step_checks(segs, pres, SIZES, gdt, opts, eff, step_before, f"fused step {t}")
            assert (res.sumsq, res.nonfinite, res.found_inf, res.updated, res.clip_coef, res.total_norm) == \
                (tres.sumsq, tres.nonfinite, tres.found_inf, tres.updated, tres.clip_coef, tres.total_norm)
            assert step == tstep
            if t == 4:
                assert res.found_inf and res.nonfinite == 1 and not res.updated and step == 3
            else:
                assert res.updated and res.clip_coef < 1.0
            for i, (s, tw) in enumerate(zip(segs, twins)):
                _same_bits(s, tw, False, f"fused step {t} segment {i}")
            if t == 1:
                for i, s in enumerate(segs):
                    if SIZES[i]:
                        oracle.adamw_step(refs[i][0], grad_host(s.grad), gdt, refs[i][1], oracle_opts(opts), eff_ref)
                        contract_one_step(host(s.param), refs[i][0], f"fused segment {i} p")
        assert step == 4


def test_list_writeback_matches_multi_writeback():
    announce("list write-back")
    gdt, key = "f32", (0, "listwb")
    opts = ra.options(lr=1e-3, weight_decay=1e-4)
    segs, _ = _make(SIZES, gdt, False, key)
    twins, _ = _make(SIZES, gdt, False, key)
    models = [None if i % 4 == 1 else torch.zeros(n, dtype=torch.bfloat16, device=DEV) for i, n in enumerate(SIZES)]
    tmodels = [None if m is None else torch.zeros_like(m) for m in models]
    with ra.TensorList(segs, False, models) as lst:
        step = tstep = 0
        for t in range(1, 3):
            _fill_grads(segs, twins, SIZES, gdt, 1.0, key, t)
            _, step = lst.step(step, opts, ra.control())
            _, tstep = ra.radamw_step_multi_writeback(twins, tmodels, tstep, opts, ra.control())
        torch.cuda.synchronize()
        assert step == tstep == 2
        for i, (s, tw) in enumerate(zip(segs, twins)):
            _same_bits(s, tw, False, f"write-back segment {i}")
            if models[i] is not None:
                assert torch.equal(models[i].view(torch.int16), tmodels[i].view(torch.int16))
                want = oracle.round_copy(host(s.param), "bf16")
                assert np.array_equal(host(models[i].view(torch.int16)).view(np.uint16), want)


def test_list_rejections_and_empty_lists():
    announce("list rejections")
    n = 1000
    mk = lambda: torch.zeros(n, device=DEV)
    seg = ra.Segment(mk(), mk(), mk(), mk())
    with ra.TensorList([seg], False) as lst:
        with pytest.raises(ra.RadamwError) as e:  # AMSGrad flag differs from the list's
            lst.step(0, ra.options(amsgrad=True), ra.control())
        assert e.value.status == -2
        with pytest.raises(ra.RadamwError) as e:
            lst.fused_step(0, ra.options(), -1.0, None, True)
        assert e.value.status == -1
    with pytest.raises(RuntimeError):
        lst.step(0, ra.options(), ra.control())
    # overlapping written ranges are refused at creation
    shared = mk()
    with pytest.raises(ra.RadamwError) as e:
        ra.TensorList([ra.Segment(mk(), mk(), shared, mk()), ra.Segment(mk(), mk(), shared, mk())], False)
    assert e.value.status == -3
    # AMSGrad list without v_max buffers
    with pytest.raises(ra.RadamwError) as e:
        ra.TensorList([seg], True)
    assert e.value.status == -2
    # an all-empty list launches nothing and never steps
    empty = ra.Segment(torch.empty(0, device=DEV), torch.empty(0, device=DEV), torch.empty(0, device=DEV),
                       torch.empty(0, device=DEV))
    with ra.TensorList([empty, empty], False) as lst:
        before = ra.radamw_launch_count()
        assert lst.step(7, ra.options(), ra.control()) == (False, 7)
        res, step = lst.fused_step(7, ra.options(), 1.0, 1.0, True)
        assert step == 7 and not res.updated and res.clip_coef == 1.0
        assert ra.radamw_launch_count() == before


def test_list_fused_launch_count_and_reuse():
    """A fused list step is one analysis launch, the merges and the update
    launches; many steps reuse the same device tables."""
    announce("list fused launches")
    gdt, key = "f32", (0, "listlc")
    sizes = [SOLO, 4096, 33, 2_000_000]
    segs, _ = _make(sizes, gdt, False, key, misaligned=False)
    for i, s in enumerate(segs):
        s.grad.copy_(synth.stored_grad(sizes[i], 1e-4, 1.0, gdt, key + (i, "g")).to(DEV))
    rows = sum(ra.radamw_grad_stats_rows(n, torch.float32) for n in sizes)
    extra = ra.radamw_stats_plan(rows)[1]
    with ra.TensorList(segs, False) as lst:
        step = 0
        for t in range(1, 21):
            before = ra.radamw_launch_count()
            res, step = lst.fused_step(step, ra.options(), 1.0, 1.0, True)
            assert res.updated and step == t
            assert ra.radamw_launch_count() - before == 1 + extra + 1 + 2  # stats, merges, solo + shared
    torch.cuda.synchronize()
    assert all(torch.isfinite(s.param).all() for s in segs)


def test_lists_fused_step_two_groups_match_oracle():
    """Two parameter groups (AMSGrad with strong decay; AdamW) at different
    step counts: one statistics reduction over both, one clip decision, each
    group updated with its own options; an injected NaN skips both."""
    announce("lists fused step, two groups")
    gdt, key, max_norm, scale = "f16", (0, "lists2"), 0.05, 1024.0
    sizes_a, sizes_b = [4096, 2049, SOLO + 3], [1, 70_001, 0, 3000]
    opts_a = ra.options(lr=1e-2, weight_decay=0.1, amsgrad=True)
    opts_b = ra.options(lr=1e-3, weight_decay=0.01)
    segs_a, refs_a = _make(sizes_a, gdt, True, key + ("a",), misaligned=False)
    segs_b, refs_b = _make(sizes_b, gdt, False, key + ("b",), misaligned=False)
    groups = [(segs_a, refs_a, sizes_a, opts_a), (segs_b, refs_b, sizes_b, opts_b)]
    # group b starts three updates behind group a's count
    steps = [3, 0]
    for r in refs_a:
        r[1].step = 3
    for s in segs_a:  # a steady state for the AMSGrad group, mirrored into the oracle
        s.exp_avg.fill_(1e-5); s.exp_avg_sq.fill_(1e-8); s.max_exp_avg_sq.fill_(2e-8)
    for r in refs_a:
        r[1].exp_avg[:] = np.float32(1e-5); r[1].exp_avg_sq[:] = np.float32(1e-8)
        r[1].max_exp_avg_sq[:] = np.float32(2e-8)
    with ra.TensorList(segs_a, True) as la, ra.TensorList(segs_b, False) as lb:
        for t in range(1, 4):
            grads = []
            for gi, (segs, _, sizes, _) in enumerate(groups):
                for i, s in enumerate(segs):
                    s.grad.copy_(synth.stored_grad(sizes[i], 1e-4, scale, gdt, key + (gi, i, "g", t)).to(DEV))
                    grads.append(s.grad)
            if t == 2:
                segs_b[1].grad[777] = float("nan")
            acc = oracle.StatsAccumulator()
            for g in grads:
                acc.add(grad_host(g), gdt)
            sumsq, count = acc.result
            skip, eff = oracle.decide(sumsq, count, scale, max_norm)
            pres = [_pre(segs) for segs, _, _, _ in groups]
            res, new_steps = ra.radamw_lists_fused_step([la, lb], steps, [opts_a, opts_b], scale, max_norm, True)
            torch.cuda.synchronize()
            if res.updated:  # each group one update from its own state, at the decided clip
                _, eff_dev = oracle.decide(res.sumsq, res.nonfinite, scale, max_norm)
                for (segs, _, sizes, opts), pre, st in zip(groups, pres, steps):
                    _one_step_checks(segs, pre, sizes, gdt, opts, eff_dev, st, f"lists step {t}")
            assert bool(res.found_inf) == skip == (t == 2) and res.nonfinite == count
            assert abs(res.sumsq - sumsq) <= (sum(sizes_a + sizes_b) * 2.0**-53 + 1e-12) * sumsq
            if skip:
                assert new_steps == steps and not res.updated
            else:
                assert new_steps == [steps[0] + 1, steps[1] + 1] and res.updated and res.clip_coef < 1.0
            steps = new_steps
            for segs, refs, sizes, opts in groups:
                for i, s in enumerate(segs):
                    if sizes[i] == 0:
                        continue
                    oracle.adamw_step(refs[i][0], grad_host(s.grad), gdt, refs[i][1], oracle_opts(opts), eff, skip)
                    contract_one_step(host(s.param), refs[i][0], f"step {t} n={sizes[i]} p")
                    contract_one_step(host(s.exp_avg_sq), refs[i][1].exp_avg_sq, f"step {t} n={sizes[i]} v")
        assert steps == [5, 2]


def test_lists_fused_step_of_one_list_is_list_fused_step():
    announce("lists fused step, one list")
    gdt, key = "bf16", (0, "lists1")
    opts = ra.options(lr=1e-3, weight_decay=1e-4)
    segs, _ = _make(SIZES, gdt, False, key)
    twins, _ = _make(SIZES, gdt, False, key)
    with ra.TensorList(segs, False) as la, ra.TensorList(twins, False) as lb:
        sa = sb = 0
        for t in range(1, 4):
            _fill_grads(segs, twins, SIZES, gdt, 1.0, key, t)
            ra_, (sa,) = ra.radamw_lists_fused_step([la], [sa], [opts], 1.0, 0.05, True)
            rb, sb = lb.fused_step(sb, opts, 1.0, 0.05, True)
            torch.cuda.synchronize()
            assert (ra_.sumsq, ra_.nonfinite, ra_.clip_coef, ra_.updated) == (rb.sumsq, rb.nonfinite, rb.clip_coef,
                                                                               rb.updated)
            assert sa == sb == t
            for i, (s, tw) in enumerate(zip(segs, twins)):
                _same_bits(s, tw, False, f"step {t} segment {i}")
        with pytest.raises(ra.RadamwError):  # the same list twice
            ra.radamw_lists_fused_step([la, la], [sa, sa], [opts, opts], 1.0, 1.0, True)
