"""FusedAdamW on the GPU against the oracle: parameter groups, step counts
that differ between tensors, the fused statistics path with global-norm
clipping, the whole-step skip on a non-finite gradient, and resume from a
state_dict.  Page abbreviation: TR-zh = "训练与状态保存"."""
import io

import numpy as np
import pytest
import torch

import oracle
import synth
import optimizer_step_dl_amd as ra
from optimizer_step_dl_amd.optim import FusedAdamW
from gpu_helpers import DEV, announce, contract_one_step, grad_host, host

pytestmark = pytest.mark.gpu

SIZES = [1000, 4097, 65536, 2049]


def _model(key):
    return [torch.nn.Parameter(synth.normal(n, 0.02, key + (i, "p")).to(DEV)) for i, n in enumerate(SIZES)]


def _groups(params):
    return [{"params": params[:2], "lr": 1e-2, "weight_decay": 0.1, "amsgrad": True},
            {"params": params[2:], "lr": 1e-3, "weight_decay": 0.01}]


class OracleMirror:
    """The oracle stepping the same tensors with the same group options."""

    def __init__(self, params, groups):
        self.p = [host(p) for p in params]
        self.st = []
        self.opts = []
        for gi, grp in enumerate(groups):
            for p in grp["params"]:
                o = oracle.Options(lr=grp["lr"], weight_decay=grp["weight_decay"], amsgrad=grp.get("amsgrad", False))
                self.opts.append(o)
                self.st.append(oracle.State(p.numel(), o.amsgrad))

    def step(self, grads, scale=1.0, which=None, skip=False):
        for i, g in enumerate(grads):
            if g is None or (which is not None and i not in which):
                continue
            oracle.adamw_step(self.p[i], grad_host(g), "f32", self.st[i], self.opts[i], scale, skip)


def _set_grads(params, t, key, std=1e-3, scale=1.0, which=None):
    grads = []
    for i, p in enumerate(params):
        if which is not None and i not in which:
            p.grad = None
            grads.append(None)
            continue
        g = synth.stored_grad(p.numel(), std, scale, "f32", key + (i, "g", t)).to(DEV)
        p.grad = g
        grads.append(g)
    return grads


def test_groups_and_lagging_steps_match_oracle():
    announce("FusedAdamW groups")
    params = _model((0, "opt"))
    mirror = OracleMirror(params, _groups(params))
    opt = FusedAdamW(_groups(params))
    for t in range(1, 6):
        which = None if t != 3 else {0, 2}  # tensors 1 and 3 have no gradient on step 3
        grads = _set_grads(params, t, (0, "opt"), which=which)
        opt.step(gradient_scale=1.0)
        mirror.step(grads, which=which)
        torch.cuda.synchronize()
        for i, p in enumerate(params):
            contract_one_step(host(p), mirror.p[i], f"param {i} step {t}")
            assert opt.state[p]["step"] == mirror.st[i].step
    assert opt.state[params[1]]["step"] == 4 and opt.state[params[0]]["step"] == 5
    for i, p in enumerate(params):  # .grad is kept
        assert p.grad is not None


@pytest.mark.parametrize("hierarchical", [False, True])
def test_fused_step_clip_and_skip(hierarchical):
    announce(f"FusedAdamW fused hier={hierarchical}")
    params = _model((0, "optf"))
    mirror = OracleMirror(params, _groups(params))
    opt = FusedAdamW(_groups(params), fused_step=True, max_grad_norm=0.05, hierarchical_stats=hierarchical)
    scale = 256.0
    for t in range(1, 5):
        grads = _set_grads(params, t, (0, "optf"), std=1e-3, scale=scale)
        if t == 3:
            grads[2][123] = float("nan")
        acc = oracle.StatsAccumulator()
        for g in grads:
            acc.add(grad_host(g), "f32")
        sumsq, count = acc.result
        skip, eff = oracle.decide(sumsq, count, scale, 0.05)
        steps_before = [opt.state[p]["step"] if p in opt.state else 0 for p in params]
        opt.step(gradient_scale=scale)
        mirror.step(grads, scale=eff, skip=skip)
        torch.cuda.synchronize()
        res = opt.last_result
        assert bool(res.found_inf) == skip == (t == 3) and res.nonfinite == count
        if not skip:
            assert res.clip_coef < 1.0  # norm ~ sqrt(72k) * 1e-3 ~ 0.27 > 0.05
        for i, p in enumerate(params):
            contract_one_step(host(p), mirror.p[i], f"param {i} step {t}")
            assert opt.state[p]["step"] == mirror.st[i].step == steps_before[i] + (0 if skip else 1)


@pytest.mark.parametrize("gdt", ["bf16", "f16"])
def test_sixteen_bit_gradients_on_fp32_masters(gdt):
    """FP32 master parameters with 16-bit .grad tensors (the parameter's
    grad_dtype set where torch checks it), loss scale 1024, fused step with
    clipping: each step matches the oracle run on the same stored gradients
    with the same clip decision."""
    announce(f"FusedAdamW {gdt} grads")
    params = _model((0, "opt16", gdt))
    ref = [host(p) for p in params]
    states = [oracle.State(p.numel(), False) for p in params]
    oo = oracle.Options(lr=1e-3, weight_decay=0.01)
    opt = FusedAdamW(params, lr=1e-3, weight_decay=0.01, fused_step=True, max_grad_norm=0.05)
    scale = 1024.0
    for t in range(1, 4):
        grads = []
        for i, p in enumerate(params):
            g = synth.stored_grad(p.numel(), 1e-3, scale, gdt, (0, "opt16", gdt, i, "g", t)).to(DEV)
            if hasattr(p, "grad_dtype"):
                p.grad_dtype = g.dtype
            p.grad = g
            grads.append(grad_host(g))
        opt.step(gradient_scale=scale)
        torch.cuda.synchronize()
        res = opt.last_result
        acc = oracle.StatsAccumulator()
        for g in grads:
            acc.add(g, gdt)
        sumsq, count = acc.result
        skip, eff = oracle.decide(res.sumsq, count, scale, 0.05)
        assert res.nonfinite == count == 0 and not skip and res.clip_coef < 1.0
        assert abs(res.sumsq - sumsq) <= (sum(SIZES) - 1) * 2.0**-53 * sumsq  # the oracle's sequential bound
        for i, g in enumerate(grads):
            oracle.adamw_step(ref[i], g, gdt, states[i], oo, eff)
            contract_one_step(host(params[i]), ref[i], f"{gdt} param {i} step {t}")
        assert all(opt.state[p]["step"] == t for p in params)


def test_state_dict_resume_is_bit_exact():
    announce("FusedAdamW resume")
    pa = _model((0, "optr"))
    opt_a = FusedAdamW(_groups(pa), fused_step=True, hierarchical_stats=True)
    for t in range(1, 4):
        _set_grads(pa, t, (0, "optr"))
        opt_a.step()
    buf = io.BytesIO()
    torch.save({"params": [p.detach().clone() for p in pa], "opt": opt_a.state_dict()}, buf)
    for t in range(4, 7):
        _set_grads(pa, t, (0, "optr"))
        opt_a.step()
    buf.seek(0)
    ck = torch.load(buf, weights_only=True)
    pb = [torch.nn.Parameter(x.to(DEV)) for x in ck["params"]]
    opt_b = FusedAdamW(_groups(pb))
    opt_b.load_state_dict(ck["opt"])
    assert opt_b.fused_step and opt_b.hierarchical_stats
    for t in range(4, 7):
        _set_grads(pb, t, (0, "optr"))
        opt_b.step()
    torch.cuda.synchronize()
    for a, b in zip(pa, pb):
        assert torch.equal(a.detach().view(torch.int32), b.detach().view(torch.int32))
        assert torch.equal(opt_a.state[a]["exp_avg_sq"].view(torch.int32), opt_b.state[b]["exp_avg_sq"].view(torch.int32))


def test_close_to_torch_adamw_on_gpu():
    """Cross-check against torch.optim.AdamW (FP32, same options, eps set
    explicitly) over 10 steps: agreement within the contract's tolerances."""
    announce("FusedAdamW vs torch AdamW")
    pa = _model((0, "optt"))
    pb = [torch.nn.Parameter(p.detach().clone()) for p in pa]
    opt_a = FusedAdamW([{"params": pa, "lr": 1e-3, "weight_decay": 0.01, "amsgrad": True}])
    opt_b = torch.optim.AdamW(pb, lr=1e-3, betas=(0.9, 0.999), eps=1e-5, weight_decay=0.01, amsgrad=True,
                              foreach=False)
    for t in range(1, 11):
        grads = _set_grads(pa, t, (0, "optt"))
        for p, g in zip(pb, grads):
            p.grad = g.clone()
        opt_a.step()
        opt_b.step()
        torch.cuda.synchronize()
        for a, b in zip(pa, pb):
            if t == 1:
                contract_one_step(host(a), host(b), f"step {t}")
    for a, b in zip(pa, pb):
        ref = host(b).astype(np.float64)
        assert np.abs(host(a) - ref).max() <= 1e-5 * np.abs(ref).max()


def test_bucket_lists_reused_while_storage_unchanged():
    """Each launch bucket is a persistent tensor list: gradients refreshed
    in place keep the lists; new gradient tensors rebuild them; a group whose
    tensors have no gradient frees its list."""
    announce("FusedAdamW list cache")
    key = (0, "optc")
    params = _model(key)
    opt = FusedAdamW(_groups(params), fused_step=True, max_grad_norm=1.0)
    _set_grads(params, 1, key)
    opt.step()
    first = {k: v[1] for k, v in opt._cache.items()}
    assert len(first) == 2  # one list per parameter group
    for i, p in enumerate(params):
        p.grad.copy_(synth.stored_grad(p.numel(), 1e-3, 1.0, "f32", key + (i, "g", 2)).to(DEV))
    opt.step()
    assert {k: v[1] for k, v in opt._cache.items()} == first
    _set_grads(params, 3, key)
    opt.step()
    third = {k: v[1] for k, v in opt._cache.items()}
    assert len(third) == 2 and all(third[k] is not first[k] for k in third)
    _set_grads(params, 4, key, which={0, 1})  # the second group has no gradient
    opt.step()
    assert len(opt._cache) == 1
    torch.cuda.synchronize()
    assert [opt.state[p]["step"] for p in params] == [4, 4, 3, 3]


# ---------------------------------------------------------- flatten=True --

def _flat_pair(key, **kw):
    """Two copies of the same model: one under FusedAdamW(flatten=True), one
    under the default per-tensor FusedAdamW, with the same options."""
    pa = _model(key)
    pb = [torch.nn.Parameter(p.detach().clone()) for p in pa]
    opt_a = FusedAdamW(_groups(pa), flatten=True, **kw)
    opt_b = FusedAdamW(_groups(pb), **kw)
    return pa, pb, opt_a, opt_b


def _same(a, b):
    return torch.equal(a.detach().view(torch.int32), b.detach().view(torch.int32))


@pytest.mark.parametrize("fused", [False, True])
def test_flatten_equals_per_tensor_steps(fused):
    """flatten=True puts each group's parameters, gradients and moments in
    one bucket allocation (views of it) and steps it as one segment; without
    clipping the results are those of per-tensor steps bit for bit (the
    update is elementwise), and every state tensor is a view of the bucket."""
    announce(f"FusedAdamW flatten fused={fused}")
    key = (0, "optflat", fused)
    pa, pb, opt_a, opt_b = _flat_pair(key, fused_step=fused)
    for b in opt_a._flat:
        arena = b["streams"]
        base = arena[0].data_ptr()
        assert base % (2 << 20) == 0
        for p, off, n in b["members"]:
            assert p.data_ptr() == base + 4 * off and p.grad.data_ptr() == arena[1].data_ptr() + 4 * off
            assert opt_a.state[p]["exp_avg"].data_ptr() == arena[2].data_ptr() + 4 * off
    for t in range(1, 5):
        for i, (a, b) in enumerate(zip(pa, pb)):
            g = synth.stored_grad(a.numel(), 1e-3, 1.0, "f32", key + (i, "g", t)).to(DEV)
            a.grad.copy_(g)
            b.grad = g.clone()
        launches = ra.radamw_launch_count()
        opt_a.step()
        if not fused:
            assert ra.radamw_launch_count() - launches == 2  # one update launch per group
        opt_b.step()
        torch.cuda.synchronize()
        for a, b in zip(pa, pb):
            assert _same(a, b)
            for name in ("exp_avg", "exp_avg_sq"):
                assert _same(opt_a.state[a][name], opt_b.state[b][name])
            assert opt_a.state[a]["step"] == opt_b.state[b]["step"] == t


def test_flatten_clip_matches_oracle_and_skips():
    """Fused step with clipping over flattened groups: each step matches the
    oracle at the clip the step reported; a NaN skips the whole step."""
    announce("FusedAdamW flatten clip")
    params = _model((0, "optflc"))
    mirror = OracleMirror(params, _groups(params))
    opt = FusedAdamW(_groups(params), fused_step=True, max_grad_norm=0.05, hierarchical_stats=True, flatten=True)
    for t in range(1, 5):
        grads = []
        for i, p in enumerate(params):
            g = synth.stored_grad(p.numel(), 1e-3, 256.0, "f32", (0, "optflc", i, "g", t)).to(DEV)
            if t == 3 and i == 2:
                g[123] = float("nan")
            p.grad.copy_(g)
            grads.append(g)
        opt.step(gradient_scale=256.0)
        torch.cuda.synchronize()
        res = opt.last_result
        skip, eff = oracle.decide(res.sumsq, res.nonfinite, 256.0, 0.05)
        assert bool(res.found_inf) == skip == (t == 3)
        mirror.step(grads, scale=eff, skip=skip)
        for i, p in enumerate(params):
            contract_one_step(host(p), mirror.p[i], f"flat param {i} step {t}")
            assert opt.state[p]["step"] == mirror.st[i].step


def test_flatten_backward_accumulates_into_the_bucket():
    """A small model trained with loss.backward(): the gradients land in the
    bucket (autograd accumulates into the existing .grad in place),
    zero_grad() zeroes them there, and the weights follow the per-tensor
    optimizer bit for bit."""
    announce("FusedAdamW flatten with autograd")
    torch.manual_seed(0)
    ma = torch.nn.Sequential(torch.nn.Linear(64, 128), torch.nn.ReLU(), torch.nn.Linear(128, 10)).to(DEV)
    mb = torch.nn.Sequential(torch.nn.Linear(64, 128), torch.nn.ReLU(), torch.nn.Linear(128, 10)).to(DEV)
    mb.load_state_dict(ma.state_dict())
    opt_a = FusedAdamW(ma.parameters(), lr=1e-2, weight_decay=0.01, flatten=True)
    opt_b = FusedAdamW(mb.parameters(), lr=1e-2, weight_decay=0.01)
    g_arena = opt_a._flat[0]["streams"][1]
    for t in range(5):
        x = synth.normal(32 * 64, 1.0, (0, "optfla", t, "x")).view(32, 64).to(DEV)
        y = torch.arange(32, device=DEV) % 10
        for m, o in ((ma, opt_a), (mb, opt_b)):
            o.zero_grad()
            torch.nn.functional.cross_entropy(m(x), y).backward()
            o.step()
        for p in ma.parameters():
            lo = g_arena.data_ptr()
            assert lo <= p.grad.data_ptr() < lo + g_arena.numel() * 4
        torch.cuda.synchronize()
        for a, b in zip(ma.parameters(), mb.parameters()):
            assert _same(a, b), t
    opt_a.zero_grad()
    assert int(torch.count_nonzero(g_arena)) == 0
    assert all(p.grad is not None for p in ma.parameters())


def test_flatten_state_dict_is_compact_and_resumes_bit_exact():
    """state_dict() of a flattened optimizer stores compact copies of each
    parameter's state (not the bucket behind the views); loading it puts
    the state back into the bucket, and the resumed run equals the
    uninterrupted one bit for bit."""
    announce("FusedAdamW flatten resume")
    key = (0, "optflr")
    pa = _model(key)
    opt_a = FusedAdamW(_groups(pa), fused_step=True, flatten=True)
    for t in range(1, 4):
        for i, p in enumerate(pa):
            p.grad.copy_(synth.stored_grad(p.numel(), 1e-3, 1.0, "f32", key + (i, "g", t)).to(DEV))
        opt_a.step()
    buf = io.BytesIO()
    torch.save({"params": [p.detach().clone() for p in pa], "opt": opt_a.state_dict()}, buf)
    assert buf.tell() < 3 * 4 * sum(SIZES) + (1 << 20)  # p, m, v once each (+ v_max of one group), no bucket
    for t in range(4, 7):
        for i, p in enumerate(pa):
            p.grad.copy_(synth.stored_grad(p.numel(), 1e-3, 1.0, "f32", key + (i, "g", t)).to(DEV))
        opt_a.step()
    buf.seek(0)
    ck = torch.load(buf, weights_only=True)
    pb = [torch.nn.Parameter(x.to(DEV)) for x in ck["params"]]
    opt_b = FusedAdamW(_groups(pb), flatten=True)
    opt_b.load_state_dict(ck["opt"])
    arena = opt_b._flat[0]["streams"]
    assert opt_b.state[pb[0]]["exp_avg"].data_ptr() == arena[2].data_ptr()
    for t in range(4, 7):
        for i, p in enumerate(pb):
            p.grad.copy_(synth.stored_grad(p.numel(), 1e-3, 1.0, "f32", key + (i, "g", t)).to(DEV))
        opt_b.step()
    torch.cuda.synchronize()
    for a, b in zip(pa, pb):
        assert _same(a, b) and _same(opt_a.state[a]["exp_avg_sq"], opt_b.state[b]["exp_avg_sq"])


def test_flatten_follows_group_options_after_load():
    """load_state_dict replaces the parameter-group dicts.  A flattened group
    then steps with the options of the current dicts, the ones an LR
    scheduler edits: bit for bit the per-tensor optimizer under the same
    edits (with the options held before the load, lr and weight decay would
    differ)."""
    announce("FusedAdamW flatten options after load")
    key = (0, "optflo")
    pa, pb, opt_a, opt_b = _flat_pair(key)

    def set_grads(t):
        for i, (a, b) in enumerate(zip(pa, pb)):
            g = synth.stored_grad(a.numel(), 1e-3, 1.0, "f32", key + (i, "g", t)).to(DEV)
            a.grad.copy_(g)
            b.grad = g.clone()

    for t in (1, 2):
        set_grads(t)
        opt_a.step()
        opt_b.step()
    for o in (opt_a, opt_b):
        o.load_state_dict(o.state_dict())
        o.param_groups[0]["lr"] = 3e-3
        o.param_groups[1]["weight_decay"] = 0.0
    for t in (3, 4):
        set_grads(t)
        opt_a.step()
        opt_b.step()
    torch.cuda.synchronize()
    for a, b in zip(pa, pb):
        assert _same(a, b)
        for name in ("exp_avg", "exp_avg_sq"):
            assert _same(opt_a.state[a][name], opt_b.state[b][name])
        assert opt_a.state[a]["step"] == opt_b.state[b]["step"] == 4


def test_flatten_sixteen_bit_gradients_and_replaced_grad():
    """A BF16 gradient bucket under FP32 masters; a .grad replaced by a new
    tensor is copied back into the bucket before the step; the result
    matches the oracle."""
    announce("FusedAdamW flatten bf16 grads")
    params = _model((0, "optflb"))
    ref = [host(p) for p in params]
    states = [oracle.State(p.numel(), False) for p in params]
    oo = oracle.Options(lr=1e-3, weight_decay=0.01)
    opt = FusedAdamW(params, lr=1e-3, weight_decay=0.01, flatten=True, flatten_grad_dtype=torch.bfloat16)
    assert opt._flat[0]["streams"][1].dtype == torch.bfloat16
    for t in range(1, 4):
        grads = []
        for i, p in enumerate(params):
            g = synth.stored_grad(p.numel(), 1e-3, 1.0, "bf16", (0, "optflb", i, "g", t)).to(DEV)
            if i == 1 and t == 2:
                p.grad = g.clone()  # a new tensor: copied back into the bucket
            else:
                p.grad.copy_(g)
            grads.append(grad_host(g))
        opt.step()
        torch.cuda.synchronize()
        for i, g in enumerate(grads):
            oracle.adamw_step(ref[i], g, "bf16", states[i], oo, 1.0)
            contract_one_step(host(params[i]), ref[i], f"flat bf16 param {i} step {t}")
    g_arena = opt._flat[0]["streams"][1]
    assert params[1].grad.data_ptr() == g_arena.data_ptr() + 2 * SIZES[0]
