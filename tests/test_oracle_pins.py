"""Pins of the CPU oracle against facts fixed outside it.

Each test checks the oracle (oracle/radamw_oracle.c through oracle/__init__.py)
against closed forms, invariants, an independent float64 restatement, torch's
CPU AdamW, exact arithmetic, or numbers printed on the pages -- never against
a retyping of its own formula.  Page abbreviations: FA-ja = "実験的なデバイス上の
融合 AdamW / AMSGrad", FA-zh = "实验性融合 AdamW / AMSGrad", TR-zh = "训练与状态保存".
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import brute64
from conftest import load_golden

GDTS = ["f32", "f16", "bf16"]
MATRIX = list(itertools.product(GDTS, [False, True], [False, True]))


def _grad(n, std, mult, gdt, key):
    return synth.grad_numpy(synth.stored_grad(n, std, mult, gdt, key))


def _params(n, key):
    return synth.normal(n, 0.02, key).numpy().copy()


def _run(p, grads, gdt, opts, scale=1.0, state=None):
    p = p.copy()
    st = state.copy() if state is not None else oracle.State(p.size, opts.amsgrad)
    for g in grads:
        oracle.adamw_step(p, g, gdt, st, opts, scale)
    return p, st


def ulp32(x):
    x = np.abs(np.asarray(x, np.float32))
    return np.spacing(x).astype(np.float64)


# ------------------------------------------------------------ closed forms --

@pytest.mark.parametrize("gdt", GDTS)
@pytest.mark.parametrize("amsgrad", [False, True])
def test_zero_gradient_is_pure_decay(gdt, amsgrad):
    """g = 0 from zero state: every step multiplies p by the FP32 decay factor
    1 - lr*wd exactly, and all moments stay exactly zero (FA-ja, formula)."""
    n = 257
    opts = oracle.Options(lr=1e-2, weight_decay=0.1, amsgrad=amsgrad)
    p0 = _params(n, (0, "zero", "p"))
    zero = np.zeros(n, np.float32) if gdt == "f32" else np.zeros(n, np.uint16)
    decay = np.float32(1.0 - opts.lr * opts.weight_decay)
    p, st = p0.copy(), oracle.State(n, amsgrad)
    expect = p0.copy()
    for t in range(1, 11):
        assert oracle.adamw_step(p, zero, gdt, st, opts)
        expect = (expect * decay).astype(np.float32)
        assert st.step == t
        assert np.array_equal(p.view(np.uint32), expect.view(np.uint32))
        assert not np.any(st.exp_avg) and not np.any(st.exp_avg_sq)
        if amsgrad:
            assert not np.any(st.max_exp_avg_sq)


@pytest.mark.parametrize("gdt", GDTS)
def test_first_step_closed_form(gdt):
    """From zero state the bias-corrected moments are g and g^2, so the first
    update is lr*g/(|g|+eps) on top of the decay (FA-ja formula with t = 1)."""
    n = 4096
    opts = oracle.Options(lr=1e-2, weight_decay=0.1, eps=1e-3)
    p0 = _params(n, (0, "first", "p"))
    g = _grad(n, 1e-3, 1.0, gdt, (0, "first", "g"))
    p, st = _run(p0, [g], gdt, opts)
    x = oracle.widen(g, gdt).astype(np.float64)
    closed = p0.astype(np.float64) * (1 - opts.lr * opts.weight_decay) - opts.lr * x / (np.abs(x) + opts.eps)
    upd = opts.lr * np.abs(x) / (np.abs(x) + opts.eps)
    # roundings: the decay factor's cast and p*decay (ulp of p0), the final
    # subtraction (ulp of the result), a few ulps of the update itself
    err = np.abs(p - closed)
    assert np.all(err <= ulp32(p0) + ulp32(closed) + 8 * 2**-24 * upd), err.max()
    assert np.allclose(st.exp_avg, (1 - opts.beta1) * x, rtol=4 * 2**-24, atol=0)
    assert np.allclose(st.exp_avg_sq, (1 - opts.beta2) * x * x, rtol=6 * 2**-24, atol=0)


def test_zero_betas_every_step_is_sign_like():
    """beta1 = beta2 = 0: m = g, v = g^2, no bias correction left, so every
    step is decay plus lr*g/(|g|+eps) (FA-ja formula, degenerate betas)."""
    n = 1024
    opts = oracle.Options(lr=1e-2, beta1=0.0, beta2=0.0, eps=1e-3, weight_decay=0.05)
    p = _params(n, (0, "b0", "p"))
    st = oracle.State(n, False)
    for t in range(6):
        g = _grad(n, 1e-3, 1.0, "f32", (0, "b0", "g", t))
        before = p.astype(np.float64).copy()
        oracle.adamw_step(p, g, "f32", st, opts)
        x = g.astype(np.float64)
        closed = before * (1 - opts.lr * opts.weight_decay) - opts.lr * x / (np.abs(x) + opts.eps)
        upd = opts.lr * np.abs(x) / (np.abs(x) + opts.eps)
        assert np.all(np.abs(p - closed) <= ulp32(before) + ulp32(closed) + 8 * 2**-24 * upd)


def test_zero_lr_leaves_params_bit_unchanged_but_moves_moments():
    n = 777
    opts = oracle.Options(lr=0.0, weight_decay=0.3, amsgrad=True)
    p0 = _params(n, (0, "lr0", "p"))
    grads = [_grad(n, 1e-3, 1.0, "bf16", (0, "lr0", "g", t)) for t in range(4)]
    p, st = _run(p0, grads, "bf16", opts)
    assert np.array_equal(p.view(np.uint32), p0.view(np.uint32))
    assert np.any(st.exp_avg) and np.any(st.exp_avg_sq) and np.any(st.max_exp_avg_sq)


# -------------------------------------------------------------- invariants --

@pytest.mark.parametrize("gdt,amsgrad", list(itertools.product(GDTS, [False, True])))
def test_maximize_mirrors_sign_bit_exact(gdt, amsgrad):
    """maximize on G gives exactly the run on -G (FA-ja: g is negated when
    maximizing); the first step mirrors the sign of the update."""
    n = 515
    p0 = _params(n, (0, "max", "p"))
    grads = [_grad(n, 1e-3, 64.0, gdt, (0, "max", "g", t)) for t in range(5)]
    neg = [(-g) if gdt == "f32" else (g ^ np.uint16(0x8000)) for g in grads]
    a_opts = oracle.Options(amsgrad=amsgrad, maximize=True)
    b_opts = oracle.Options(amsgrad=amsgrad, maximize=False)
    pa, sa = _run(p0, grads, gdt, a_opts, scale=64.0)
    pb, sb = _run(p0, neg, gdt, b_opts, scale=64.0)
    for x, y in [(pa, pb), (sa.exp_avg, sb.exp_avg), (sa.exp_avg_sq, sb.exp_avg_sq)]:
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    # first step: the update moves p against the descent direction
    p1, _ = _run(p0, grads[:1], gdt, oracle.Options(weight_decay=0.0, maximize=True), 64.0)
    x = oracle.widen(grads[0], gdt)
    moved = np.sign(p1.astype(np.float64) - p0)
    nz = (x != 0) & (moved != 0)
    assert np.all(moved[nz] == np.sign(x[nz]))


@pytest.mark.parametrize("gdt", GDTS)
def test_power_of_two_unscale_is_exact(gdt):
    """Dividing by a power-of-two scale is exact, so run(scale=2^k, G*2^k)
    equals run(scale=1, G) bit for bit (FA-ja: g = stored / gradient_scale)."""
    n = 300
    p0 = _params(n, (0, "unscale", "p"))
    base = [synth.stored_grad(n, 1e-3, 1.0, gdt, (0, "unscale", "g", t)) for t in range(4)]
    scaled = [synth.grad_numpy(b * 1024) for b in base]  # exact: power of two, no overflow
    plain = [synth.grad_numpy(b) for b in base]
    for amsgrad in (False, True):
        opts = oracle.Options(amsgrad=amsgrad)
        pa, sa = _run(p0, scaled, gdt, opts, scale=1024.0)
        pb, sb = _run(p0, plain, gdt, opts, scale=1.0)
        assert np.array_equal(pa.view(np.uint32), pb.view(np.uint32))
        assert np.array_equal(sa.exp_avg_sq.view(np.uint32), sb.exp_avg_sq.view(np.uint32))


@pytest.mark.parametrize("amsgrad", [False, True])
def test_skip_and_empty_touch_nothing(amsgrad):
    """skip_update or an empty tensor: nothing written, no step increment
    (FA-zh "增加的实际能力")."""
    n = 100
    opts = oracle.Options(amsgrad=amsgrad)
    p0 = _params(n, (0, "skip", "p"))
    g = _grad(n, 1e-3, 1.0, "f32", (0, "skip", "g"))
    p, st = _run(p0, [g, g], "f32", opts)
    snap = (p.copy(), st.copy())
    assert not oracle.adamw_step(p, g, "f32", st, opts, skip_update=True)
    assert st.step == 2
    assert np.array_equal(p, snap[0]) and np.array_equal(st.exp_avg, snap[1].exp_avg)
    assert np.array_equal(st.exp_avg_sq, snap[1].exp_avg_sq)
    empty_state = oracle.State(0, amsgrad)
    empty_state.step = 7
    assert not oracle.adamw_step(np.zeros(0, np.float32), np.zeros(0, np.float32), "f32",
                                 empty_state, opts)
    assert empty_state.step == 7


@pytest.mark.parametrize("gdt", GDTS)
def test_amsgrad_running_max_properties(gdt):
    """v_max never decreases, is never below the current v, and always equals
    one of (old v_max, new v) bitwise; kept uncorrected (FA-ja formula)."""
    n = 2048
    opts = oracle.Options(amsgrad=True, beta2=0.9)
    p = _params(n, (0, "ams", "p"))
    st = oracle.State(n, True)
    for t in range(8):
        # alternate large and small gradients so v falls below v_max
        g = _grad(n, 1e-3 if t % 2 == 0 else 1e-5, 1.0, gdt, (0, "ams", "g", t))
        old = st.max_exp_avg_sq.copy()
        oracle.adamw_step(p, g, gdt, st, opts)
        new, v = st.max_exp_avg_sq, st.exp_avg_sq
        assert np.all(new >= old) and np.all(new >= v)
        assert np.all((new.view(np.uint32) == old.view(np.uint32)) | (new.view(np.uint32) == v.view(np.uint32)))
        if t > 0:
            assert np.any(new > v)  # the max is actually used


@pytest.mark.parametrize("gdt", GDTS)
def test_amsgrad_first_step_equals_adamw_first_step(gdt):
    n = 999
    p0 = _params(n, (0, "ams1", "p"))
    g = _grad(n, 1e-3, 1.0, gdt, (0, "ams1", "g"))
    pa, sa = _run(p0, [g], gdt, oracle.Options(amsgrad=True))
    pb, sb = _run(p0, [g], gdt, oracle.Options(amsgrad=False))
    assert np.array_equal(pa.view(np.uint32), pb.view(np.uint32))
    assert np.array_equal(sa.exp_avg.view(np.uint32), sb.exp_avg.view(np.uint32))
    assert np.array_equal(sa.max_exp_avg_sq.view(np.uint32), sa.exp_avg_sq.view(np.uint32))


def test_resume_from_parts_equals_uninterrupted_run():
    """k steps, hand the step count and moments over to a fresh state, k more
    steps == 2k uninterrupted steps (FA-ja "低レベルの使用", into/from parts)."""
    n, k = 333, 4
    opts = oracle.Options(amsgrad=True, weight_decay=0.01)
    p0 = _params(n, (0, "resume", "p"))
    grads = [_grad(n, 1e-3, 128.0, "bf16", (0, "resume", "g", t)) for t in range(2 * k)]
    p_full, s_full = _run(p0, grads, "bf16", opts, scale=128.0)
    p_half, s_half = _run(p0, grads[:k], "bf16", opts, scale=128.0)
    parts = (s_half.step, s_half.exp_avg.tobytes(), s_half.exp_avg_sq.tobytes(), s_half.max_exp_avg_sq.tobytes())
    restored = oracle.State(n, True)
    restored.step = parts[0]
    restored.exp_avg = np.frombuffer(parts[1], np.float32).copy()
    restored.exp_avg_sq = np.frombuffer(parts[2], np.float32).copy()
    restored.max_exp_avg_sq = np.frombuffer(parts[3], np.float32).copy()
    p_res, s_res = _run(np.frombuffer(p_half.tobytes(), np.float32).copy(), grads[k:], "bf16", opts,
                        scale=128.0, state=restored)
    assert s_res.step == s_full.step == 2 * k
    for a, b in [(p_res, p_full), (s_res.exp_avg, s_full.exp_avg), (s_res.exp_avg_sq, s_full.exp_avg_sq),
                 (s_res.max_exp_avg_sq, s_full.max_exp_avg_sq)]:
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ------------------------------------------- independent float64 restatement --

# Options chosen so every term of the formula is far above one FP32 ulp of p:
# large lr*wd, eps comparable to |g|, betas whose bias corrections stay large.
PIN_OPTS = dict(lr=1e-2, beta1=0.8, beta2=0.95, eps=1e-3, weight_decay=0.1)


@pytest.mark.parametrize("gdt,amsgrad,maximize", MATRIX)
def test_oracle_matches_float64_brute_force(gdt, amsgrad, maximize):
    n, steps, scale = 64, 5, 128.0
    opts = oracle.Options(amsgrad=amsgrad, maximize=maximize, **PIN_OPTS)
    p = _params(n, (0, "b64", "p"))
    st = oracle.State(n, amsgrad)
    p64, m64, v64 = p.astype(np.float64), np.zeros(n), np.zeros(n)
    vmax64 = np.zeros(n) if amsgrad else None
    upd_sum = np.zeros(n)
    m_scale = np.zeros(n)  # running magnitude of the terms summed into m (cancellation-free)
    for t in range(1, steps + 1):
        # mix magnitudes so eps matters for some elements and not others
        g = _grad(n, 1e-3 if t % 2 else 5e-2, scale, gdt, (0, "b64", "g", t))
        x = oracle.widen(g, gdt).astype(np.float64)
        oracle.adamw_step(p, g, gdt, st, opts, scale)
        prev = p64
        p64, m64, v64, vmax64 = brute64.step64(p64, x, m64, v64, vmax64, t, opts.lr, opts.beta1,
                                               opts.beta2, opts.eps, opts.weight_decay, amsgrad,
                                               maximize, scale)
        upd_sum += np.abs(prev * (1 - opts.lr * opts.weight_decay) - p64)
        m_scale = opts.beta1 * m_scale + (1 - opts.beta1) * np.abs(x / scale)
        assert np.all(np.abs(p - p64) <= t * ulp32(p64) + 1e-6 * upd_sum), t
        assert np.all(np.abs(st.exp_avg - m64) <= 4 * t * 2**-24 * m_scale + 1e-30), t
        assert np.all(np.abs(st.exp_avg_sq - v64) <= 8 * t * ulp32(v64) + 1e-30), t
        if amsgrad:
            assert np.all(np.abs(st.max_exp_avg_sq - vmax64) <= 8 * t * ulp32(vmax64) + 1e-30), t


def test_brute_force_pin_is_sensitive_to_each_term():
    """The float64 comparison above would catch a dropped or mis-signed term:
    perturbing any single ingredient of the f64 model moves p by far more than
    the bound used there."""
    n, t = 64, 1
    p = _params(n, (0, "sens", "p")).astype(np.float64)
    x = oracle.widen(_grad(n, 1e-3, 1.0, "f32", (0, "sens", "g")), "f32").astype(np.float64)
    base = brute64.step64(p, x, np.zeros(n), np.zeros(n), None, t, **PIN_OPTS, amsgrad=False,
                          maximize=False, gradient_scale=1.0)[0]
    bound = ulp32(base) + 1e-6 * np.abs(p * (1 - 1e-3) - base)
    variants = {
        "no weight decay": dict(PIN_OPTS, weight_decay=0.0),
        "eps inside sqrt": None,
        "no bias correction": None,
        "wrong sign": None,
    }
    alt = brute64.step64(p, x, np.zeros(n), np.zeros(n), None, t, **variants["no weight decay"],
                         amsgrad=False, maximize=False, gradient_scale=1.0)[0]
    assert np.all(np.abs(alt - base) > bound)
    lr, b1, b2, eps, wd = (PIN_OPTS[k] for k in ("lr", "beta1", "beta2", "eps", "weight_decay"))
    m, v = (1 - b1) * x, (1 - b2) * x * x
    inside = p * (1 - lr * wd) - lr * (m / (1 - b1)) / np.sqrt(v / (1 - b2) + eps)
    nobc = p * (1 - lr * wd) - lr * m / (np.sqrt(v) + eps)
    sign = p * (1 - lr * wd) + lr * (m / (1 - b1)) / (np.sqrt(v / (1 - b2)) + eps)
    for alt in (inside, nobc, sign):
        assert np.all(np.abs(alt - base) > bound)


# --------------------------------------------------- library routine (torch) --

@pytest.mark.parametrize("gdt,amsgrad,maximize", MATRIX)
def test_oracle_matches_torch_cpu_adamw(gdt, amsgrad, maximize):
    """The 12-case matrix x 5 steps of FA-ja "検証およびベンチマーク コマンド",
    regenerated with torch.optim.AdamW on the CPU (the pages' formula
    reference), eps set explicitly, grads pre-divided by the scale."""
    n, steps, scale = 64, 5, 128.0
    opts = oracle.Options(lr=1e-3, weight_decay=0.01, amsgrad=amsgrad, maximize=maximize)
    p0 = _params(n, (0, "torch", "p"))
    p, st = p0.copy(), oracle.State(n, amsgrad)
    tp = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    topt = torch.optim.AdamW([tp], lr=opts.lr, betas=(opts.beta1, opts.beta2), eps=opts.eps,
                             weight_decay=opts.weight_decay, amsgrad=amsgrad, maximize=maximize,
                             foreach=False)
    m_scale = np.zeros(n)  # magnitude of the terms summed into m
    for t in range(steps):
        g = _grad(n, 1e-3, scale, gdt, (0, "torch", "g", t))
        oracle.adamw_step(p, g, gdt, st, opts, scale)
        tp.grad = torch.from_numpy(oracle.widen(g, gdt)) / scale
        m_scale = opts.beta1 * m_scale + (1 - opts.beta1) * np.abs(tp.grad.numpy().astype(np.float64))
        topt.step()
        ref = tp.detach().numpy()
        tstate = topt.state[tp]
        assert np.all(np.abs(p - ref) <= 1e-6 * (1 + np.abs(ref)))
        # the moments are compared relatively (an absolute bound is vacuous at
        # 1e-6 scale); m relative to its terms, since torch forms it with lerp
        assert np.all(np.abs(st.exp_avg - tstate["exp_avg"].numpy()) <= 8 * (t + 1) * 2**-24 * m_scale)
        assert np.allclose(st.exp_avg_sq, tstate["exp_avg_sq"].numpy(), rtol=1e-5, atol=0)
        if amsgrad:
            assert np.allclose(st.max_exp_avg_sq, tstate["max_exp_avg_sq"].numpy(), rtol=1e-5, atol=0)
        assert st.step == t + 1


# ----------------------------------------------------------- coefficients --

@pytest.mark.parametrize("betas", [(0.9, 0.999), (0.8, 0.95)])
def test_bias_corrections_match_exact_arithmetic(betas):
    """FP32 cast of 1 - beta^t formed in FP64 == correctly rounded exact value
    (FA-ja: FP64 integer power, FP32 cast)."""
    opts = oracle.Options(beta1=betas[0], beta2=betas[1])
    ts = list(range(1, 400)) + [1000, 4096, 10_000]
    for t in ts:
        c = oracle.coefficients(opts, t)
        for beta, key in ((betas[0], "bc1"), (betas[1], "bc2")):
            exact = 1 - Fraction(beta) ** t
            want = np.float32(float(exact))  # double rounding only matters at exact ties
            assert c[key] == want, (t, key, c[key], want)
    c = oracle.coefficients(oracle.Options(lr=1e-3, weight_decay=1e-4), 1)
    assert c["decay"] == np.float32(1 - Fraction(1e-3) * Fraction(1e-4))


def _decimal_bias(beta: float, t: int) -> np.float32:
    """FP32 rounding of 1 - beta^t with beta^t evaluated in 80-digit decimal
    arithmetic from the exact binary value of beta."""
    import decimal
    with decimal.localcontext() as ctx:
        ctx.prec = 80
        val = 1 - decimal.Decimal(beta) ** t
        return np.float32(float(val))


@pytest.mark.parametrize("betas", [(0.9, 0.999), (0.8, 0.95), (0.95, 0.9999)])
def test_bias_corrections_up_to_a_million_steps(betas):
    """Late steps (t in [1e4, 1e6], log-spaced, plus the region where
    1 - beta2^t reaches 1 in FP32): the oracle's FP64 power stays within the
    correctly rounded FP32 value of the exact quantity."""
    opts = oracle.Options(beta1=betas[0], beta2=betas[1])
    ts = sorted(set(int(round(x)) for x in np.logspace(4, 6, 25)) | {16_000, 17_000, 18_000, 170_000, 180_000})
    for t in ts:
        c = oracle.coefficients(opts, t)
        for beta, key in ((betas[0], "bc1"), (betas[1], "bc2")):
            want = _decimal_bias(beta, t)
            assert c[key] == want, (t, key, c[key], want)
    # beyond the point where beta2^t < 2^-25 the FP32 bias correction is exactly 1
    assert oracle.coefficients(oracle.Options(), 1_000_000)["bc2"] == np.float32(1.0)


# --------------------------------------------------------------- decoding --

def test_half_decoder_matches_numpy_for_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.widen(bits, "f16")
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_decoder_matches_torch_for_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.widen(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


# ------------------------------------------------------------------ stats --

def _widen_lib(g, gdt):
    """Library widening (numpy / torch conversion), independent of the oracle's decoder."""
    if gdt == "f32":
        return g.astype(np.float64)
    if gdt == "f16":
        return g.view(np.float16).astype(np.float64)
    return torch.from_numpy(g.view(np.int16)).view(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("gdt", GDTS)
def test_stats_count_and_sum_against_fsum(gdt):
    n = 5000
    g = _grad(n, 1.0, 1.0, gdt, (0, "stats", "g"))
    pos = synth.nonfinite_positions(n, 37, (0, "stats", "pos"))
    vals = synth.nonfinite_values(37)
    if gdt == "f32":
        g[pos] = vals
    else:
        t = torch.from_numpy(g.view(np.int16)).view(synth.GRAD_TORCH_DTYPES[gdt]).clone()
        t[torch.from_numpy(pos)] = torch.tensor(vals, dtype=t.dtype)
        g = t.view(torch.int16).numpy().view(np.uint16)
    sumsq, count = oracle.grad_stats(g, gdt)
    x = _widen_lib(g, gdt)
    fin = np.isfinite(x)
    assert count == int((~fin).sum()) == 37
    exact = math.fsum((x[fin] ** 2).tolist())  # squares exact in f64 for these inputs
    assert abs(sumsq - exact) <= 1e-12 * exact


def test_stats_dyadic_sum_is_exact_and_concatenation_holds():
    n = 1 << 16
    g = np.full(n, 2.0**-8, np.float32)
    assert oracle.grad_stats(g, "f32") == (n * 2.0**-16, 0)
    a, b = _grad(1000, 1e-2, 1.0, "bf16", (0, "cat", 0)), _grad(777, 1e-2, 1.0, "bf16", (0, "cat", 1))
    acc = oracle.StatsAccumulator().add(a, "bf16").add(b, "bf16")
    assert acc.result == oracle.grad_stats(np.concatenate([a, b]), "bf16")


def test_stats_count_saturates():
    acc = oracle.StatsAccumulator()
    acc.nonfinite.value = 2**32 - 3
    acc.add(np.array([np.inf, np.nan, -np.inf, np.nan, 1.0], np.float32), "f32")
    assert acc.result == (1.0, 2**32 - 1)


def test_stats_plan_matches_page_figures():
    gold = load_golden("stats_plan.json")
    fan = gold["fan_in"]
    assert oracle.stats_plan(gold["rows_min"] - 1) is None
    assert oracle.stats_plan(gold["rows_max"] + 1) is None
    assert oracle.stats_plan(gold["no_extra_merge_up_to_rows"]) == (0, 0)
    se, extra = oracle.stats_plan(gold["rows_max"])
    assert extra == gold["max_extra_merge_kernels"]
    assert se * 4 == gold["max_scratch_bytes"]
    assert oracle.stats_plan(1025) == (6, 1)
    assert oracle.stats_plan(fan * fan) == (3 * fan, 1)
    assert oracle.stats_plan(fan * fan + 1)[1] == 2


@pytest.mark.parametrize("rows", [1, 2, 1023, 1024, 1025, 5000, 1048576, 1048577, 3_000_001, 4194304])
def test_stats_plan_against_brute_force_grouping(rows):
    """Count the records a fan-in-1024 tree actually produces by grouping
    list lengths until at most 1024 remain; the final merge reduces those to
    the report.  Worst-case scratch over all rows stays within 49,200 B."""
    levels, c = [], rows
    while c > 1024:
        c = len(range(0, c, 1024))
        levels.append(c)
    assert oracle.stats_plan(rows) == (3 * sum(levels), len(levels))
    assert 12 * sum(levels) <= load_golden("stats_plan.json")["max_scratch_bytes"]


# ------------------------------------------------------------------- clip --

def test_clip_decision_matches_torch_clip_grad_norm():
    n, scale, max_norm = 4096, 128.0, 1.0
    g = _grad(n, 1e-1, scale, "f32", (0, "clip", "g"))  # norm ~ 6.4
    sumsq, count = oracle.grad_stats(g, "f32")
    skip, eff = oracle.decide(sumsq, count, scale, max_norm)
    assert not skip
    t = torch.nn.Parameter(torch.zeros(n))
    t.grad = torch.from_numpy(g.astype(np.float64) / scale).float()
    norm = torch.nn.utils.clip_grad_norm_([t], max_norm).item()
    assert norm > max_norm  # clipping active in this case
    ours = g.astype(np.float64) / eff
    assert np.allclose(ours, t.grad.numpy(), rtol=1e-6, atol=0)
    # below the threshold the scale passes through unchanged (bit identity)
    skip, eff2 = oracle.decide(sumsq, count, scale, max_norm=1e6)
    assert eff2 == scale and not skip
    assert oracle.decide(sumsq, 3, scale, max_norm) == (True, scale)
    assert oracle.decide(sumsq, 0, scale, None) == (False, scale)


# ------------------------------------------------ low-precision write-back --

def _rounding_probe_values():
    rng = np.random.Generator(np.random.PCG64(7))
    parts = [
        rng.standard_normal(200_000).astype(np.float32) * np.float32(0.02),
        (rng.standard_normal(100_000) * 1e4).astype(np.float32),
        (np.exp(rng.uniform(-120, 88, 100_000)) * rng.choice([-1, 1], 100_000)).astype(np.float32),
        rng.integers(0, 2**32, 200_000, dtype=np.uint64).astype(np.uint32).view(np.float32),  # every bit pattern class
        np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 65504.0, 65519.99, 65520.0, 2.0**-24, 2.0**-25,
                  2.0**-25 * 1.0000001, 3 * 2.0**-26, 2.0**-14, 2.0**-14 * (1 - 2.0**-11), 1.0 + 2.0**-11,
                  1.0 + 3 * 2.0**-11, 3.4028235e38, 1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8], np.float32),
    ]
    # exact ties for both formats
    base = rng.standard_normal(50_000).astype(np.float32).view(np.uint32)
    parts.append(((base & ~np.uint32(0xFFFF)) | np.uint32(0x8000)).view(np.float32))
    parts.append(((base & ~np.uint32(0x1FFF)) | np.uint32(0x1000)).view(np.float32))
    return np.concatenate(parts)


def test_f16_rounding_matches_numpy():
    x = _rounding_probe_values()
    ours = oracle.round_copy(x, "f16")
    with np.errstate(over="ignore"):  # overflow to infinity is the expected rounding
        ref = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all(np.isnan(ours[nan].view(np.float16)))


def test_bf16_rounding_matches_torch():
    x = _rounding_probe_values()
    ours = oracle.round_copy(x, "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all(np.isnan(torch.from_numpy(ours[nan].view(np.int16)).view(torch.bfloat16).float().numpy()))
