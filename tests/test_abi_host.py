"""Host-side checks of libradamw.so that need no GPU: the library loads, it
exports every symbol include/radamw.h declares, and its host-only logic (merge
plan, row geometry, FP32 coefficients, clip decision, argument validation that
returns before any HIP call) agrees with the oracle and the pages' figures."""
import ctypes
import os
import re
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from conftest import ROOT, load_golden

import optimizer_step_dl_amd as ra
from optimizer_step_dl_amd import _abi


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ra.LIB_PATH):
        from optimizer_step_dl_amd import build
        build.build()
    return ra.load()


def declared_symbols():
    with open(os.path.join(ROOT, "include", "radamw.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(radamw_[a-z0-9_]+)\s*\(", text))


def test_library_exports_every_declared_symbol(lib):
    declared = declared_symbols()
    assert len(declared) >= 15
    for name in declared:
        assert hasattr(lib, name), name
    assert declared == set(ra.EXPORTS)


def test_no_oracle_symbols_in_product_library(lib):
    # the product library shares nothing with the oracle
    import subprocess
    out = subprocess.run(["nm", "-D", ra.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle_" not in out


def test_options_default_matches_page_defaults(lib):
    gold = load_golden("defaults.json")
    o = ra.radamw_options_default()
    assert (o.beta1, o.beta2, o.eps, o.weight_decay) == (gold["beta1"], gold["beta2"], gold["eps"],
                                                          gold["weight_decay"])
    assert o.lr == gold["example_lr"] and o.amsgrad == 0 and o.maximize == 0


@pytest.mark.parametrize("rows", [1, 2, 1023, 1024, 1025, 4096, 65535, 1048576, 1048577, 2_500_000, 4194304])
def test_stats_plan_matches_oracle(lib, rows):
    assert ra.radamw_stats_plan(rows) == oracle.stats_plan(rows)


def test_stats_plan_rejects_out_of_range(lib):
    gold = load_golden("stats_plan.json")
    for rows in (0, -1, gold["rows_max"] + 1):
        with pytest.raises(ra.RadamwError) as e:
            ra.radamw_stats_plan(rows)
        assert e.value.status == -5
    se, ex = ra.radamw_stats_plan(gold["rows_max"])
    assert se * 4 == gold["max_scratch_bytes"] and ex == gold["max_extra_merge_kernels"]


def test_grad_stats_rows_is_deterministic_and_bounded(lib):
    for dt in (torch.float32, torch.float16, torch.bfloat16):
        assert ra.radamw_grad_stats_rows(0, dt) == 0
        assert ra.radamw_grad_stats_rows(1, dt) == 1
        prev = 0
        for n in (1, 100, 4096, 8192, 8193, 10**6, 10**8, 5 * 10**9):
            r = ra.radamw_grad_stats_rows(n, dt)
            assert 1 <= r <= 8192 and r >= prev
            prev = r
    # the 6.7B-parameter list stays far inside the plan's row limit
    import synth
    rows = sum(ra.radamw_grad_stats_rows(n, torch.bfloat16) for _, n in synth.decoder_7b_shapes())
    assert rows <= load_golden("stats_plan.json")["rows_max"]


def _exact32(x: Fraction) -> np.float32:
    return np.float32(float(x))


@pytest.mark.parametrize("betas", [(0.9, 0.999), (0.8, 0.95)])
def test_host_coefficients_agree_with_oracle_and_exact_values(lib, betas):
    """The library's FP32 constants: those shared with the oracle are
    bit-identical; lr/bc1 and 1/bc2 are the correctly rounded exact values."""
    opts = ra.options(lr=1e-3, beta1=betas[0], beta2=betas[1], weight_decay=0.01)
    oopts = oracle.Options(lr=1e-3, beta1=betas[0], beta2=betas[1], weight_decay=0.01)
    off = 0
    ts = list(range(1, 300)) + [1000, 4096, 10_000]
    for t in ts:
        c = ra.radamw_host_coefficients(opts, t, 128.0)
        o = oracle.coefficients(oopts, t)
        assert np.float32(c[0]) == o["beta1"] and np.float32(c[1]) == o["one_minus_beta1"]
        assert np.float32(c[2]) == o["beta2"] and np.float32(c[3]) == o["one_minus_beta2"]
        assert np.float32(c[5]) == o["decay"] and np.float32(c[8]) == o["eps"]
        assert np.float32(c[4]) == np.float32(1 / 128)
        step = _exact32(Fraction(1e-3) / (1 - Fraction(betas[0]) ** t))
        ibc2 = _exact32(1 / (1 - Fraction(betas[1]) ** t))
        for got, want in ((np.float32(c[6]), step), (np.float32(c[7]), ibc2)):
            d = abs(int(got.view(np.int32)) - int(want.view(np.int32)))
            assert d <= 1
            off += d
    assert off <= 2  # at most rare double-rounding ties
    neg = ra.radamw_host_coefficients(ra.options(maximize=True), 1, 4.0)
    assert neg[4] == -0.25


def _stats(sumsq, count):
    s = ra.Stats()
    bits = np.array([sumsq], np.float64).view(np.uint32)
    s.w[0], s.w[1], s.w[2] = int(bits[0]), int(bits[1]), count
    return s


@pytest.mark.parametrize("sumsq,count,scale,max_norm", [
    (123.456, 0, 128.0, 1.0), (1e-8, 0, 1.0, 1.0), (4e4, 0, 1.0, None), (5.0, 7, 2.0, 1.0),
    (67.38, 0, 1.0, 1.0), (0.0, 0, 1.0, 1.0), (1e6, 0, 1024.0, 1e9)])
def test_decide_matches_oracle(lib, sumsq, count, scale, max_norm):
    ctrl, res = ra.radamw_decide(_stats(sumsq, count), scale, max_norm)
    skip, eff = oracle.decide(sumsq, count, scale, max_norm)
    assert bool(ctrl.skip_update) == skip and res.found_inf == int(skip)
    assert ctrl.gradient_scale == eff
    assert res.nonfinite == count and res.sumsq == sumsq


def test_validation_before_any_device_call(lib):
    """Bad scalars are rejected before the library touches HIP, and nothing
    is launched."""
    before = ra.radamw_launch_count()
    st = _abi._State(0, None, None, None)
    upd = ctypes.c_int32(-7)
    good = ra.options()
    bad_opts = [ra.options(lr=-1.0), ra.options(eps=float("nan")), ra.options(beta1=1.0),
                ra.options(beta2=-0.1), ra.options(weight_decay=float("inf"))]
    for o in bad_opts:
        rc = lib.radamw_step_inplace(None, None, 0, 16, ctypes.byref(st), ctypes.byref(o),
                                     ctypes.byref(ra.control()), None, ctypes.byref(upd))
        assert rc == -1
    for c in (ra.control(0.0), ra.control(-1.0), ra.control(float("inf")), _abi.Control(1.0, 2)):
        rc = lib.radamw_step_inplace(None, None, 0, 16, ctypes.byref(st), ctypes.byref(good),
                                     ctypes.byref(c), None, ctypes.byref(upd))
        assert rc == -1
    rc = lib.radamw_step_inplace(None, None, 7, 16, ctypes.byref(st), ctypes.byref(good),
                                 ctypes.byref(ra.control()), None, ctypes.byref(upd))
    assert rc == -1
    rc = lib.radamw_step_inplace(None, None, 0, -1, ctypes.byref(st), ctypes.byref(good),
                                 ctypes.byref(ra.control()), None, ctypes.byref(upd))
    assert rc == -1
    # AMSGrad without a v_max buffer is a state error, not an implicit init
    ams = ra.options(amsgrad=True)
    rc = lib.radamw_step_inplace(None, None, 0, 16, ctypes.byref(st), ctypes.byref(ams),
                                 ctypes.byref(ra.control()), None, ctypes.byref(upd))
    assert rc == -2
    # element counts whose byte sizes could overflow: a range error, checked before any pointer
    rc = lib.radamw_step_inplace(None, None, 0, 2**60, ctypes.byref(st), ctypes.byref(good),
                                 ctypes.byref(ra.control()), None, ctypes.byref(upd))
    assert rc == -5
    st_out = _abi._State(0, None, None, None)
    rc = lib.radamw_step(None, None, 0, 2**48 + 1, ctypes.byref(st), None, ctypes.byref(st_out), ctypes.byref(good),
                         ctypes.byref(ra.control()), None, ctypes.byref(upd))
    assert rc == -5 and st_out.step == 0
    assert lib.radamw_grad_stats_rows(2**48 + 1, 0) == -5
    assert lib.radamw_grad_stats_rows(2**48, 2) == 8192
    huge = (_abi._Segment * 2)(_abi._Segment(None, None, None, None, None, 16),
                               _abi._Segment(None, None, None, None, None, 2**62))
    assert lib.radamw_fused_workspace_bytes(huge, 2, 0) == -5
    overflow = _abi._State(2**64 - 1, None, None, None)
    rc = lib.radamw_step_inplace(None, None, 0, 16, ctypes.byref(overflow), ctypes.byref(good),
                                 ctypes.byref(ra.control()), None, ctypes.byref(upd))
    assert rc == -2
    # empty tensor: accepted, nothing launched, no step change
    st7 = _abi._State(7, None, None, None)
    rc = lib.radamw_step_inplace(None, None, 0, 0, ctypes.byref(st7), ctypes.byref(good),
                                 ctypes.byref(ra.control()), None, ctypes.byref(upd))
    assert rc == 0 and upd.value == 0 and st7.step == 7
    assert upd.value == 0
    assert ra.radamw_launch_count() == before
    assert ra.radamw_status_string(-3) == "overlapping buffers"


def test_binding_rejects_host_and_strided_tensors(lib):
    p = torch.zeros(8)
    with pytest.raises(ValueError):
        ra.radamw_step_inplace(p, torch.zeros(8), ra.AdamWState(0, torch.zeros(8), torch.zeros(8)),
                               ra.options(), ra.control())


def test_list_entry_points_validate_before_any_device_call(lib):
    """The persistent-list entry points reject bad arguments before the
    library touches HIP; destroying NULL is a no-op."""
    before = ra.radamw_launch_count()
    out = ctypes.c_void_p()
    seg = (_abi._Segment * 1)(_abi._Segment(None, None, None, None, None, 16))
    bad_n = (_abi._Segment * 1)(_abi._Segment(None, None, None, None, None, -1))
    models = (ctypes.c_void_p * 1)()
    assert lib.radamw_list_create(seg, 1, 0, 0, None, 0, None, None) == -1          # no list_out
    assert lib.radamw_list_create(seg, -1, 0, 0, None, 0, None, ctypes.byref(out)) == -1
    assert lib.radamw_list_create(None, 2, 0, 0, None, 0, None, ctypes.byref(out)) == -1
    assert lib.radamw_list_create(seg, 1, 7, 0, None, 0, None, ctypes.byref(out)) == -1  # dtype
    assert lib.radamw_list_create(seg, 1, 0, 2, None, 0, None, ctypes.byref(out)) == -1  # amsgrad flag
    assert lib.radamw_list_create(seg, 1, 0, 0, models, 0, None, ctypes.byref(out)) == -1  # FP32 copies
    assert lib.radamw_list_create(bad_n, 1, 0, 0, None, 0, None, ctypes.byref(out)) == -1
    assert out.value is None
    step = ctypes.c_uint64(3)
    upd = ctypes.c_int32(-7)
    good = ra.options()
    assert lib.radamw_list_step(None, ctypes.byref(step), ctypes.byref(good), ctypes.byref(ra.control()), None,
                                ctypes.byref(upd)) == -1
    assert lib.radamw_list_step(None, ctypes.byref(step), ctypes.byref(ra.options(lr=-1.0)),
                                ctypes.byref(ra.control()), None, ctypes.byref(upd)) == -1
    assert lib.radamw_list_step(None, ctypes.byref(step), ctypes.byref(good), ctypes.byref(ra.control(0.0)), None,
                                ctypes.byref(upd)) == -1
    res = _abi.FusedResult()
    assert lib.radamw_list_fused_step(None, ctypes.byref(step), ctypes.byref(good), 1.0, 1.0, 1, None,
                                      ctypes.byref(res)) == -1
    assert lib.radamw_list_fused_step(None, ctypes.byref(step), ctypes.byref(good), float("nan"), 1.0, 1, None,
                                      ctypes.byref(res)) == -1
    assert lib.radamw_list_fused_step(None, ctypes.byref(step), ctypes.byref(good), 1.0, 1.0, 2, None,
                                      ctypes.byref(res)) == -1
    assert lib.radamw_list_destroy(None) == 0
    assert step.value == 3 and upd.value == -7
    assert ra.radamw_launch_count() == before


@pytest.mark.parametrize("n,sizes", [(1 << 28, [4, 4, 4, 4]), (1261529088, [4, 2, 4, 4, 4]), (100_000_007, [4, 2]),
                                     (1, [8]), (0, [4, 4]), (3 * 4096 + 1031, [4, 2, 4, 4, 4, 4, 4, 4, 4])])
def test_bucket_layout_rule(lib, n, sizes):
    """Stream k of a bucket starts at k * pitch, pitch = the widest stream
    rounded up to 2 MiB plus 12 KiB; the streams fit and never overlap."""
    offs, total = ra.radamw_bucket_layout(n, sizes)
    widest = n * max(sizes)
    pitch = -(-widest // (2 << 20)) * (2 << 20) + (12 << 10)
    assert offs == [k * pitch for k in range(len(sizes))] and total == len(sizes) * pitch
    for k, es in enumerate(sizes):
        assert offs[k] % 4096 == 0 and offs[k] + n * es <= (offs[k + 1] if k + 1 < len(sizes) else total)


def test_bucket_layout_rejects_bad_arguments(lib):
    offs = (ctypes.c_int64 * 4)()
    total = ctypes.c_int64(-9)
    eb = (ctypes.c_int32 * 4)(4, 4, 4, 4)
    assert lib.radamw_bucket_layout(16, eb, 0, offs, ctypes.byref(total)) == -1
    assert lib.radamw_bucket_layout(16, eb, 17, offs, ctypes.byref(total)) == -1
    assert lib.radamw_bucket_layout(-1, eb, 4, offs, ctypes.byref(total)) == -1
    assert lib.radamw_bucket_layout(16, None, 4, offs, ctypes.byref(total)) == -1
    assert lib.radamw_bucket_layout(16, eb, 4, None, ctypes.byref(total)) == -1
    assert lib.radamw_bucket_layout(16, eb, 4, offs, None) == -1
    assert lib.radamw_bucket_layout(16, (ctypes.c_int32 * 4)(4, 3, 4, 4), 4, offs, ctypes.byref(total)) == -1
    assert lib.radamw_bucket_layout((1 << 48) + 1, eb, 4, offs, ctypes.byref(total)) == -5
    assert total.value == -9


def test_check_decision_flags_any_disagreement(lib):
    """The fused steps' check of the device's decision against the host's
    (host only): agreement is exact, and every forged disagreement returns
    RADAMW_ERR_DECISION with ``updated`` following the device, which is the
    decision the queued kernels applied."""
    sumsq = 9.0e4  # norm 300 at scale 1: clip = 1 / (300 + 1e-6)
    rep = _stats(sumsq, 0)
    ctrl, want = ra.radamw_decide(rep, 1.0, 1.0)
    inv_bits = int(np.float32(1.0 / ctrl.gradient_scale).view(np.uint32))
    ok, res = ra.radamw_check_decision(rep, 0, inv_bits, 1.0, 1.0)
    assert ok and res.updated == 1 and res.clip_coef == want.clip_coef and res.sumsq == sumsq
    ok, res = ra.radamw_check_decision(rep, 1, inv_bits, 1.0, 1.0)  # device skipped a clean step
    assert not ok and res.updated == 0 and res.found_inf == 0
    ok, res = ra.radamw_check_decision(rep, 0, inv_bits + 1, 1.0, 1.0)  # one FP32 ulp of unscale factor
    assert not ok and res.updated == 1
    bad = _stats(sumsq, 3)  # the host skips
    ok, res = ra.radamw_check_decision(bad, 1, 0x7fc00000, 1.0, 1.0)  # a skip ignores the factor
    assert ok and res.updated == 0 and res.found_inf == 1 and res.nonfinite == 3
    ok, res = ra.radamw_check_decision(bad, 0, inv_bits, 1.0, 1.0)  # device updated a step with inf
    assert not ok and res.updated == 1 and res.found_inf == 1
    dec = (ctypes.c_uint32 * 2)(0, inv_bits)
    assert lib.radamw_check_decision(None, dec, 1.0, 1.0, ctypes.byref(_abi.FusedResult())) == -1
    assert lib.radamw_check_decision(ctypes.byref(rep), None, 1.0, 1.0, ctypes.byref(_abi.FusedResult())) == -1
    assert lib.radamw_check_decision(ctypes.byref(rep), dec, 1.0, 1.0, None) == -1
    assert lib.radamw_check_decision(ctypes.byref(rep), dec, 0.0, 1.0, ctypes.byref(_abi.FusedResult())) == -1
    assert ra.radamw_status_string(-7).startswith("host and device decisions differ")


def test_stream_probe_validates_before_any_device_call(lib):
    """The streaming probe's counts, cap and element count are checked
    before any pointer or device is looked at."""
    before = ra.radamw_launch_count()
    fake = (ctypes.c_void_p * 5)(*([0x1000] * 5))
    call = lambda nr, nw, n=1024, cap=0, ins=fake, outs=fake: lib.radamw_stream_probe(ins, nr, outs, nw, n, cap, None)
    assert call(6, 1) == -1          # more than 5 read streams
    assert call(1, 5) == -1          # more than 4 write streams
    assert call(0, 0) == -1          # no stream at all
    assert call(-1, 1) == -1
    assert call(1, 1, cap=33) == -1  # cap above 32 workgroups per CU
    assert call(1, 1, cap=-1) == -1
    assert call(1, 1, n=-4) == -1
    assert call(1, 1, ins=None) == -1
    assert call(1, 0, outs=None) == -1  # a read-only probe still needs its sink
    assert call(1, 1, n=1022) == -4  # not a whole number of 16-byte chunks
    assert call(1, 1, n=(1 << 48) + 4) == -5
    assert call(1, 1, n=0) == 0      # empty: nothing to launch
    assert ra.radamw_launch_count() == before


def test_lists_fused_step_validates_before_any_device_call(lib):
    """The multi-list fused step rejects a bad array before it reads any
    handle: a handle given twice is caught before it is dereferenced."""
    before = ra.radamw_launch_count()
    res = _abi.FusedResult()
    steps = (ctypes.c_uint64 * 2)(4, 4)
    opts = (_abi.Options * 2)(ra.options(), ra.options())
    fake = ctypes.c_void_p(0x1000)
    twice = (ctypes.c_void_p * 2)(fake.value, fake.value)
    with_null = (ctypes.c_void_p * 2)(fake.value, None)
    call = lambda lists, n, scale=1.0, clip=1.0, hier=1, st=steps, op=opts, out=res: lib.radamw_lists_fused_step(
        lists, n, st, op, scale, clip, hier, None, ctypes.byref(out) if out is not None else None)
    assert call(twice, 2) == -1                   # the same handle twice
    assert call(with_null, 2) == -1               # a NULL handle
    assert call(None, 2) == -1
    assert call(twice, 0) == -1                   # no lists
    assert call(twice, 65537) == -1               # too many lists
    assert call(twice, 2, scale=0.0) == -1
    assert call(twice, 2, clip=float("inf")) == -1
    assert call(twice, 2, hier=3) == -1
    assert call(twice, 2, st=None) == -1
    assert call(twice, 2, op=None) == -1
    assert call(twice, 2, out=None) == -1
    assert list(steps) == [4, 4]
    assert ra.radamw_launch_count() == before


@pytest.mark.parametrize("betas", [(0.9, 0.999), (0.95, 0.9999)])
def test_host_coefficients_at_late_steps(lib, betas):
    """t in [1e4, 1e6]: the library's lr/bc1 and 1/bc2 stay within one FP32
    ulp of the correctly rounded exact values (80-digit decimal powers),
    and its betas are the oracle's."""
    import decimal
    opts = ra.options(lr=1e-3, beta1=betas[0], beta2=betas[1], weight_decay=0.01)
    oopts = oracle.Options(lr=1e-3, beta1=betas[0], beta2=betas[1], weight_decay=0.01)
    for t in sorted(set(int(round(x)) for x in np.logspace(4, 6, 21))):
        c = ra.radamw_host_coefficients(opts, t, 1.0)
        o = oracle.coefficients(oopts, t)
        assert np.float32(c[0]) == o["beta1"] and np.float32(c[2]) == o["beta2"]
        with decimal.localcontext() as ctx:
            ctx.prec = 80
            bc1 = 1 - decimal.Decimal(betas[0]) ** t
            bc2 = 1 - decimal.Decimal(betas[1]) ** t
            step = np.float32(float(decimal.Decimal(1e-3) / bc1))
            ibc2 = np.float32(float(1 / bc2))
        for got, want in ((np.float32(c[6]), step), (np.float32(c[7]), ibc2)):
            assert abs(int(got.view(np.int32)) - int(want.view(np.int32))) <= 1, (t, got, want)


def test_plain_c_consumer(lib, tmp_path):
    """include/radamw.h compiles as strict C99 (gcc -std=c99 -pedantic
    -Werror), libradamw.so links from C, and the entry points that need no
    device answer from C as through the binding: the pages' defaults and
    merge-plan figures, the oracle's FP32 coefficients, the empty-call and
    bad-scale contracts, and no launch."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = os.path.join(ROOT, "tests", "c_abi", "radamw_c_consumer.c")
    exe = str(tmp_path / "radamw_c_consumer")
    libdir = os.path.dirname(ra.LIB_PATH)
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    src, "-L", libdir, "-l:libradamw.so", f"-Wl,-rpath,{libdir}", "-o", exe], check=True)
    out = subprocess.run([exe], capture_output=True, text=True, check=True, timeout=60).stdout
    vals = dict(line.split(" ", 1) for line in out.strip().splitlines())
    gold = load_golden("defaults.json")
    assert float(vals["beta1"]) == gold["beta1"] and float(vals["beta2"]) == gold["beta2"]
    assert float(vals["eps"]) == gold["eps"] and float(vals["weight_decay"]) == gold["weight_decay"]
    assert float(vals["lr"]) == gold["example_lr"] and vals["amsgrad"] == "0" and vals["maximize"] == "0"
    plan = load_golden("stats_plan.json")
    assert vals["plan_rc"] == "0"
    assert int(vals["plan_scratch_elements"]) * 4 == plan["max_scratch_bytes"]
    assert int(vals["plan_extra_merge_kernels"]) == plan["max_extra_merge_kernels"]
    assert int(vals["plan_out_of_range"]) == -5
    assert vals["coef_rc"] == "0"
    c = [np.float32(float(vals[f"coef{i}"])) for i in range(9)]
    o = oracle.coefficients(oracle.Options(), 1000)
    assert (c[0], c[1], c[2], c[3]) == (o["beta1"], o["one_minus_beta1"], o["beta2"], o["one_minus_beta2"])
    assert c[5] == o["decay"] and c[8] == o["eps"] and c[4] == np.float32(1 / 128)
    py = ra.radamw_host_coefficients(ra.options(), 1000, 128.0)
    assert c[6] == np.float32(py[6]) and c[7] == np.float32(py[7])
    assert (vals["empty_rc"], vals["empty_updated"], vals["empty_step"]) == ("0", "0", "7")
    assert vals["bad_scale_rc"] == "-1" and vals["status_alias"] == "overlapping buffers"
    assert vals["launches"] == "0"
