"""Benchmark of the fused AdamW step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--variants all|none|LIST]
                    [--no-cpu-baseline] [--copy-calibration]

One timed step is one pass of the whole path over a 268,435,456-element flat
FP32 bucket (FP32 gradients, steady state at t = 1000, moments pre-warmed),
one radamw_fused_step_multi call: gradient statistics, the hierarchical
fan-in-1024 merge whose final kernel also takes the skip / clip decision
(global norm clipped at 1.0) on the device, the in-place fused update queued
right behind it, and the 12-byte report read back to the host (the step's
one wait, which overlaps the update).  Inputs are resident in HBM before the
timer starts.  Inside the timed region the update kernel's own start / end HIP
events (radamw_time_next_update: hipExtLaunchKernelGGL on the launch stream)
give the kernel duration the roofline object uses.

Prints ONE JSON line (rank 0).  Extra keys beside the contract's:
"roofline", "cpu_baseline", "cpu_baseline_all_cores", "kernels" (update
kernel timing, rest of the step), "device" (GPU, versions, clocks), "variants" (update-only timings of the bucket's other
configurations), "staged_vs_fused" (the pages' staged baseline A/B),
"decoder_1b_list" (per-tensor vs radamw_step_multi launches),
"decoder_7b_fused_step" (the whole step over a 6.7B-parameter list),
"copy_ceiling" (torch elementwise copy bandwidth, context only).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "fused AdamW step params/s + achieved HBM GB/s (% of peak), 268M FP32"
N_BUCKET = 268_435_456
HBM_PEAK_GBS = 8000.0
BYTES_PER_PARAM = {  # algorithmic bytes moved per element by one update
    ("adamw", "f32", False): 28, ("adamw", "bf16", False): 26, ("adamw", "f16", False): 26,
    ("amsgrad", "f32", False): 36, ("amsgrad", "bf16", False): 34, ("amsgrad", "f16", False): 34,
    ("adamw", "f32", True): 20, ("amsgrad", "f32", True): 24,
    ("adamw", "f32", "bf16copy"): 30,
}
PROFILE_COUNTERS = os.path.join(HERE, "profiles", "update_adamw_f32_268M_counters.md")
KERNEL_SOURCES = [os.path.join(HERE, "optimizer_step_dl_amd", "csrc", f)
                  for f in ("radamw_update.hip", "radamw_math.h", "radamw_internal.h")]


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def kernel_source_hash() -> str:
    """Hash of the update kernel's sources with comments and whitespace
    removed: an edit of code (or of a macro) changes it, a comment does not."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def counters_from_profile():
    """HBM bytes per update dispatch from the committed rocprofv3 counter
    summary, scaled by the copy-kernel calibration recorded with it; None if
    absent or taken on a different kernel source."""
    if not os.path.exists(PROFILE_COUNTERS):
        return None
    with open(PROFILE_COUNTERS) as f:
        text = f.read()
    vals = dict(re.findall(r"^- ([a-z_0-9]+): ([0-9A-Za-z.+\-e]+)\s*$", text, flags=re.M))
    try:
        if vals.get("kernel_source_sha256_16") != kernel_source_hash():
            return None
        return float(vals["hbm_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


def build_inputs(torch, synth, n, variant, gdt, device):
    """Config-3 bucket: p ~ N(0, 0.02), g ~ N(0, 1e-3), m ~ N(0, 1e-4),
    v = N(0, 1e-3)^2, v_max = v * U(1, 1.5); drawn on the device."""
    key = (0, "bucket", n)
    p = synth.normal(n, 0.02, key + ("p",), device)
    g = synth.stored_grad(n, 1e-3, 1.0, gdt, key + ("g",), device)
    m, v, vmax = synth.steady_state(n, key, variant == "amsgrad", device, m_std=1e-4, v_root_std=1e-3)
    return p, g, m, v, vmax


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--n", type=int, default=N_BUCKET)
    ap.add_argument("--variants", default="all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB torch copy (the counter calibration kernel)")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        sys.stderr.write("bench.py: the optimizer step is measured on one GPU only; --gpus above 1 is not "
                         "supported (sharding the step over GPUs is designed, not implemented).\n")
        return 2

    import torch
    import synth
    import optimizer_step_dl_amd as ra
    from optimizer_step_dl_amd import _abi

    lib = ra.load()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    sptr = ctypes.c_void_p(stream.cuda_stream)
    n = args.n
    props = torch.cuda.get_device_properties(dev)
    log(f"device {props.name} ({props.gcnArchName}), {props.multi_processor_count} CUs, n={n}")
    smi_before = smi_snapshot()

    # ---------------------------------------------------- headline step --
    p, g, m, v, _ = build_inputs(torch, synth, n, "adamw", "f32", dev)
    opts = ra.options(lr=1e-3, weight_decay=1e-4)
    seglist = ra.SegmentList([ra.Segment(p, g, m, v, None)])
    ws = torch.empty(ra.radamw_fused_workspace_bytes(seglist), dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = ws.data_ptr(), ws.numel()
    step = ctypes.c_uint64(999)
    result = _abi.FusedResult()
    max_norm = 1.0
    rows_n = lib.radamw_grad_stats_rows(n, 0)
    se, ex = ra.radamw_stats_plan(rows_n)

    def one_step(ev=None):
        # the whole step in one C call: statistics -> merge -> read-back ->
        # decision -> update; ev: the update kernel's own start/end events
        # (the launch follows the read-back synchronisation, so events
        # recorded from the host around it would also time the submission)
        if ev is not None:
            lib.radamw_time_next_update(ev[0].cuda_event, ev[1].cuda_event)
        rc = lib.radamw_fused_step_multi(seglist.array, 1, seglist.code, ctypes.byref(step), ctypes.byref(opts),
                                         1.0, max_norm, 1, ws_ptr, ws_bytes, sptr, ctypes.byref(result))
        if rc != 0:
            raise ra.RadamwError(rc, "radamw_fused_step_multi")
        if not result.updated:
            raise RuntimeError("unexpected non-finite gradient in the benchmark bucket")

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for ev in events:  # create the device events before handing them to the library
        for e in ev:
            e.record(stream)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for k in range(args.steps):
        one_step(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    upd_ms = [e[0].elapsed_time(e[1]) for e in events]
    ms_per_step = wall * 1e3 / args.steps
    value = n / (ms_per_step * 1e-3)
    upd_avg = sum(upd_ms) / len(upd_ms)
    bpp = BYTES_PER_PARAM[("adamw", "f32", False)]
    achieved = bpp * n / (upd_avg * 1e-3) / 1e9
    traffic = counters_from_profile()
    log(f"step {ms_per_step:.3f} ms, update {upd_avg:.3f} ms ({achieved:.0f} GB/s), statistics + merge + "
        f"read-back + decision {ms_per_step - upd_avg:.3f} ms, clip {result.clip_coef:.4f}, norm {result.total_norm:.4f}")
    kernels = {
        "update_adamw_f32_inplace": {"avg_ms": upd_avg, "min_ms": min(upd_ms), "max_ms": max(upd_ms),
                                     "bytes_per_param": bpp, "gbs": achieved},
        "rest_of_step": {"avg_ms": ms_per_step - upd_avg, "what": "grad statistics (4 B/param read), "
                         f"{ex} merge level(s) + final merge, decision taken on the device by the final merge (the host reads the 12-byte report while the update runs), launch latencies",
                         "rows": rows_n, "extra_merge_kernels": ex},
    }
    del p, g, m, v, ws, seglist
    torch.cuda.empty_cache()

    # ------------------------------------------------ update-only variants --
    wanted = [] if args.variants == "none" else (
        ["adamw_f32_outofplace", "amsgrad_f32_inplace", "amsgrad_f32_outofplace", "adamw_bf16_inplace",
         "adamw_f32_firststep", "adamw_f32_bf16copy"] if args.variants == "all" else
        [v for v in args.variants.split(",") if v not in ("decoder_1b", "decoder_7b", "staged", "optim_1b")])
    variants = {}
    for name in wanted:
        variant, gdt, mode = name.split("_")
        first = mode == "firststep"
        amsgrad = variant == "amsgrad"
        p, g, m, v, vmax = build_inputs(torch, synth, n, variant, gdt, dev)
        o = ra.options(lr=1e-3, weight_decay=1e-4, amsgrad=amsgrad)
        c = ra.control(1.0)
        st_step = 0 if first else 999
        if mode == "bf16copy":
            # in place, plus the BF16 model copy written in the same pass
            model = torch.empty(n, dtype=torch.bfloat16, device=dev)
            seg = [ra.Segment(p, g, m, v, vmax)]

            def launch(k):
                ra.radamw_step_multi_writeback(seg, [model], st_step + k, o, c)
        elif mode == "outofplace":
            outs = [torch.empty_like(p), torch.empty_like(m), torch.empty_like(v),
                    torch.empty_like(vmax) if amsgrad else None]
            sets = [(p, m, v, vmax), tuple(outs)]

            def launch(k):
                a, b = sets[k % 2], sets[(k + 1) % 2]
                sin = ra.AdamWState(st_step + k, a[1], a[2], a[3])
                sout = ra.AdamWState(0, b[1], b[2], b[3])
                ra.radamw_step(a[0], g, sin, o, c, b[0], sout)
        else:
            def launch(k):
                st = ra.AdamWState(0 if first else st_step + k, m, v, vmax)
                ra.radamw_step_inplace(p, g, st, o, c)
        for k in range(3):
            launch(k)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        for a, b in ev:
            a.record(stream)
            b.record(stream)
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(ev):
            ra.radamw_time_next_update(a, b)
            launch(k)
        torch.cuda.synchronize()
        ms = [a.elapsed_time(b) for a, b in ev]
        avg = sum(ms) / len(ms)
        bp = BYTES_PER_PARAM[(variant, gdt, "bf16copy" if mode == "bf16copy" else first)]
        variants[name] = {"avg_ms": avg, "min_ms": min(ms), "bytes_per_param": bp,
                          "params_per_s": n / (avg * 1e-3), "gbs": bp * n / (avg * 1e-3) / 1e9,
                          "frac_of_peak": bp * n / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS}
        log(f"variant {name}: {avg:.3f} ms, {variants[name]['gbs']:.0f} GB/s")
        del p, g, m, v, vmax
        if mode == "outofplace":
            del outs, sets
        torch.cuda.empty_cache()

    # --------------------------------------------------- copy ceiling --
    # ------------------------------- staged baseline A/B (the pages' bench) --
    staged = None
    if args.variants == "all" or "staged" in args.variants.split(","):
        staged = bench_staged(torch, synth, ra, dev, stream, n)

    # ----------------------------- tensor list: per-tensor vs one launch --
    decoder = None
    if args.variants == "all" or "decoder_1b" in args.variants.split(","):
        decoder = bench_decoder_list(torch, synth, ra, dev, stream)

    # ------------------ the 6.7B-parameter list: whole fused step at scale --
    decoder7 = None
    if args.variants == "all" or "decoder_7b" in args.variants.split(","):
        decoder7 = bench_decoder_7b(torch, synth, ra, dev, stream)

    # ------------- the torch optimizer over the 1.1B decoder's parameters --
    optim_1b = None
    if args.variants == "all" or "optim_1b" in args.variants.split(","):
        optim_1b = bench_optimizer_1b(torch, synth, ra, dev, stream)

    # A plain elementwise copy of known size (1 GiB read, 1 GiB written):
    # torch's unary negation kernel.  It is the calibration kernel for the
    # rocprofv3 HBM counters and, timed, a context ceiling for streaming.
    copy_ceiling = None
    if args.copy_calibration or wanted:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            torch.neg(a, out=b)
        e1.record(stream)
        torch.cuda.synchronize()
        cms = e0.elapsed_time(e1) / 10
        copy_ceiling = {"kernel": "torch.neg (elementwise copy)", "bytes": 2 * a.numel() * 4, "avg_ms": cms,
                        "gbs": 2 * a.numel() * 4 / (cms * 1e-3) / 1e9}
        log(f"copy ceiling: {copy_ceiling['gbs']:.0f} GB/s")
        del a, b

    # --------------------------------------------------- CPU oracle --
    cpu = cpu_all = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(torch, synth, args.cpu_seconds)
        cpu_all = cpu_baseline_threads(torch, synth, max(1.0, args.cpu_seconds / 4))

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded normal draws on the device)",
        "config": {
            "workload": (f"flat bucket of {n:,} FP32 params, FP32 grads, AdamW lr 1e-3 betas (0.9,0.999) eps 1e-5 "
                         "wd 1e-4, steady state from t=1000, in place; step = grad stats + hierarchical merge + "
                         "12-byte read-back + global-norm clip at 1.0 + fused update"),
            "n_params": n, "grad_dtype": "f32", "optimizer": "adamw", "storage": "in-place",
            "parallelism": "none (1 GPU)",
        },
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "adamw_update_single<f32, adamw, steady>",
                     "algorithmic_bytes_per_launch": bpp * n},
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_all,
        "kernels": kernels,
        "variants": variants,
        "copy_ceiling": copy_ceiling,
        "decoder_1b_list": decoder,
        "staged_vs_fused": staged,
        "decoder_7b_fused_step": decoder7,
        "fusedadamw_1b": optim_1b,
        "device": {"name": props.name, "arch": props.gcnArchName, "cus": props.multi_processor_count,
                   "torch": torch.__version__, "hip": torch.version.hip,
                   "memory_bytes": props.total_memory, "rocm_smi_before": smi_before,
                   "rocm_smi_after": smi_snapshot()},
    }
    print(json.dumps(out), flush=True)
    return 0


def bench_staged(torch, synth, ra, dev, stream, n):
    """Fused update against the staged baseline (4 launches, 5 with AMSGrad,
    through a delta buffer; 48 / 60 B per parameter in the pages' model).
    (1) Device time per step on the 2^28 bucket, back-to-back launches.
    (2) The pages' A/B shape: 65,536 elements, BF16 grads, AMSGrad, 20
    iterations per sample x 7 samples, every arm started from the same
    materialised state, order reversed every other sample, synchronised
    before and after every batch, wall-clock ms per step (median / min /
    max).  Arms: fused in place, staged, and fused out of place with its
    outputs allocated every step (the pages' out-of-place API allocates)."""
    out = {}
    for variant, bpp_f, bpp_s in (("adamw", 28, 48), ("amsgrad", 36, 60)):
        amsgrad = variant == "amsgrad"
        p, g, m, v, vmax = build_inputs(torch, synth, n, variant, "f32", dev)
        delta = torch.empty_like(p)
        o = ra.options(lr=1e-3, weight_decay=1e-4, amsgrad=amsgrad)
        c = ra.control(1.0)
        res = {}
        for name, fn in (("fused", lambda k: ra.radamw_step_inplace(p, g, ra.AdamWState(999 + k, m, v, vmax), o, c)),
                         ("staged", lambda k: ra.radamw_step_staged_inplace(p, g, ra.AdamWState(999 + k, m, v, vmax),
                                                                            delta, o, c))):
            for k in range(3):
                fn(k)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for k in range(20):
                fn(k)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 20
            bpp = bpp_f if name == "fused" else bpp_s
            res[name] = {"device_ms": ms, "model_bytes_per_param": bpp, "params_per_s": n / (ms * 1e-3),
                         "model_gbs": bpp * n / (ms * 1e-3) / 1e9}
        res["speedup"] = res["staged"]["device_ms"] / res["fused"]["device_ms"]
        log(f"staged vs fused, {variant} 2^28: fused {res['fused']['device_ms']:.3f} ms, staged "
            f"{res['staged']['device_ms']:.3f} ms, x{res['speedup']:.2f}")
        out[f"{variant}_f32_bucket"] = res
        del p, g, m, v, vmax, delta
        torch.cuda.empty_cache()

    # the pages' A/B shape
    small = 65536
    key = (0, "ab-small")
    p0 = synth.normal(small, 0.02, key + ("p",), dev)
    g = synth.stored_grad(small, 1e-3, 128.0, "bf16", key + ("g",), dev)
    m0, v0, x0 = synth.steady_state(small, key, True, dev)
    o = ra.options(lr=1e-3, weight_decay=0.01, amsgrad=True)
    c = ra.control(128.0)
    names = ("fused", "staged", "fused_out_of_place")
    arms = {}
    for name in names:
        arms[name] = [p0.clone(), m0.clone(), v0.clone(), x0.clone(), torch.empty_like(p0)]

    def run(name, k):
        p, m, v, x, d = arms[name]
        st = ra.AdamWState(10 + k, m, v, x)
        if name == "fused":
            ra.radamw_step_inplace(p, g, st, o, c)
        elif name == "staged":
            ra.radamw_step_staged_inplace(p, g, st, d, o, c)
        else:
            # the pages' out-of-place form: fresh outputs allocated every step
            out = [torch.empty_like(p), torch.empty_like(m), torch.empty_like(v), torch.empty_like(x)]
            ra.radamw_step(p, g, st, o, c, out[0], ra.AdamWState(0, out[1], out[2], out[3]))
            arms[name][:4] = out

    for name in arms:  # warm both
        for k in range(5):
            run(name, k)
    for name in arms:  # restart both from the same materialised state
        for dst, src in zip(arms[name][:4], (p0, m0, v0, x0)):
            dst.copy_(src)
    torch.cuda.synchronize()
    samples = {name: [] for name in names}
    same = True
    for sample in range(7):
        order = names if sample % 2 == 0 else names[::-1]
        for name in order:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for k in range(20):
                run(name, 20 * sample + k)
            torch.cuda.synchronize()
            samples[name].append((time.perf_counter() - t0) * 1e3 / 20)
        # every arm has now run the same iterations: parameters and moments
        # must agree bit for bit after every measured batch
        same = same and all(torch.equal(a.view(torch.int32), b.view(torch.int32))
                            for other in ("staged", "fused_out_of_place")
                            for a, b in zip(arms["fused"][:4], arms[other][:4]))
    shape = {"elements": small, "grad_dtype": "bf16", "amsgrad": True, "iterations": 20, "samples": 7,
             "states_bit_identical_after_every_batch": bool(same)}
    for name, xs in samples.items():
        xs = sorted(xs)
        shape[name] = {"wall_ms_per_step_median": xs[len(xs) // 2], "min": xs[0], "max": xs[-1]}
    log(f"A/B 65,536 bf16 AMSGrad wall ms/step: fused {shape['fused']['wall_ms_per_step_median']:.4f}, staged "
        f"{shape['staged']['wall_ms_per_step_median']:.4f}, fused out of place with allocation "
        f"{shape['fused_out_of_place']['wall_ms_per_step_median']:.4f}, identical states: {same}")
    out["pages_ab_shape_65536_bf16_amsgrad"] = shape
    return out


def bench_decoder_7b(torch, synth, ra, dev, stream):
    """The whole fused step over 291 tensors shaped like a 6.7B decoder
    (BF16 grads N(0,1e-4), in-place AdamW, steady state at t = 11):
    statistics of all gradients (13.5 GB read), hierarchical merge, 12-byte
    read-back, clip at 1.0, update (227 launches: 226 large tensors alone,
    the 65 norm vectors in one).  Timed twice: one radamw_fused_step_multi
    call per step (every call validates 1164 buffers), then the same steps
    through a persistent tensor list (validated once)."""
    shapes = synth.decoder_7b_shapes()
    total = synth.total(shapes)
    segs = []
    for i, (_, n) in enumerate(shapes):
        key = (0, "dec7b-bench", i)
        p = synth.normal(n, 0.02, key + ("p",), dev)
        g = synth.stored_grad(n, 1e-4, 1.0, "bf16", key + ("g",), dev)
        m, v, _ = synth.steady_state(n, key, False, dev, m_std=1e-5, v_root_std=1e-4)
        segs.append(ra.Segment(p, g, m, v, None))
    seglist = ra.SegmentList(segs)
    ws = torch.empty(ra.radamw_fused_workspace_bytes(seglist), dtype=torch.uint8, device=dev)
    opts = ra.options(lr=1e-3, weight_decay=1e-4)

    def timed(call, step):
        times, upd = [], []
        for k in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            b.record(stream)
            torch.cuda.synchronize()
            ra.radamw_time_next_update(a, b)
            t0 = time.perf_counter()
            res, step = call(step)
            torch.cuda.synchronize()
            times.append((time.perf_counter() - t0) * 1e3)
            upd.append(a.elapsed_time(b))
        return sorted(times)[2], sorted(upd)[2], res, step

    per_call = lambda st: ra.radamw_fused_step_multi(seglist, st, opts, 1.0, 1.0, True, ws)
    res, step = per_call(10)  # warm
    torch.cuda.synchronize()
    ms_call, ums_call, res, step = timed(per_call, step)
    lst = ra.TensorList(seglist, False)
    listed = lambda st: lst.fused_step(st, opts, 1.0, 1.0, True)
    res, step = listed(step)  # warm
    torch.cuda.synchronize()
    ms, ums, res, step = timed(listed, step)
    lst.close()
    out = {"tensors": len(shapes), "n_params": total, "grad_dtype": "bf16", "steps_timed": 5,
           "path": "radamw_list_fused_step (persistent tensor list)",
           "step_ms_median": ms, "params_per_s": total / (ms * 1e-3), "update_ms_median": ums,
           "update_gbs": 26 * total / (ums * 1e-3) / 1e9, "stats_and_decision_ms": ms - ums,
           "per_call": {"path": "radamw_fused_step_multi (validates every call)", "step_ms_median": ms_call,
                        "update_ms_median": ums_call, "stats_and_decision_ms": ms_call - ums_call},
           "clip_coef": res.clip_coef, "total_norm": res.total_norm, "found_inf": res.found_inf}
    log(f"decoder 6.7B fused step (list): {ms:.2f} ms ({out['params_per_s']:.3g} params/s), update {ums:.2f} ms "
        f"({out['update_gbs']:.0f} GB/s), stats + read-back {ms - ums:.2f} ms; per call {ms_call:.2f} ms; "
        f"clip {res.clip_coef:.4f}")
    del seglist, segs, ws
    torch.cuda.empty_cache()
    return out


def bench_optimizer_1b(torch, synth, ra, dev, stream):
    """FusedAdamW.step() -- the torch optimizer over the C ABI -- on the 201
    parameters of the 1.1B decoder shapes, BF16 gradients N(0,1e-4), AdamW,
    fused_step=True, max_grad_norm=1.0, hierarchical statistics: statistics,
    merge, read-back, decision and update through one persistent tensor list
    per launch bucket.  Wall-clock ms per step between synchronisations,
    next to the C call alone on the same lists (radamw_lists_fused_step)."""
    from optimizer_step_dl_amd.optim import FusedAdamW
    shapes = synth.decoder_1b_shapes()
    n_total = synth.total(shapes)
    params = []
    for i, (_, n) in enumerate(shapes):
        key = (0, "optim-1b", i)
        p = torch.nn.Parameter(synth.normal(n, 0.02, key + ("p",), dev))
        if hasattr(p, "grad_dtype"):
            p.grad_dtype = torch.bfloat16  # a BF16 .grad on an FP32 master parameter
        p.grad = synth.stored_grad(n, 1e-4, 1.0, "bf16", key + ("g",), dev)
        params.append(p)
    opt = FusedAdamW(params, lr=1e-3, weight_decay=1e-4, fused_step=True, max_grad_norm=1.0,
                     hierarchical_stats=True)
    for _ in range(3):
        opt.step()
    torch.cuda.synchronize()
    steps = 20
    t0 = time.perf_counter()
    for _ in range(steps):
        opt.step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    # the same work as one C call per step on the optimizer's own lists
    lists = list(opt._cache.values())
    tlists = [lst for _, lst in lists]
    group = opt.param_groups[0]
    st = [opt.state[params[0]]["step"]] * len(tlists)
    o = [opt._options(group)] * len(tlists)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        _, st = ra.radamw_lists_fused_step(tlists, st, o, 1.0, 1.0, True)
    torch.cuda.synchronize()
    c_ms = (time.perf_counter() - t0) * 1e3 / steps
    res = opt.last_result
    out = {"tensors": len(shapes), "n_params": n_total, "grad_dtype": "bf16", "launch_buckets": len(tlists),
           "step_ms": ms, "params_per_s": n_total / (ms * 1e-3), "c_call_ms": c_ms,
           "python_overhead_ms": ms - c_ms, "clip_coef": res.clip_coef if res else None}
    log(f"FusedAdamW 1.1B fused step: {ms:.3f} ms ({out['params_per_s']:.3g} params/s), the C call alone "
        f"{c_ms:.3f} ms, {len(tlists)} launch bucket(s)")
    del opt, params, lists, tlists
    torch.cuda.empty_cache()
    return out


def bench_decoder_list(torch, synth, ra, dev, stream):
    """201 tensors shaped like a 1.1B decoder, FP16 grads (N(0,1e-4) x 1024,
    scale 1024), AMSGrad at t = 50: 201 per-tensor launches (the pages'
    torch front-end launches one update kernel per parameter) against one
    radamw_step_multi launch over the same list."""
    shapes = synth.decoder_1b_shapes()
    n_total = synth.total(shapes)
    segs = []
    for i, (_, n) in enumerate(shapes):
        key = (0, "dec1b-bench", i)
        p = synth.normal(n, 0.02, key + ("p",), dev)
        g = synth.stored_grad(n, 1e-4, 1024.0, "f16", key + ("g",), dev)
        m, v, vmax = synth.steady_state(n, key, True, dev, m_std=1e-5, v_root_std=1e-4)
        segs.append(ra.Segment(p, g, m, v, vmax))
    opts = ra.options(lr=1e-3, weight_decay=1e-4, amsgrad=True)
    ctrl = ra.control(1024.0)
    states = [ra.AdamWState(49, s.exp_avg, s.exp_avg_sq, s.max_exp_avg_sq) for s in segs]

    def per_tensor():
        for s, st in zip(segs, states):
            st.step = 49
            ra.radamw_step_inplace(s.param, s.grad, st, opts, ctrl)

    def one_launch():
        ra.radamw_step_multi(segs, 49, opts, ctrl)

    out = {"tensors": len(shapes), "n_params": n_total, "bytes_per_param": 34}
    for name, fn in (("per_tensor", per_tensor), ("one_launch", one_launch)):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(10):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / 10
        ms = e0.elapsed_time(e1) / 10
        out[name] = {"device_ms": ms, "wall_ms": wall * 1e3, "params_per_s": n_total / (ms * 1e-3),
                     "gbs": 34 * n_total / (ms * 1e-3) / 1e9}
        log(f"decoder 1.1B list {name}: {ms:.3f} ms device, {wall * 1e3:.3f} ms wall, {out[name]['gbs']:.0f} GB/s")
    del segs, states
    torch.cuda.empty_cache()
    return out


def _cpu_sample(synth, n):
    import oracle
    key = (0, "bucket-cpu", n)
    p = synth.normal(n, 0.02, key + ("p",)).numpy().copy()
    g = synth.grad_numpy(synth.stored_grad(n, 1e-3, 1.0, "f32", key + ("g",)))
    m, v, _ = synth.steady_state(n, key, False)
    st = oracle.State.__new__(oracle.State)
    st.step, st.exp_avg, st.exp_avg_sq, st.max_exp_avg_sq = 999, m.numpy().copy(), v.numpy().copy(), None
    return p, g, st


def cpu_baseline(torch, synth, seconds):
    """The oracle's full step (statistics, decision, update) on a bounded
    sample of the same bucket: the first 2^24 elements, drawn on the CPU with
    the same recipe; repeated until `seconds` have passed.  One core."""
    import oracle
    n = 1 << 24
    p, g, st = _cpu_sample(synth, n)
    opts = oracle.Options(lr=1e-3, weight_decay=1e-4)
    steps = 0
    t0 = time.perf_counter()
    while True:
        sumsq, count = oracle.grad_stats(g, "f32")
        skip, eff = oracle.decide(sumsq, count, 1.0, 1.0)
        oracle.adamw_step(p, g, "f32", st, opts, eff, skip)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    log(f"cpu oracle: {steps} steps of {n} elements in {el:.1f} s")
    return {"value": n * steps / el, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": f"first 2^24 = {n:,} elements of the same bucket recipe (CPU draws), full step "
                      f"(stats + decision + update), {steps} steps in {el:.1f} s, single thread",
            "bytes_per_param_model": 28}


def cpu_baseline_threads(torch, synth, seconds):
    """The same oracle step on all host cores this process may use (at most
    16): the element range is split into one contiguous slice per thread and
    every thread runs the oracle's own scalar loops on its slice (ctypes
    releases the GIL).  The update is elementwise, so the slices compute
    exactly what one call would; the per-slice sums of squares are added
    afterwards, which changes only their FP64 rounding order."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    n = 1 << 24
    p, g, st = _cpu_sample(synth, n)
    opts = oracle.Options(lr=1e-3, weight_decay=1e-4)
    bounds = [(n * k // cores, n * (k + 1) // cores) for k in range(cores)]
    states = []
    for lo, hi in bounds:
        s = oracle.State.__new__(oracle.State)
        s.step, s.exp_avg, s.exp_avg_sq, s.max_exp_avg_sq = st.step, st.exp_avg[lo:hi], st.exp_avg_sq[lo:hi], None
        states.append(s)
    steps = 0
    with ThreadPoolExecutor(max_workers=cores) as pool:
        t0 = time.perf_counter()
        while True:
            parts = list(pool.map(lambda b: oracle.grad_stats(g[b[0]:b[1]], "f32"), bounds))
            skip, eff = oracle.decide(sum(s for s, _ in parts), sum(c for _, c in parts), 1.0, 1.0)
            list(pool.map(lambda k: oracle.adamw_step(p[bounds[k][0]:bounds[k][1]], g[bounds[k][0]:bounds[k][1]],
                                                      "f32", states[k], opts, eff, skip), range(cores)))
            steps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    log(f"cpu oracle on {cores} threads: {steps} steps of {n} elements in {el:.1f} s")
    return {"value": n * steps / el, "unit": "params/s", "cores": cores, "kind": "oracle",
            "sample": f"first 2^24 = {n:,} elements of the same bucket recipe, full step, element range split "
                      f"into {cores} contiguous slices (one thread each), {steps} steps in {el:.1f} s"}


def smi_snapshot():
    """Clocks, power, DPM performance level, temperature, GPU and memory use
    and driver version as rocm-smi reports them (best effort; None if the
    tool is missing or says nothing).  Taken before and after the timed work,
    so that the record shows the settings and any other load on the GPU."""
    import subprocess
    try:
        out = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--showperflevel", "--showtemp",
                              "--showuse", "--showmemuse", "--showdriverversion", "--json"],
                             capture_output=True, text=True, timeout=30)
        data = json.loads(out.stdout)
        snap = {}
        for name, fields in data.items():
            if isinstance(fields, dict):
                snap.update({k.strip(): v for k, v in fields.items()})
        return snap or None
    except Exception:
        return None


if __name__ == "__main__":
    sys.exit(main())
