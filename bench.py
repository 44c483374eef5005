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
"roofline" (with the update's fraction of the measured streaming ceiling),
"cpu_baseline", "cpu_baseline_threads", "kernels" (update kernel timing, rest
of the step, the step timed as 7 samples of 20 steps), "stream_ceiling"
(radamw_stream_probe: the update's access pattern with trivial arithmetic),
"device" (GPU, versions, clocks from sysfs), "provenance" (command line,
commit, source and library hashes), "variants" (update-only timings of the
bucket's other configurations),
"staged_vs_fused" (the pages' staged baseline A/B), "decoder_1b_list"
(per-tensor launches, the multi-tensor call over the list, and one
flattened bucket), "decoder_7b_fused_step" (the whole step over a
6.7B-parameter list and as one bucket, with the streaming ceiling at that
stream length), "fusedadamw_1b" (the torch optimizer),
"copy_calibration" (torch's copy kernel used to scale the HBM counters).
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


def time_update(torch, ra, stream, p, g, m, v, vmax, opts, reps=20):
    """Average of the update kernel's own start / end events over ``reps``
    in-place launches at t = 1000."""
    c = ra.control(1.0)
    for k in range(3):
        ra.radamw_step_inplace(p, g, ra.AdamWState(999 + k, m, v, vmax), opts, c)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    for k, (a, b) in enumerate(ev):
        ra.radamw_time_next_update(a, b)
        ra.radamw_step_inplace(p, g, ra.AdamWState(999 + k, m, v, vmax), opts, c)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / reps


def build_inputs(torch, synth, ra, n, variant, gdt, device, layout="bucket", outputs=False):
    """Config-3 bucket: p ~ N(0, 0.02), g ~ N(0, 1e-3), m ~ N(0, 1e-4),
    v = N(0, 1e-3)^2, v_max = v * U(1, 1.5); drawn on the device.  layout
    "bucket": one allocation in the library's stream placement
    (ra.bucket_arena; with ``outputs`` also the out-of-place outputs p', m',
    v', v_max'); "separate": one allocation per stream.  Returns (p, g, m, v,
    v_max or None, outputs or None)."""
    key = (0, "bucket", n)
    amsgrad = variant == "amsgrad"
    p = synth.normal(n, 0.02, key + ("p",), device)
    g = synth.stored_grad(n, 1e-3, 1.0, gdt, key + ("g",), device)
    m, v, vmax = synth.steady_state(n, key, amsgrad, device, m_std=1e-4, v_root_std=1e-3)
    state = [p, g, m, v] + ([vmax] if amsgrad else [])
    nout = (4 if amsgrad else 3) if outputs else 0
    if layout == "separate":
        outs = [torch.empty(n, dtype=torch.float32, device=device) for _ in range(nout)]
    else:
        views = ra.bucket_arena(n, [t.dtype for t in state] + [torch.float32] * nout, device)
        for dst, src in zip(views, state):
            dst.copy_(src)
        state, outs = views[:len(state)], views[len(state):]
        del p, g, m, v, vmax
    outs = (outs + [None])[:4] if outputs else None
    if outs is not None and not amsgrad:
        outs = outs[:3] + [None]
    return state[0], state[1], state[2], state[3], (state[4] if amsgrad else None), outs


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
    smi_before = clock_snapshot(props)

    # ---------------------------------------------------- headline step --
    p, g, m, v, _, _ = build_inputs(torch, synth, ra, n, "adamw", "f32", dev)
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
    # the update kernel's own start / end events on every TIMING_EVERY-th
    # step of the timed region: each pair adds a few microseconds of GPU
    # time to its step, which the step's throughput should not carry
    timed = list(range(0, args.steps, TIMING_EVERY))
    events = {k: [torch.cuda.Event(enable_timing=True) for _ in range(2)] for k in timed}
    for ev in events.values():  # create the device events before handing them to the library
        for e in ev:
            e.record(stream)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps (update events on {len(timed)} of them)")
    t0 = time.perf_counter()
    for k in range(args.steps):
        one_step(events.get(k))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    upd_ms = [events[k][0].elapsed_time(events[k][1]) for k in timed]
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
                                     "launches_timed": len(upd_ms), "of_steps": args.steps,
                                     "bytes_per_param": bpp, "gbs": achieved},
        "rest_of_step": {"avg_ms": ms_per_step - upd_avg, "what": "grad statistics (4 B/param read), "
                         f"{ex} merge level(s) + final merge, decision taken on the device by the final merge (the host reads the 12-byte report while the update runs), launch latencies",
                         "rows": rows_n, "extra_merge_kernels": ex},
    }
    # after the timed region, the pages' timing shape: 7 samples of 20
    # back-to-back steps, each between synchronisations, timed by HIP events
    # on the stream around the sample and by the host's clock
    per_step, per_step_wall = [], []
    for _ in range(7):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        e0.record(stream)
        for _ in range(20):
            one_step()
        e1.record(stream)
        torch.cuda.synchronize()
        per_step_wall.append((time.perf_counter() - t1) * 1e3 / 20)
        per_step.append(e0.elapsed_time(e1) / 20)
    per_step.sort()
    per_step_wall.sort()
    kernels["step_seven_samples_of_20"] = {
        "median_ms": per_step[3], "min_ms": per_step[0], "max_ms": per_step[-1],
        "wall_median_ms": per_step_wall[3], "wall_min_ms": per_step_wall[0], "wall_max_ms": per_step_wall[-1],
        "what": "per step, 7 samples of 20 steps outside the timed region: HIP events on the stream around "
                "each sample, and the host's clock between synchronisations"}
    log(f"step, 7 samples of 20 (events): median {per_step[3]:.4f} ms [{per_step[0]:.4f}, {per_step[-1]:.4f}]; "
        f"wall clock median {per_step_wall[3]:.4f} ms")
    del p, g, m, v, ws, seglist
    torch.cuda.empty_cache()

    # the same update over the same recipe in separate allocations (one per
    # stream), beside the bucket placement the headline uses
    sep = build_inputs(torch, synth, ra, n, "adamw", "f32", dev, layout="separate")
    sep_ms = time_update(torch, ra, stream, sep[0], sep[1], sep[2], sep[3], None, ra.options(lr=1e-3, weight_decay=1e-4))
    sep_gbs = bpp * n / (sep_ms * 1e-3) / 1e9
    kernels["update_adamw_f32_inplace_separate_allocations"] = {"avg_ms": sep_ms, "gbs": sep_gbs,
                                                                "frac_of_peak": sep_gbs / HBM_PEAK_GBS}
    log(f"update in separate allocations: {sep_ms:.3f} ms ({sep_gbs:.0f} GB/s)")
    del sep
    torch.cuda.empty_cache()

    # ------------------------------------- streaming ceiling of the pattern --
    ceiling = bench_stream_ceiling(torch, ra, dev, stream, n)
    ceil_gbs = ceiling["adamw_in_place"]["gbs"]
    log(f"update / ceiling of its own access pattern: {achieved / ceil_gbs:.4f}")

    # ------------------------------------------------ update-only variants --
    wanted = [] if args.variants == "none" else (
        ["adamw_f32_outofplace", "amsgrad_f32_inplace", "amsgrad_f32_outofplace", "adamw_bf16_inplace",
         "amsgrad_f16_inplace", "adamw_f32_firststep", "adamw_f32_bf16copy"] if args.variants == "all" else
        [v for v in args.variants.split(",") if v not in ("decoder_1b", "decoder_7b", "staged", "optim_1b")])
    variants = {}
    for name in wanted:
        variant, gdt, mode = name.split("_")
        first = mode == "firststep"
        amsgrad = variant == "amsgrad"
        p, g, m, v, vmax, outs = build_inputs(torch, synth, ra, n, variant, gdt, dev, outputs=mode == "outofplace")
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
        pattern = VARIANT_CEILING.get(name)
        if pattern in ceiling:
            variants[name].update(stream_ceiling_pattern=pattern,
                                  frac_of_stream_ceiling=variants[name]["gbs"] / ceiling[pattern]["gbs"])
        log(f"variant {name}: {avg:.3f} ms, {variants[name]['gbs']:.0f} GB/s")
        del p, g, m, v, vmax, outs
        if mode == "outofplace":
            del sets
        torch.cuda.empty_cache()

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
    # torch's unary negation kernel, the calibration kernel for the rocprofv3
    # HBM counters (timed too, for context: torch's own launch geometry).
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
        copy_ceiling = {"kernel": "torch.neg (elementwise copy, counter calibration)", "bytes": 2 * a.numel() * 4, "avg_ms": cms,
                        "gbs": 2 * a.numel() * 4 / (cms * 1e-3) / 1e9}
        log(f"copy calibration kernel: {copy_ceiling['gbs']:.0f} GB/s")
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
            "layout": "p, g, m, v in one allocation placed by radamw_bucket_layout",
            "parallelism": "none (1 GPU)",
        },
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "adamw_update_single<f32, adamw, steady>",
                     "algorithmic_bytes_per_launch": bpp * n,
                     "stream_ceiling_gbs": ceil_gbs, "frac_of_stream_ceiling": achieved / ceil_gbs,
                     "stream_ceiling_kernel": "stream_probe<4, 3> over the update's own streams (4 reads, 3 written "
                                              "back in place, bucket placement), best over per-CU caps",
                     "layout": "one allocation, radamw_bucket_layout placement",
                     "separate_allocations_gbs": sep_gbs},
        "cpu_baseline": cpu,
        "cpu_baseline_threads": cpu_all,
        "kernels": kernels,
        "variants": variants,
        "stream_ceiling": ceiling,
        "copy_calibration": copy_ceiling,
        "decoder_1b_list": decoder,
        "staged_vs_fused": staged,
        "decoder_7b_fused_step": decoder7,
        "fusedadamw_1b": optim_1b,
        "device": {"name": props.name, "arch": props.gcnArchName, "cus": props.multi_processor_count,
                   "torch": torch.__version__, "hip": torch.version.hip,
                   "memory_bytes": props.total_memory, "clocks_before": smi_before,
                   "clocks_after": clock_snapshot(props)},
        "provenance": provenance(sys.argv if argv is None else ["bench.py", *argv]),
    }
    print(json.dumps(out), flush=True)
    return 0


STREAM_PATTERNS = (("read_only_1r", 1, 0), ("write_only_1w", 0, 1), ("copy_1r1w", 1, 1),
                   ("first_step_2r3w", 2, 3), ("adamw_4r3w", 4, 3), ("amsgrad_5r4w", 5, 4))
TIMING_EVERY = 5  # the headline's update events go on every 5th timed step
CEILING_CAPS = (0, 4, 5, 6, 7, 8, 9, 10, 11, 12, 14, 16, 32)  # 0: the update kernels' own occupancy rule
# the probe pattern that moves each FP32-gradient variant's streams (a
# 16-bit gradient or model-copy stream has no FP32 probe pattern)
VARIANT_CEILING = {"adamw_f32_outofplace": "adamw_4r3w", "amsgrad_f32_inplace": "amsgrad_in_place",
                   "amsgrad_f32_outofplace": "amsgrad_5r4w", "adamw_f32_firststep": "first_step_in_place"}


def _probe_best(torch, ra, stream, ins, outs, sink, n, nbytes, reps):
    per_cap = {}
    for cap in CEILING_CAPS:
        args = (ins, outs, cap, sink)
        for _ in range(2):
            ra.radamw_stream_probe(*args)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            b.record(stream)
        torch.cuda.synchronize()
        for a, b in ev:
            ra.radamw_time_next_update(a, b)
            ra.radamw_stream_probe(*args)
        torch.cuda.synchronize()
        avg = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
        per_cap["rule" if cap == 0 else str(cap)] = nbytes * n / (avg * 1e-3) / 1e9
    best = max(per_cap, key=per_cap.get)
    return {"gbs": per_cap[best], "best_cap": best, "gbs_at_update_rule": per_cap["rule"],
            "gbs_by_cap": {k: round(v, 1) for k, v in per_cap.items()}}


def bench_stream_ceiling(torch, ra, dev, stream, n, reps=10):
    """radamw_stream_probe over n-element FP32 streams: the update kernel's
    geometry and cache hints with one add per stream instead of the
    optimizer's arithmetic, each pattern at the update's occupancy rule and
    at fixed caps of 4-32 resident workgroups per CU, its ceiling the best
    of them.  "adamw_in_place" is the headline update's own pattern -- four
    streams in the bucket placement, three of them written back in place --
    and is the ceiling the roofline is compared with; "amsgrad_in_place"
    (five streams, four written back) and "first_step_in_place" (p and g
    read, p written back, m and v written) are the other in-place updates'
    patterns; the other patterns use
    separate streams in the bucket placement (4 reads / 3 writes is AdamW out
    of place, 5 / 4 AMSGrad, 2 / 3 a first step), and
    "adamw_4r3w_separate_allocations" one allocation per stream.  Kernel
    start / end events per launch, averaged over `reps` launches."""
    out = {}
    arena = ra.bucket_arena(n, [torch.float32] * 9, dev)
    for k, t in enumerate(arena):
        t.fill_(1.0 + k)
    ins, outs = arena[:5], arena[5:]
    # the in-place updates' own patterns: p, g, m, v (, v_max) read and all
    # but g written back; a first step reads p and g and writes p, m, v
    in_place = (("adamw_in_place", ins[:4], [ins[0], ins[2], ins[3]], 28),
                ("amsgrad_in_place", ins[:5], [ins[0], ins[2], ins[3], ins[4]], 36),
                ("first_step_in_place", ins[:2], [ins[0], ins[2], ins[3]], 20))
    for name, rd, wr, nbytes in in_place:
        r = _probe_best(torch, ra, stream, rd, wr, None, n, nbytes, reps)
        out[name] = dict(r, reads=len(rd), writes=len(wr), bytes_per_element=nbytes, layout="bucket, in place")
        log(f"stream ceiling {name}: {r['gbs']:.0f} GB/s (cap {r['best_cap']}; {r['gbs_at_update_rule']:.0f} "
            "at the update's rule)")
    for name, nr, nw in STREAM_PATTERNS:
        r = _probe_best(torch, ra, stream, ins[:nr], outs[:nw], outs[0] if nw == 0 else None, n, 4 * (nr + nw), reps)
        out[name] = dict(r, reads=nr, writes=nw, bytes_per_element=4 * (nr + nw), layout="bucket")
        log(f"stream ceiling {name}: {r['gbs']:.0f} GB/s (cap {r['best_cap']}; {r['gbs_at_update_rule']:.0f} at the "
            "update's rule)")
    del arena, ins, outs
    torch.cuda.empty_cache()
    sep = [torch.full((n,), 1.0 + k, dtype=torch.float32, device=dev) for k in range(7)]
    r = _probe_best(torch, ra, stream, sep[:4], sep[4:], None, n, 28, reps)
    out["adamw_4r3w_separate_allocations"] = dict(r, reads=4, writes=3, bytes_per_element=28, layout="separate")
    log(f"stream ceiling adamw_4r3w_separate_allocations: {r['gbs']:.0f} GB/s (cap {r['best_cap']})")
    del sep
    torch.cuda.empty_cache()
    return out


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
        p, g, m, v, vmax, _ = build_inputs(torch, synth, ra, n, variant, "f32", dev)
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
    the 65 norm vectors in one).  Timed three ways: one
    radamw_fused_step_multi call per step (every call validates 1164
    buffers), the same steps through a persistent tensor list (validated
    once), and the same parameters as one flattened bucket in the library's
    placement (one analysis and one update launch).  Then the streaming
    probe over FP32 streams of the same element count, the ceiling at this
    stream length."""
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
    del seglist, segs, ws, lst
    torch.cuda.empty_cache()
    # the same parameters as one flattened bucket: p, the BF16 gradient, m
    # and v each one stream of all 6.7e9 elements, in one allocation placed
    # by radamw_bucket_layout, filled tensor by tensor with the same draws
    arena = ra.bucket_arena(total, [torch.float32, torch.bfloat16, torch.float32, torch.float32], dev)
    off = 0
    for i, (_, n) in enumerate(shapes):
        key = (0, "dec7b-bench", i)
        arena[0][off:off + n] = synth.normal(n, 0.02, key + ("p",), dev)
        arena[1][off:off + n] = synth.stored_grad(n, 1e-4, 1.0, "bf16", key + ("g",), dev)
        m, v, _ = synth.steady_state(n, key, False, dev, m_std=1e-5, v_root_std=1e-4)
        arena[2][off:off + n], arena[3][off:off + n] = m, v
        off += n
    del m, v
    flat = ra.TensorList([ra.Segment(*arena)], False)
    flat_step = lambda st: flat.fused_step(st, opts, 1.0, 1.0, True)
    res, step = flat_step(step)  # warm
    torch.cuda.synchronize()
    fms, fums, res, step = timed(flat_step, step)
    flat.close()
    out["flat_bucket"] = {"path": "radamw_list_fused_step over one segment in the bucket placement",
                          "step_ms_median": fms, "params_per_s": total / (fms * 1e-3), "update_ms_median": fums,
                          "update_gbs": 26 * total / (fums * 1e-3) / 1e9, "stats_and_decision_ms": fms - fums,
                          "clip_coef": res.clip_coef}
    log(f"decoder 6.7B fused step (one flattened bucket): {fms:.2f} ms ({total / (fms * 1e-3):.3g} params/s), update "
        f"{fums:.2f} ms ({out['flat_bucket']['update_gbs']:.0f} GB/s), stats + read-back {fms - fums:.2f} ms")
    del arena
    torch.cuda.empty_cache()
    # the streaming ceiling at this size: what the memory system gives the
    # update's geometry falls with the stream length, so the update is also
    # compared with the probe over streams of the same element count
    probe = ra.bucket_arena(total, [torch.float32] * 4, dev)
    for k, t in enumerate(probe):
        t.fill_(1.0 + k)
    r = _probe_best(torch, ra, stream, probe, [probe[0], probe[2], probe[3]], None, total, 28, 3)
    del probe
    torch.cuda.empty_cache()
    out["stream_ceiling"] = dict(
        r, kernel="stream_probe<4, 3>",
        what="4 FP32 streams of the same element count in the bucket placement, 3 written back in place "
             "(28 B/element; the update's BF16 gradient stream moves 2 B/element)",
        list_update_frac=out["update_gbs"] / r["gbs"], flat_update_frac=out["flat_bucket"]["update_gbs"] / r["gbs"])
    log(f"decoder 6.7B stream ceiling (same element count): {r['gbs']:.0f} GB/s (cap {r['best_cap']}); update "
        f"{out['update_gbs'] / r['gbs']:.3f} (list), {out['flat_bucket']['update_gbs'] / r['gbs']:.3f} (flat) of it")
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
    del opt, lists, tlists
    torch.cuda.empty_cache()
    # the same parameters and gradients under flatten=True: one bucket
    # allocation in the library's placement, one analysis and one update
    # launch per step
    opt = FusedAdamW(params, lr=1e-3, weight_decay=1e-4, fused_step=True, max_grad_norm=1.0,
                     hierarchical_stats=True, flatten=True)
    for _ in range(3):
        opt.step()
    torch.cuda.synchronize()
    launches = ra.radamw_launch_count()
    t0 = time.perf_counter()
    for _ in range(steps):
        opt.step()
    torch.cuda.synchronize()
    fms = (time.perf_counter() - t0) * 1e3 / steps
    out["flatten"] = {"step_ms": fms, "params_per_s": n_total / (fms * 1e-3),
                      "launches_per_step": (ra.radamw_launch_count() - launches) / steps,
                      "gbs_at_28_bytes_per_param": 28 * n_total / (fms * 1e-3) / 1e9}
    log(f"FusedAdamW 1.1B fused step, flatten=True: {fms:.3f} ms ({out['flatten']['params_per_s']:.3g} params/s, "
        f"{out['flatten']['launches_per_step']:.0f} launches per step)")
    del opt, params
    torch.cuda.empty_cache()
    return out


def decoder_1b_flat(torch, synth, ra, dev, shapes, key0):
    """The 1.1B decoder's state as one flattened bucket: p, the FP16
    gradient, m, v and v_max of all 1,261,529,088 elements in one allocation
    placed by radamw_bucket_layout, filled tensor by tensor with the list's
    own draws (FP32 masters N(0, 0.02), FP16 gradients N(0, 1e-4) x 1024,
    m ~ N(0, 1e-5), v = N(0, 1e-4)^2, v_max = v U(1, 1.5)).  Returns the five
    streams and each tensor's (offset, size)."""
    total = synth.total(shapes)
    arena = ra.bucket_arena(total, [torch.float32, torch.float16, torch.float32, torch.float32, torch.float32], dev)
    spans, off = [], 0
    for i, (_, n) in enumerate(shapes):
        key = key0 + (i,)
        arena[0][off:off + n] = synth.normal(n, 0.02, key + ("p",), dev)
        arena[1][off:off + n] = synth.stored_grad(n, 1e-4, 1024.0, "f16", key + ("g",), dev)
        m, v, vmax = synth.steady_state(n, key, True, dev, m_std=1e-5, v_root_std=1e-4)
        arena[2][off:off + n], arena[3][off:off + n], arena[4][off:off + n] = m, v, vmax
        spans.append((off, n))
        off += n
    return arena, spans


def bench_decoder_list(torch, synth, ra, dev, stream):
    """201 tensors shaped like a 1.1B decoder, FP16 grads (N(0,1e-4) x 1024,
    scale 1024), AMSGrad at t = 50 (34 B/param), four ways:
      per_tensor   201 radamw_step_inplace calls (the pages' torch front-end
                   launches one update kernel per parameter);
      multi_list   one radamw_step_multi call over the 201 separately
                   allocated tensors: 156 large tensors launched alone, the
                   45 norm vectors in one shared launch, over two streams;
      multi_views  the same call over 201 views of one arena per stream (in
                   the bucket placement of radamw_bucket_layout), which the
                   library merges into one segment: one launch;
      flat_bucket  one radamw_step_multi call over the arena as a single
                   segment: one launch of 1,261,529,088 elements (the pages'
                   pre-flattened bucket, which shares options and step)."""
    shapes = synth.decoder_1b_shapes()
    n_total = synth.total(shapes)
    segs = []
    for i, (_, n) in enumerate(shapes):
        key = (0, "dec1b-bench", i)
        p = synth.normal(n, 0.02, key + ("p",), dev)
        g = synth.stored_grad(n, 1e-4, 1024.0, "f16", key + ("g",), dev)
        m, v, vmax = synth.steady_state(n, key, True, dev, m_std=1e-5, v_root_std=1e-4)
        segs.append(ra.Segment(p, g, m, v, vmax))
    arena, spans = decoder_1b_flat(torch, synth, ra, dev, shapes, (0, "dec1b-bench"))
    views = [ra.Segment(*[a[o:o + n] for a in arena]) for o, n in spans]
    flat = [ra.Segment(*arena)]
    opts = ra.options(lr=1e-3, weight_decay=1e-4, amsgrad=True)
    ctrl = ra.control(1024.0)
    states = [ra.AdamWState(49, s.exp_avg, s.exp_avg_sq, s.max_exp_avg_sq) for s in segs]
    lists = {"multi_list": ra.SegmentList(segs), "multi_views": ra.SegmentList(views),
             "flat_bucket": ra.SegmentList(flat)}

    def per_tensor():
        for s, st in zip(segs, states):
            st.step = 49
            ra.radamw_step_inplace(s.param, s.grad, st, opts, ctrl)

    arms = [("per_tensor", per_tensor)] + [(k, (lambda sl: lambda: ra.radamw_step_multi(sl, 49, opts, ctrl))(sl))
                                           for k, sl in lists.items()]
    out = {"tensors": len(shapes), "n_params": n_total, "bytes_per_param": 34}
    for name, fn in arms:
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        launches = ra.radamw_launch_count()
        fn()
        torch.cuda.synchronize()
        launches = ra.radamw_launch_count() - launches
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(10):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / 10
        ms = e0.elapsed_time(e1) / 10
        gbs = 34 * n_total / (ms * 1e-3) / 1e9
        out[name] = {"device_ms": ms, "wall_ms": wall * 1e3, "launches_per_step": launches,
                     "params_per_s": n_total / (ms * 1e-3), "gbs": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS}
        log(f"decoder 1.1B list {name}: {launches} launches, {ms:.3f} ms device, {wall * 1e3:.3f} ms wall, "
            f"{gbs:.0f} GB/s")
    del segs, states, lists, views, flat, arena
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


CPU_SHARE = 16  # host threads one GPU's job is given on the measurement boxes


def cpu_baseline_threads(torch, synth, seconds):
    """The same oracle step on as many threads as the process may use, at
    most CPU_SHARE (the CPU share of one GPU's job; the record also states
    the affinity mask and the machine's CPU count): the element range is split into one contiguous slice per thread and
    every thread runs the oracle's own scalar loops on its slice (ctypes
    releases the GIL).  The update is elementwise, so the slices compute
    exactly what one call would; the per-slice sums of squares are added
    afterwards, which changes only their FP64 rounding order."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    affinity = len(os.sched_getaffinity(0))
    cores = max(1, min(CPU_SHARE, affinity))
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
            "cpu_share_cap": CPU_SHARE, "affinity_cpus": affinity, "os_cpu_count": os.cpu_count(),
            "sample": f"first 2^24 = {n:,} elements of the same bucket recipe, full step, element range split "
                      f"into {cores} contiguous slices (one thread each), {steps} steps in {el:.1f} s"}


def _read(path):
    try:
        with open(path) as f:
            return f.read().strip()
    except OSError:
        return None


def _gpu_sysfs_dir(props):
    """sysfs directory of the device torch calls cuda:0, found by its PCI
    address; None when the box exposes no amdgpu sysfs for it."""
    addr = f"{props.pci_domain_id:04x}:{props.pci_bus_id:02x}:{props.pci_device_id:02x}.0"
    d = os.path.join("/sys/bus/pci/devices", addr)
    return d if os.path.exists(os.path.join(d, "pp_dpm_sclk")) else None


def clock_snapshot(props):
    """Clocks, DPM performance level, temperatures, power, GPU / memory
    activity and the driver version, read in-process from the amdgpu sysfs
    files of the benchmarked device (no child process: under a profiler's
    preload a spawned tool would initialise the GPU itself).  Taken before
    and after the timed work.  None when sysfs does not expose the device."""
    d = _gpu_sysfs_dir(props)
    if d is None:
        return None

    def current(level_file):
        text = _read(os.path.join(d, level_file))
        if not text:
            return None
        for line in text.splitlines():
            if line.rstrip().endswith("*"):
                return line.split(":", 1)[-1].replace("*", "").strip()
        return None

    snap = {"sysfs": d, "sclk": current("pp_dpm_sclk"), "mclk": current("pp_dpm_mclk"),
            "fclk": current("pp_dpm_fclk"), "socclk": current("pp_dpm_socclk"),
            "perf_level": _read(os.path.join(d, "power_dpm_force_performance_level")),
            "gpu_busy_percent": _read(os.path.join(d, "gpu_busy_percent")),
            "mem_busy_percent": _read(os.path.join(d, "mem_busy_percent")),
            "driver": _read("/sys/module/amdgpu/version")}
    hw = os.path.join(d, "hwmon")
    try:
        for h in sorted(os.listdir(hw)):
            base = os.path.join(hw, h)
            for f in sorted(os.listdir(base)):
                if f.startswith("temp") and f.endswith("_input"):
                    label = _read(os.path.join(base, f.replace("_input", "_label"))) or f
                    val = _read(os.path.join(base, f))
                    if val is not None:
                        snap[f"temp_{label}_C"] = int(val) / 1000.0
                elif f in ("power1_average", "power1_input"):
                    val = _read(os.path.join(base, f))
                    if val is not None:
                        snap[f"{f}_W"] = int(val) / 1e6
    except OSError:
        pass
    return snap


def provenance(argv):
    """What produced this record: the command line, the commit (when the
    tree carries its .git directory), hashes of the update kernel's code and
    of every product source file, and of the library that was loaded."""
    def git_head():
        head = _read(os.path.join(HERE, ".git", "HEAD"))
        if not head:
            return None
        if not head.startswith("ref:"):
            return head
        ref = head.split(None, 1)[1]
        val = _read(os.path.join(HERE, ".git", ref))
        if val:
            return val
        packed = _read(os.path.join(HERE, ".git", "packed-refs")) or ""
        for line in packed.splitlines():
            if line.endswith(" " + ref):
                return line.split()[0]
        return None

    h = hashlib.sha256()
    files = []
    for sub in ("include", os.path.join("optimizer_step_dl_amd", "csrc"), "optimizer_step_dl_amd", "synth"):
        base = os.path.join(HERE, sub)
        for f in sorted(os.listdir(base)):
            if f.endswith((".h", ".hip", ".cpp", ".py")):
                files.append(os.path.join(sub, f))
    files.append("bench.py")
    for rel in files:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    lib = os.path.join(HERE, "optimizer_step_dl_amd", "libradamw.so")
    with open(lib, "rb") as f:
        lib_hash = hashlib.sha256(f.read()).hexdigest()[:16]
    return {"argv": list(argv), "git_commit": git_head(), "kernel_source_sha256_16": kernel_source_hash(),
            "source_tree_sha256_16": h.hexdigest()[:16], "source_files": len(files),
            "library_sha256_16": lib_hash}


if __name__ == "__main__":
    sys.exit(main())
