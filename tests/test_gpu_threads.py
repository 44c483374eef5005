"""Concurrent callers: the per-device state the library shares between calls
(segment-table staging ring, mapped report page, second update stream) is
locked, and each call orders on its own stream.  Two host threads running
fused steps at the same time, each on its own stream, must get exactly the
results of the same steps run one after the other.

Page abbreviation: TR-zh = "训练与状态保存" (the fused step)."""
import threading

import pytest
import torch

import synth
import optimizer_step_dl_amd as ra
from gpu_helpers import DEV, announce, bits_equal

pytestmark = pytest.mark.gpu

SIZES = {"a": [1 << 22, 5000, 3_000_000, 77, (1 << 22) + 3, 4096],
         "b": [2048, 1 << 22, 100_000, (1 << 22) + 100, 9]}


def _list(name, gdt):
    segs = []
    for i, n in enumerate(SIZES[name]):
        key = (0, "threads", name, i)
        p = synth.normal(n, 0.02, key + ("p",), DEV)
        g = synth.stored_grad(n, 1e-3, 1.0, gdt, key + ("g",), DEV)
        m, v, _ = synth.steady_state(n, key, False, DEV)
        segs.append(ra.Segment(p, g, m, v, None))
    return segs


def _clone(segs):
    return [ra.Segment(s.param.clone(), s.grad.clone(), s.exp_avg.clone(), s.exp_avg_sq.clone(), None) for s in segs]


def _steps(segs, ws, stream, out, key):
    """Three fused steps from t = 10 on `stream`, clipping at 0.5."""
    opts = ra.options(lr=1e-3, weight_decay=1e-4)
    with torch.cuda.stream(stream):
        step = 9
        results = []
        for _ in range(3):
            res, step = ra.radamw_fused_step_multi(segs, step, opts, 1.0, 0.5, True, ws)
            results.append((res.updated, res.nonfinite, res.sumsq, res.clip_coef, step))
    out[key] = results


@pytest.mark.parametrize("gdt", ["f32", "bf16"])
def test_two_threads_on_two_streams_match_sequential_steps(gdt):
    announce(f"two threads fused steps {gdt}")
    lists = {name: _list(name, gdt) for name in SIZES}
    twins = {name: _clone(segs) for name, segs in lists.items()}
    ws = {name: torch.empty(ra.radamw_fused_workspace_bytes(segs), dtype=torch.uint8, device=DEV)
          for name, segs in lists.items()}
    ws_twin = {name: torch.empty_like(w) for name, w in ws.items()}
    torch.cuda.synchronize()
    streams = {name: torch.cuda.Stream() for name in SIZES}
    out = {}
    errors = []

    def worker(name):
        try:
            _steps(lists[name], ws[name], streams[name], out, name)
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(name,), daemon=True) for name in SIZES]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    seq = {}
    for name in SIZES:  # the same steps, one list after the other, on the default stream
        _steps(twins[name], ws_twin[name], torch.cuda.current_stream(), seq, name)
    torch.cuda.synchronize()
    for name in SIZES:
        assert out[name] == seq[name], name
        for s, tw in zip(lists[name], twins[name]):
            assert bits_equal(s.param, tw.param) and bits_equal(s.exp_avg, tw.exp_avg)
            assert bits_equal(s.exp_avg_sq, tw.exp_avg_sq)
