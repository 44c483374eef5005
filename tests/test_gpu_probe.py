"""GPU checks of the streaming-ceiling probe (radamw_stream_probe), the
measurement kernel the update's bandwidth is compared with: every read and
write stream is really moved (the outputs equal the sums of the inputs), a
read-only probe writes nothing, and the argument checks hold.

Page abbreviation: FA-ja = "実験的なデバイス上の融合 AdamW / AMSGrad"
(section "残りゲート": optimise from measured profiles)."""
import numpy as np
import pytest
import torch

import synth
import optimizer_step_dl_amd as ra
from gpu_helpers import DEV, announce

pytestmark = pytest.mark.gpu

PATTERNS = [(nr, nw) for nr in range(6) for nw in range(5) if nr + nw > 0]


@pytest.mark.parametrize("nr,nw", PATTERNS)
@pytest.mark.parametrize("cap", [0, 3, 32])
def test_probe_moves_every_stream(nr, nw, cap):
    """out[w] = ((in[0] + in[1]) + ...) + w exactly (FP32 adds in that order);
    a ragged grid: 4 * (3 * 64 * 11 + 17) elements, not a whole number of
    256-element tiles."""
    n = 4 * (3 * 64 * 11 + 17)
    announce(f"stream probe {nr}r/{nw}w cap {cap}")
    ins_h = [synth.normal(n, 1.0, (0, "probe", r)) for r in range(nr)]
    ins = [t.to(DEV) for t in ins_h]
    outs = [torch.full((n,), -7.0, device=DEV) for _ in range(nw)]
    sink = torch.zeros(n, device=DEV) if nw == 0 else None
    ra.radamw_stream_probe(ins, outs, cap, sink)
    torch.cuda.synchronize()
    s = np.zeros(n, np.float32)
    for r, t in enumerate(ins_h):
        s = t.numpy().copy() if r == 0 else (s + t.numpy()).astype(np.float32)
    for w, o in enumerate(outs):
        want = (s + np.float32(w)).astype(np.float32)
        assert np.array_equal(o.cpu().numpy().view(np.uint32), want.view(np.uint32)), (nr, nw, w)
    if sink is not None:
        assert int(torch.count_nonzero(sink)) == 0


def test_probe_in_place_streams():
    """Outputs that are inputs are updated in place, the update's own
    pattern: 4 reads, 3 of them written back."""
    n = 4 * 5003
    announce("stream probe in place 4r/3w")
    host = [synth.normal(n, 1.0, (0, "probe-ip", r)) for r in range(4)]
    ins = [t.to(DEV) for t in host]
    ra.radamw_stream_probe(ins, [ins[0], ins[2], ins[3]])
    torch.cuda.synchronize()
    s = host[0].numpy().copy()
    for t in host[1:]:
        s = (s + t.numpy()).astype(np.float32)
    for w, t in enumerate((ins[0], ins[2], ins[3])):
        assert np.array_equal(t.cpu().numpy().view(np.uint32), (s + np.float32(w)).astype(np.float32).view(np.uint32))
    assert np.array_equal(ins[1].cpu().numpy(), host[1].numpy())  # the read-only stream is untouched


def test_probe_argument_checks():
    announce("stream probe argument checks")
    n = 1024
    a = [torch.ones(n, device=DEV) for _ in range(3)]
    base = torch.empty(n + 4, device=DEV)
    with pytest.raises(ra.RadamwError) as e:  # written range partly overlapping a read range
        ra.radamw_stream_probe([a[0][4:]], [a[0][:n - 4]])
    assert e.value.status == -3
    with pytest.raises(ra.RadamwError) as e:  # the same output twice
        ra.radamw_stream_probe([a[0]], [a[1], a[1]])
    assert e.value.status == -3
    with pytest.raises(ra.RadamwError) as e:  # not 16-byte aligned
        ra.radamw_stream_probe([a[0]], [base[1:n + 1]])
    assert e.value.status == -4
    with pytest.raises(ra.RadamwError) as e:  # n not a multiple of 4
        ra.radamw_stream_probe([a[0][:n - 2]], [a[1][:n - 2]])
    assert e.value.status == -4
    with pytest.raises(ra.RadamwError) as e:  # cap out of range
        ra.radamw_stream_probe([a[0]], [a[1]], 33)
    assert e.value.status == -1
    launches = ra.radamw_launch_count()
    ra.radamw_stream_probe([a[0][:0]], [a[1][:0]])  # empty: no launch
    assert ra.radamw_launch_count() == launches
