"""The measurement probes run through the C ABI: the streaming read leaves its sink untouched
(the fold never equals the marker for this fill) and the MFMA-rate probe writes every sink entry
with a finite value, in all four modes."""
import numpy as np
import pytest
import torch

import two_tower_cross_amd as tt
from gpu_util import DEV

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("workgroups", [1, 7, 256])
def test_stream_read_probe(workgroups):
    src = torch.full((1 << 20,), 3, dtype=torch.uint8, device=DEV)
    sink = torch.zeros(workgroups, dtype=torch.int32, device=DEV)
    tt.probe_stream_read(src, workgroups, sink)
    torch.cuda.synchronize()
    assert not sink.any()


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
def test_mfma_rate_probe(mode):
    wg = 9
    sink = torch.full((wg * 512 + 5,), float("nan"), dtype=torch.float32, device=DEV)
    flops = tt.probe_mfma_rate(mode, wg, 3, sink)
    torch.cuda.synchronize()
    s = sink.cpu().numpy()
    assert flops == wg * 8 * 3 * 16 * 32768
    assert np.isfinite(s[: wg * 512]).all() and np.isnan(s[wg * 512:]).all()


def test_fence_free_timing_events():
    """Timing events created with hipEventDisableSystemFence measure a kernel like default
    events do (the streaming read of 64 MiB takes some microseconds, the two agree within 50%)."""
    from two_tower_cross_amd.timing import TimingEvent
    src = torch.full((64 << 20,), 3, dtype=torch.uint8, device=DEV)
    sink = torch.zeros(512, dtype=torch.int32, device=DEV)
    tt.probe_stream_read(src, 512, sink)                 # warm-up
    a, b = TimingEvent(), TimingEvent()
    c, d = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    tt.probe_stream_read(src, 512, sink)
    b.record()
    c.record()
    tt.probe_stream_read(src, 512, sink)
    d.record()
    torch.cuda.synchronize()
    t_free, t_default = a.elapsed_time(b), c.elapsed_time(d)
    assert 0.0 < t_free < 10.0 and 0.0 < t_default < 10.0
    assert abs(t_free - t_default) <= 0.5 * max(t_free, t_default)
