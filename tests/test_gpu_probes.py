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
