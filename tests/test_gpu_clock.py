"""The shader-clock probe, a measurement aid beside the GEMM path: one wave
reads the shader-cycle and constant-rate counters across a bounded wait."""

import pytest
import torch

from layout_aware_gemm_amd import tgemm

pytestmark = pytest.mark.gpu


def test_clock_probe_reads_a_plausible_clock():
    out = tgemm.clock_probe(ticks=2000)
    cyc, ticks, rate = out.cpu().tolist()
    assert rate > 0
    assert ticks >= 2000  # the wait ended on the counter, not on the poll cap
    assert cyc > 0
    ghz = tgemm.clock_ghz(out)
    print(f"shader clock {ghz:.3f} GHz over {ticks} ticks at {rate} Hz")
    assert 0.3 < ghz < 3.5


def test_clock_probe_on_a_side_stream():
    s = torch.cuda.Stream()
    out = torch.zeros(3, dtype=torch.int64, device="cuda")
    with torch.cuda.stream(s):
        tgemm.clock_probe(ticks=500, out=out, stream=s)
    s.synchronize()
    assert 0.3 < tgemm.clock_ghz(out) < 3.5
