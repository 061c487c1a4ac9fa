"""Measurement aids beside the GEMM path: the shader-clock probe (one wave
reads the shader-cycle and constant-rate counters across a bounded wait)
and the matrix-core ceiling (MFMAs on register operands only)."""

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


@pytest.mark.parametrize("kind", [0, 1])
def test_mfma_ceiling_runs_and_keeps_its_work(kind):
    # each accumulator block takes the same products every iteration, so two
    # iterations give twice one, up to the fp32 roundings of the matrix
    # core's accumulation (it does not add a whole product sum to the
    # accumulator in one rounding: not bit-exact); values finite, non-zero
    one = torch.zeros(256 * 4, dtype=torch.float32, device="cuda")
    two = torch.zeros_like(one)
    tgemm.mfma_ceiling(1, one, kind=kind)
    tgemm.mfma_ceiling(2, two, kind=kind)
    torch.cuda.synchronize()
    assert torch.isfinite(one).all() and torch.isfinite(two).all()
    assert (one != 0).all()
    torch.testing.assert_close(two, 2 * one, rtol=1e-5, atol=1e-6)
