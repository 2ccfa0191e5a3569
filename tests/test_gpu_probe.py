"""The MFMA rate probe on the GPU: it runs, its accumulators come back finite, and the rate it
measures is a plausible share of the published 2.5 PFLOP/s bf16 peak."""
import math

import pytest
import torch

from block_sparse_long_amd import _lib

pytestmark = pytest.mark.gpu


def test_mfma_rate_probe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load_library()
    sink, fl = _lib.bsfa_mfma_rate_probe(workgroups=1024, iters=4096)
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        _lib.bsfa_mfma_rate_probe(workgroups=1024, iters=4096, sink=sink)
    e1.record()
    torch.cuda.synchronize()
    tflops = 3 * fl / e0.elapsed_time(e1) / 1e9
    print(f"measured bf16 MFMA rate {tflops:.0f} TFLOP/s")
    assert 500.0 < tflops < 2600.0 and not math.isnan(tflops)
