"""bsfa_prefill_noalloc (the workspace in the library's static device scratch) against
bsfa_prefill with a caller workspace, through the C ABI: two calls in a row, the second on a
shorter sequence, so that the scratch still holds the first call's masks, block means and
ticket counters when the second call runs. Results must agree bit for bit."""
import math
import os

import numpy as np
import pytest
import torch

from block_sparse_long_amd import _lib, synth
from block_sparse_long_amd.table import ThresholdTable

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _outputs(Qd, Bq, nkb):
    B, N, Hq, _ = Qd.shape
    nqb = -(-N // Bq)
    return dict(O=torch.full_like(Qd, float("nan"), dtype=torch.float32),
                counts=torch.full((B, Hq, nqb), -7, dtype=torch.int32, device="cuda"),
                total=torch.zeros(1, dtype=torch.int64, device="cuda"),
                stat=torch.full((B, Hq, nqb, nkb), float("nan"), device="cuda"))


def _call(fn, Qd, Kd, Vd, out, **kw):
    fn(Qd, Kd, Vd, out["O"], kept_counts=out["counts"], kept_total=out["total"],
       debug_block_stat=out["stat"], **kw)


def _same(a, b):
    assert torch.equal(a["O"], b["O"])
    assert torch.equal(a["counts"], b["counts"])
    assert torch.equal(a["total"], b["total"])
    assert torch.equal(torch.nan_to_num(a["stat"], nan=7.0), torch.nan_to_num(b["stat"], nan=7.0))


def test_noalloc_equals_caller_workspace_twice_second_smaller():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load_library()
    tab = ThresholdTable.load(os.path.join(GOLDEN, "thresholds_llama_16k.bin"))
    dtab = tab.to_device("cuda", record_budgets=False)   # two launches: the scratch holds the masks
    Bq = 128
    cases = [("llama_16k", 16384, 0, True), ("structured_3000", 3000, 5, False)]
    for name, n, seed, mean in cases:
        print(f"case {name} n={n} mean_correction={mean}", flush=True)
        Q, K, V = synth.structured(seed, n)
        Qd, Kd, Vd = (x.cuda() for x in synth.to_bf16(Q, K, V))
        nkb = -(-n // 64)
        kw = dict(block_q=Bq, gate_mode="absolute", table=dtab, budget_slice=0,
                  mean_correction=mean)
        a = _outputs(Qd, Bq, nkb)
        _call(_lib.bsfa_prefill_noalloc, Qd, Kd, Vd, a, **kw)
        need = _lib.bsfa_prefill_workspace_bytes(Qd, Kd, block_q=Bq, mean_correction=mean)
        ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
        b = _outputs(Qd, Bq, nkb)
        _call(_lib.bsfa_prefill, Qd, Kd, Vd, b, workspace=ws, **kw)
        torch.cuda.synchronize()
        assert int(a["total"].item()) > 0
        assert (a["counts"] < torch.tensor([(i * Bq) // 64 for i in range(-(-n // Bq))],
                                          device="cuda")).any(), "nothing pruned"
        _same(a, b)
        # dense and relative through the same entry point (the scratch holds their ticket
        # counter) against a caller workspace of stale bytes
        for mode, ll in (("dense", -math.inf), ("relative", math.log(1e-3))):
            a = _outputs(Qd, Bq, nkb)
            b = _outputs(Qd, Bq, nkb)
            _call(_lib.bsfa_prefill_noalloc, Qd, Kd, Vd, a, block_q=Bq, gate_mode=mode,
                  log_lambda=ll)
            ws = torch.full((256,), 0xA5, dtype=torch.uint8, device="cuda")
            _call(_lib.bsfa_prefill, Qd, Kd, Vd, b, block_q=Bq, gate_mode=mode, log_lambda=ll,
                  workspace=ws)
            torch.cuda.synchronize()
            _same(a, b)
        del Qd, Kd, Vd
