"""The calls under HIP graph capture: the library allocates nothing and clears its counters and
totals with small kernels (no memset nodes), so a captured call replays to the eager result. Each
graph is replayed several times, with eager work and a synchronisation between replays, and
every replay is compared with the eager call bit for bit: the absolute gate in two launches
(ticket counters, gate sweep, walk) with bf16 and with FP8 gate scores, and the relative gate.
"""
import math

import numpy as np
import pytest
import torch

from block_sparse_long_amd import _lib, synth
from gpu_util import make_table

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load_library()


CASES = [
    ("absolute", "bf16"),
    ("absolute", "fp8"),
    ("relative", "bf16"),
]


@pytest.mark.parametrize("mode,gate_dtype", CASES)
def test_captured_call_replays_to_the_eager_result(mode, gate_dtype):
    N, Hq, Hkv, d, Bq = 3000, 8, 2, 128, 128
    print(f"case {mode} {gate_dtype} N={N}", flush=True)
    Q, K, V = synth.structured(31, N, heads_q=Hq, heads_kv=Hkv, d=d, needles=4)
    Qd, Kd, Vd = (x.cuda() for x in synth.to_bf16(Q, K, V))
    nqb = -(-N // Bq)
    kw = dict(block_q=Bq, gate_mode=mode)
    if mode == "absolute":
        # per head, the median of its off-diagonal block maxima (computed here on the CPU), so
        # that about half of the blocks are pruned
        Qf, Kf = (x.float() for x in synth.to_bf16(Q, K))
        T = np.full((1, Hq, nqb), -np.inf, np.float32)
        for h in range(Hq):
            S = (Qf[0, :, h] @ Kf[0, :, h // (Hq // Hkv)].T) / math.sqrt(d)
            for i in range(1, nqb):
                n_off = (i * Bq) // 64
                m = S[i * Bq:min((i + 1) * Bq, N), :n_off * 64].reshape(-1, n_off, 64)
                T[0, h, i] = float(np.median(m.amax(dim=(0, 2)).numpy()))
        # without its budgets: a workspace then always means two launches
        kw.update(table=make_table(T, Bq, d, [4]).to_device("cuda", record_budgets=False),
                  budget_slice=0, gate_dtype=gate_dtype)
        need = _lib.bsfa_prefill_workspace_bytes(Qd, Kd, block_q=Bq, gate_dtype=gate_dtype)
        kw["workspace"] = torch.zeros(need, dtype=torch.uint8, device="cuda")
    else:
        kw["log_lambda"] = math.log(1e-2)
    O = torch.empty((1, N, Hq, d), dtype=torch.float32, device="cuda")
    counts = torch.empty((1, Hq, nqb), dtype=torch.int32, device="cuda")
    total = torch.empty(1, dtype=torch.int64, device="cuda")

    def call():
        _lib.bsfa_prefill(Qd, Kd, Vd, O, kept_counts=counts, kept_total=total,
                          out_dtype=torch.float32, **kw)

    call()
    torch.cuda.synchronize()
    ref = (O.clone(), counts.clone(), total.clone())
    assert int(ref[2].item()) > 0
    if mode == "absolute":   # something was pruned, so the walk skipped tiles
        n_off = torch.tensor([(i * Bq) // 64 for i in range(nqb)], device="cuda")
        assert (ref[1] < n_off).any()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()   # warm-up off the default stream, as capture requires
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for r in range(3):
        O.fill_(float("nan"))
        counts.fill_(-7)
        total.fill_(12345)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(O, ref[0]), f"replay {r}: output"
        assert torch.equal(counts, ref[1]), f"replay {r}: kept counts"
        assert torch.equal(total, ref[2]), f"replay {r}: kept total"
        call()   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(O, ref[0])
