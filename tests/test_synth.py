"""The dialled relative-gate workload does what it claims: the oracle's relative gate keeps
exactly the off-diagonal blocks that are not cold, at every lambda of the workload's grid
(the skip rate is an input of the workload, as in the BLASST blog's scoreboard), and the
generator is deterministic."""
import math

import numpy as np
import torch

import oracle
from block_sparse_long_amd import synth


def test_dialled_workload_skips_exactly_the_cold_blocks():
    N, Hq, Hkv, d, Bq = 2048, 4, 2, 128, 128
    Q, K, V, cold = synth.dialled(11, N, 0.5, heads_q=Hq, heads_kv=Hkv, d=d)
    Q2, K2, V2, cold2 = synth.dialled(11, N, 0.5, heads_q=Hq, heads_kv=Hkv, d=d)
    assert torch.equal(Q, Q2) and torch.equal(K, K2) and torch.equal(V, V2)
    assert torch.equal(cold, cold2) and not bool(cold[:, 0].any())
    Qh, Kh, Vh = (x.to(torch.bfloat16).float().numpy() for x in (Q, K, V))
    G = Hq // Hkv
    nqb = N // Bq
    hot = np.zeros((1, Hq, nqb), np.int64)
    for h in range(Hq):
        for i in range(nqb):
            n_off = oracle.key_block_range(i, N, Bq, 64)[0]
            hot[0, h, i] = n_off - int(cold[h // G, :n_off].sum())
    for lam in (1e-4, 1e-2):
        r = oracle.oracle_prefill(Qh, Kh, Vh, block_q=Bq, block_k=64, mode="relative",
                                  log_lambda=math.log(lam))
        np.testing.assert_array_equal(r.kept_counts, hot)
        # every decision is far from the threshold (no near-ties on this workload)
        mg = r.margin[~np.isnan(r.margin)]
        assert np.abs(mg).min() > 0.5
    # about half of the off-diagonal blocks are cold
    n_off = sum(oracle.key_block_range(i, N, Bq, 64)[0] for i in range(nqb))
    assert 0.3 < 1 - hot.sum() / (Hq * n_off) < 0.7
