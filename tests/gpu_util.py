"""Helpers for the GPU parity tests: run the HIP path through the C ABI and compare it with the
CPU oracle under the near-tie rule.

Tolerances (bf16 inputs against the float32 oracle): output max-abs <= 1e-2 and mean-abs
<= 1e-3, measured on the kernel's float32 output (a bf16 output adds its own rounding, up to
0.0156 for |O| in [4, 8); the bf16 output is checked separately to be exactly the float32
result rounded to nearest even); keep decisions bit-exact except for blocks whose gate statistic lies within 1e-2 of
its threshold, where the oracle adopts the device's decision (and, under the relative gate,
carries on with the running max that decision implies).
"""
import math

import numpy as np
import torch

import oracle
from block_sparse_long_amd import _lib
from block_sparse_long_amd.table import ThresholdTable

MAX_ABS = 1e-2
MEAN_ABS = 1e-3
BAND = 1e-2


def bf16_pair(*xs):
    """(device bf16 tensors, host float32 arrays of the same rounded values)."""
    dev = [x.to(torch.bfloat16).cuda() for x in xs]
    host = [x.to(torch.bfloat16).float().numpy() for x in xs]
    return dev, host


def run_device(Qd, Kd, Vd, *, block_q, mode, table=None, budget_slice=0,
               log_lambda=-math.inf, out_dtype=torch.float32, dbg=True, O=None,
               workspace=None):
    B, N, Hq, _ = Qd.shape
    nqb, nkb = -(-N // block_q), -(-int(Kd.shape[1]) // 64)
    counts = torch.full((B, Hq, nqb), -7, dtype=torch.int32, device="cuda")
    total = torch.zeros(1, dtype=torch.int64, device="cuda")
    stat = torch.full((B, Hq, nqb, nkb), float("nan"), dtype=torch.float32, device="cuda") if dbg else None
    dtab = table.to_device("cuda") if table is not None else None
    O = _lib.bsfa_prefill(Qd, Kd, Vd, O, block_q=block_q, gate_mode=mode, table=dtab,
                          budget_slice=budget_slice, log_lambda=log_lambda, kept_counts=counts,
                          kept_total=total, debug_block_stat=stat, out_dtype=out_dtype,
                          workspace=workspace)
    torch.cuda.synchronize()
    return dict(O=O, counts=counts.cpu().numpy(), total=int(total.item()),
                stat=None if stat is None else stat.cpu().numpy())


def make_table(T, block_q, d, budgets=None, block_k=64):
    T = np.asarray(T, np.float32)
    return ThresholdTable(T=T, budgets=budgets or list(range(1, T.shape[0] + 1)),
                          block_q=block_q, block_k=block_k, head_dim=d,
                          softmax_scale=float(np.float32(1 / math.sqrt(d))))


def device_keep(dev, *, N, block_q, mode, table=None, budget_slice=0, log_lambda=-math.inf,
                prefix=0):
    """The device's keep decisions, recomputed from its dumped statistic with the same fp32
    comparison the kernel makes. Returns (keep [B, Hq, nqb, nkb], offdiag mask)."""
    stat = dev["stat"]
    B, Hq, nqb, nkb = stat.shape
    keep = np.zeros(stat.shape, bool)
    off = np.zeros(stat.shape, bool)
    for i in range(nqb):
        n_off, n_end = oracle.key_block_range(i, N, block_q, 64, prefix)
        off[:, :, i, :n_off] = True
        keep[:, :, i, n_off:n_end] = True
        if mode == "dense":
            keep[:, :, i, :n_off] = True
        elif mode == "absolute":
            col = min(prefix // block_q + i, table.t_len - 1)
            thr = table.T[budget_slice][:, col].astype(np.float32)
            keep[:, :, i, :n_off] = stat[:, :, i, :n_off] >= thr[None, :, None]
        else:
            keep[:, :, i, :n_off] = stat[:, :, i, :n_off] >= np.float32(log_lambda)
    return keep, off


def check_parity(dev, Qh, Kh, Vh, *, block_q, mode, table=None, budget_slice=0,
                 log_lambda=-math.inf, query_blocks=None, stat_atol=2e-3):
    """Compare one device run with the oracle; returns the oracle result."""
    N = Qh.shape[1]
    prefix = Kh.shape[1] - N
    keep_dev, off = device_keep(dev, N=N, block_q=block_q, mode=mode, table=table,
                                budget_slice=budget_slice, log_lambda=log_lambda, prefix=prefix)
    # kept counts are the number of kept off-diagonal blocks, and the total their sum
    counts_from_stat = (keep_dev & off).sum(-1)
    np.testing.assert_array_equal(dev["counts"], counts_from_stat)
    assert dev["total"] == int(dev["counts"].sum())
    r = oracle.oracle_prefill(Qh, Kh, Vh, block_q=block_q, block_k=64, mode=mode,
                              table=None if table is None else table.T,
                              budget_slice=budget_slice, log_lambda=log_lambda,
                              forced_keep=keep_dev, band=BAND, query_blocks=query_blocks)
    # keep mask: bit-exact outside the near-tie band
    for i in (range(keep_dev.shape[2]) if query_blocks is None else query_blocks):
        mg = r.margin[:, :, i]
        outside = ~np.isnan(mg) & (np.abs(mg) > BAND)
        np.testing.assert_array_equal(r.keep[:, :, i][outside], keep_dev[:, :, i][outside])
        np.testing.assert_array_equal(r.kept_counts[:, :, i], dev["counts"][:, :, i])
        # the dumped statistic matches the oracle's on every visible block
        vis = ~np.isnan(r.stat[:, :, i])
        a, b = dev["stat"][:, :, i][vis], r.stat[:, :, i][vis]
        fin = np.isfinite(b)
        np.testing.assert_array_equal(a[~fin], b[~fin])
        np.testing.assert_allclose(a[fin], b[fin], rtol=1e-5, atol=stat_atol)
    O = dev["O"].float().cpu().numpy()
    rows = np.ones(N, bool) if query_blocks is None else np.zeros(N, bool)
    if query_blocks is not None:
        for i in query_blocks:
            rows[i * block_q:min((i + 1) * block_q, N)] = True
    err = np.abs(O[:, rows] - r.out[:, rows])
    assert np.isfinite(O[:, rows]).all()
    assert err.max() <= MAX_ABS, f"max-abs {err.max():.3e}"
    assert err.mean() <= MEAN_ABS, f"mean-abs {err.mean():.3e}"
    return r
