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
               workspace=None, record_budgets=False):
    B, N, Hq, _ = Qd.shape
    nqb, nkb = -(-N // block_q), -(-int(Kd.shape[1]) // 64)
    counts = torch.full((B, Hq, nqb), -7, dtype=torch.int32, device="cuda")
    total = torch.zeros(1, dtype=torch.int64, device="cuda")
    stat = torch.full((B, Hq, nqb, nkb), float("nan"), dtype=torch.float32, device="cuda") if dbg else None
    dtab = table.to_device("cuda", record_budgets) if table is not None else None
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


def quantile_table(Qh, Kh, Bq, Bk, q=0.75, n_budgets=2):
    """Per-head thresholds at the q-quantile of the off-diagonal block maxima of a few query
    blocks (host numpy on the rounded inputs), so that about 1 - q of the blocks are kept."""
    B, N, Hq, d = Qh.shape
    Nk, G = Kh.shape[1], Hq // Kh.shape[2]
    P = Nk - N
    sc = np.float32(1 / math.sqrt(d))
    nqb = -(-N // Bq)
    T = np.zeros((n_budgets, Hq, P // Bq + nqb), np.float32)
    for h in range(Hq):
        maxima = []
        for i in sorted({nqb // 2, nqb - 1}):
            n_off = oracle.key_block_range(i, N, Bq, Bk, P)[0]
            if n_off == 0:
                continue
            s = (Qh[0, i * Bq:(i + 1) * Bq, h] @ Kh[0, :n_off * Bk, h // G].T) * sc
            maxima += list(s.reshape(s.shape[0], n_off, Bk).max(axis=(0, 2)))
        for sl in range(n_budgets):
            T[sl, h] = np.quantile(maxima, q - 0.2 * sl)
    return make_table(T, Bq, d, list(range(1, n_budgets + 1)), block_k=Bk)


def varlen_batch(seed, Hq, Hkv, d, nq, nk):
    """Packed sequences [tokens, H, d] of the given query / key lengths, and cu_q, cu_k."""
    g = torch.Generator().manual_seed(seed)
    cu_q = np.cumsum([0] + nq).astype(np.int32)
    cu_k = np.cumsum([0] + nk).astype(np.int32)
    Q = torch.randn(int(cu_q[-1]), Hq, d, generator=g) * 1.5
    K = torch.randn(int(cu_k[-1]), Hkv, d, generator=g)
    V = torch.randn(int(cu_k[-1]), Hkv, d, generator=g)
    return Q, K, V, cu_q, cu_k


def pages_of(X, cu, page, seed):
    """Scatter packed sequences [tokens, H, d] into a shuffled page pool (spare pages NaN);
    returns (pool, block table on the device)."""
    rng = np.random.default_rng(seed)
    lens = np.diff(cu)
    n_pages = [-(-int(n) // page) for n in lens]
    free = list(rng.permutation(sum(n_pages) + 3))
    pool = torch.full((len(free), page) + tuple(X.shape[1:]), float("nan"), dtype=X.dtype,
                      device=X.device)
    table = torch.zeros((len(lens), max(max(n_pages), 1)), dtype=torch.int32)
    for b, n in enumerate(lens):
        for j in range(n_pages[b]):
            pg = free.pop()
            table[b, j] = int(pg)
            m = min(page, int(n) - j * page)
            pool[pg, :m] = X[cu[b] + j * page: cu[b] + j * page + m]
    return pool, table.cuda()


def absolute_parity(Qd, Kd, Vd, Qh, Kh, Vh, *, Bq, Bk, tab, sl=0, query_blocks=None,
                    mean_correction=False, gate_dtype="bf16"):
    """One absolute-gate device call (masks and statistics from bsfa_gate_masks, the sweep the
    call itself runs) against the oracle under the near-tie rule; returns (O, oracle result,
    device keep decisions)."""
    B, N, Hq, d = Qh.shape
    Nk = Kh.shape[1]
    P = Nk - N
    kpb = Bk // 64
    dtab = tab.to_device("cuda", record_budgets=False)   # two launches: the sweep and the walk
    nqb, nkb = -(-N // Bq), -(-Nk // Bk)
    stat = torch.full((B, Hq, nqb, nkb), float("nan"), device="cuda")
    mask = _lib.bsfa_gate_masks(Qd, Kd, dtab, sl, block_q=Bq, block_k=Bk, debug_block_stat=stat,
                                gate_dtype=gate_dtype)
    counts = torch.full((B, Hq, nqb), -7, dtype=torch.int32, device="cuda")
    O = _lib.bsfa_prefill(Qd, Kd, Vd, block_q=Bq, block_k=Bk, gate_mode="absolute", table=dtab,
                          budget_slice=sl, kept_counts=counts, out_dtype=torch.float32,
                          mean_correction=mean_correction, gate_dtype=gate_dtype)
    torch.cuda.synchronize()
    m = np.ascontiguousarray(mask.cpu().numpy()).view(np.uint8)
    bits = np.unpackbits(m, axis=-1, bitorder="little").astype(bool)
    st = stat.cpu().numpy()
    keep = np.zeros((B, Hq, nqb, nkb), bool)
    n_off = np.array([oracle.key_block_range(i, N, Bq, Bk, P)[0] for i in range(nqb)])
    for i in range(nqb):
        keep[:, :, i, :n_off[i]] = bits[:, :, i, 0:kpb * n_off[i]:kpb]
    np.testing.assert_array_equal(counts.cpu().numpy(), keep.sum(-1))
    assert (counts.cpu().numpy() < n_off).any(), "nothing pruned"
    r = oracle.oracle_prefill(Qh, Kh, Vh, block_q=Bq, block_k=Bk, mode="absolute", table=tab.T,
                              budget_slice=sl, forced_keep=keep, band=BAND,
                              mean_correction=mean_correction, gate_dtype=gate_dtype,
                              query_blocks=query_blocks)
    blocks = range(nqb) if query_blocks is None else query_blocks
    rows = np.zeros(N, bool)
    for i in blocks:
        mg = r.margin[:, :, i, :n_off[i]]
        out = np.abs(mg) > BAND
        np.testing.assert_array_equal(r.keep[:, :, i, :n_off[i]][out], keep[:, :, i, :n_off[i]][out])
        fin = np.isfinite(r.stat[:, :, i, :n_off[i]])
        np.testing.assert_allclose(st[:, :, i, :n_off[i]][fin], r.stat[:, :, i, :n_off[i]][fin],
                                   rtol=1e-5, atol=2e-3)
        rows[i * Bq:min((i + 1) * Bq, N)] = True
    Oh = O.cpu().numpy()
    assert np.isfinite(Oh[:, rows]).all()
    err = np.abs(Oh[:, rows] - r.out[:, rows])
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (err.max(), err.mean())
    return O, r, keep
