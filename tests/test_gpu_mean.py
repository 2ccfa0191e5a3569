"""GPU parity of mean correction ("FlashPrefill V2: Block-Sparse Prefill Attention for
Long-Context LLM Serving", mean correction): the HIP path through the C ABI against the CPU
oracle with mean_correction=True, on the same seeded inputs.

Bar: keep decisions (from bsfa_gate_masks, the same sweep the call runs) bit-exact outside the
1e-2 near-tie band, kept counts exact, output max-abs <= 1e-2 and mean-abs <= 1e-3 against the
float32 oracle. Identities: with every key of a block equal, the corrected output is the dense
output; a call where nothing is pruned is bitwise the uncorrected one; packed and paged
variable-length batches are bitwise one call per sequence.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_long_amd import _lib, synth
from gpu_util import (BAND, MAX_ABS, MEAN_ABS, absolute_parity, bf16_pair, make_table,
                      pages_of, quantile_table, varlen_batch)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load_library()


def _inputs(seed, N, Hq, Hkv, d, B=1):
    if B == 1:
        Q, K, V = synth.structured(seed, N, heads_q=Hq, heads_kv=Hkv, d=d, needles=4)
    else:
        Q, K, V = synth.uniform_mix(seed, B, N, Hq, Hkv, d)
        Q = Q * 1.5
    return Q, K, V


CASES = {   # name: (B, N, P, Hq, Hkv, d, Bq, Bk, query blocks checked or None for all)
    "llama_like_ragged": (1, 1000, 0, 8, 2, 128, 128, 64, None),
    "d64_bq64_g2_batch2": (2, 333, 0, 4, 2, 64, 64, 64, None),
    "d128_bq64_g4": (1, 700, 0, 8, 2, 128, 64, 64, None),
    "g8": (1, 384, 0, 16, 2, 128, 128, 64, None),
    "prefix_256": (1, 744, 256, 8, 2, 128, 128, 64, None),
    "bk128_ragged": (1, 1000, 0, 8, 2, 128, 128, 128, None),
    "d64_bk128": (1, 515, 0, 2, 2, 64, 128, 128, None),
    # more than 64 gate blocks: two mean tiles, the second ragged
    "two_mean_tiles": (1, 4600, 0, 2, 1, 128, 128, 64, [0, 20, 34, 35]),
    "two_mean_tiles_bk128": (1, 9100, 0, 2, 1, 128, 128, 128, [1, 40, 70, 71]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_mean_correction_parity(name):
    B, N, P, Hq, Hkv, d, Bq, Bk, qb = CASES[name]
    print(f"case {name}", flush=True)
    Q, K, V = _inputs(31, N + P, Hq, Hkv, d, B)
    Q = Q[:, P:]
    (Qd, Kd, Vd), (Qh, Kh, Vh) = bf16_pair(Q, K, V)
    tab = quantile_table(Qh, Kh, Bq, Bk)
    for sl in (0, 1):
        absolute_parity(Qd, Kd, Vd, Qh, Kh, Vh, Bq=Bq, Bk=Bk, tab=tab, sl=sl, query_blocks=qb,
                        mean_correction=True)


@pytest.mark.parametrize("Bq,Bk,d", [(128, 64, 128), (64, 64, 64), (128, 128, 128)])
def test_block_constant_keys_give_the_dense_output(Bq, Bk, d):
    # every key of a gate block equal: sum_j e^{s_j} v_j = |B| e^{s} vbar, so the corrected
    # output is the dense one with every off-diagonal block pruned (T = +inf)
    N, Hq, Hkv = 1300, 4, 2
    g = torch.Generator().manual_seed(32)
    Q = torch.randn(1, N, Hq, d, generator=g)
    K = torch.randn(1, N, Hkv, d, generator=g)
    K = K[:, (torch.arange(N) // Bk) * Bk]            # each block repeats its first key
    V = torch.randn(1, N, Hkv, d, generator=g)
    (Qd, Kd, Vd), _ = bf16_pair(Q, K, V)
    T = np.full((1, Hq, 1), np.inf, np.float32)
    dtab = make_table(T, Bq, d, [1], block_k=Bk).to_device("cuda")
    kw = dict(block_q=Bq, block_k=Bk, out_dtype=torch.float32)
    dense = _lib.bsfa_prefill(Qd, Kd, Vd, gate_mode="dense", **kw)
    corr = _lib.bsfa_prefill(Qd, Kd, Vd, gate_mode="absolute", table=dtab, mean_correction=True,
                             **kw)
    plain = _lib.bsfa_prefill(Qd, Kd, Vd, gate_mode="absolute", table=dtab, **kw)
    torch.cuda.synchronize()
    err = (corr - dense).abs()
    assert err.max().item() <= MAX_ABS and err.mean().item() <= MEAN_ABS, \
        (err.max().item(), err.mean().item())
    assert (plain - dense).abs().max().item() > 0.1


@pytest.mark.parametrize("T", [-math.inf, -1e4])
def test_nothing_pruned_is_bitwise_the_uncorrected_call(T):
    B, N, Hq, Hkv, d, Bq = 1, 1000, 8, 2, 128, 128
    Q, K, V = _inputs(33, N, Hq, Hkv, d)
    (Qd, Kd, Vd), _ = bf16_pair(Q, K, V)
    dtab = make_table(np.full((1, Hq, 8), T, np.float32), Bq, d, [1]).to_device("cuda")
    kw = dict(block_q=Bq, gate_mode="absolute", table=dtab, out_dtype=torch.float32)
    a = _lib.bsfa_prefill(Qd, Kd, Vd, mean_correction=True, **kw)
    b = _lib.bsfa_prefill(Qd, Kd, Vd, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("Bk", [64, 128])
def test_varlen_and_paged_equal_one_call_per_sequence_bitwise(Bk):
    Hq, Hkv, d, Bq = 8, 2, 128, 128
    nq, nk = [1000, 0, 300, 128, 517], [1000, 0, 556, 256, 773]
    Q, K, V, cu_q, cu_k = varlen_batch(34, Hq, Hkv, d, nq, nk)
    (Qd, Kd, Vd), _ = bf16_pair(Q, K, V)
    # thresholds around the median block maximum of these inputs: about half the blocks pruned
    T = np.random.default_rng(5).uniform(5.0, 6.5, (1, Hq, 16)).astype(np.float32)
    dtab = make_table(T, Bq, d, [1], block_k=Bk).to_device("cuda")
    kw = dict(block_q=Bq, block_k=Bk, gate_mode="absolute", table=dtab, out_dtype=torch.float32,
              mean_correction=True)
    cq, ck = torch.tensor(cu_q, device="cuda"), torch.tensor(cu_k, device="cuda")
    Ov = _lib.bsfa_prefill_varlen(Qd, Kd, Vd, cq, ck, max(nq), max(nk), **kw)
    Kp, tbl = pages_of(Kd, cu_k, 128, 9)
    Vp, _ = pages_of(Vd, cu_k, 128, 9)
    lens = torch.tensor(np.diff(cu_k), dtype=torch.int32, device="cuda")
    Op = _lib.bsfa_prefill_paged(Qd, Kp, Vp, cq, lens, tbl, max(nq), max(nk), **kw)
    plain = dict(kw, mean_correction=False)
    Ou = _lib.bsfa_prefill_varlen(Qd, Kd, Vd, cq, ck, max(nq), max(nk), **plain)
    torch.cuda.synchronize()
    assert torch.equal(Ov, Op)
    assert (Ov - Ou).abs().max().item() > 1e-3      # blocks were pruned and corrected
    for b in range(len(nq)):
        if nq[b] == 0:
            continue
        q = Qd[cu_q[b]:cu_q[b + 1]][None]
        k = Kd[cu_k[b]:cu_k[b + 1]][None]
        v = Vd[cu_k[b]:cu_k[b + 1]][None]
        O1 = _lib.bsfa_prefill(q, k, v, **kw)
        torch.cuda.synchronize()
        assert torch.equal(O1[0], Ov[cu_q[b]:cu_q[b + 1]]), b


def test_varlen_mean_correction_matches_oracle():
    Hq, Hkv, d, Bq = 4, 2, 64, 64
    nq, nk = [200, 333, 64], [328, 333, 192]
    Q, K, V, cu_q, cu_k = varlen_batch(35, Hq, Hkv, d, nq, nk)
    (Qd, Kd, Vd), (Qh, Kh, Vh) = bf16_pair(Q, K, V)
    T = np.full((1, Hq, 8), 5.3, np.float32)      # about the median block maximum here
    tab = make_table(T, Bq, d, [1])
    dtab = tab.to_device("cuda")
    O = _lib.bsfa_prefill_varlen(Qd, Kd, Vd, torch.tensor(cu_q, device="cuda"),
                                 torch.tensor(cu_k, device="cuda"), max(nq), max(nk), block_q=Bq,
                                 gate_mode="absolute", table=dtab, out_dtype=torch.float32,
                                 mean_correction=True)
    # the device's decisions per sequence (the sweep of a one-sequence call), for near ties
    nqb, nkb = -(-max(nq) // Bq), -(-max(nk) // 64)
    keep = np.zeros((len(nq), Hq, nqb, nkb), bool)
    pruned = 0
    for b in range(len(nq)):
        q, k = Qd[cu_q[b]:cu_q[b + 1]][None], Kd[cu_k[b]:cu_k[b + 1]][None]
        qb = -(-nq[b] // Bq)
        mask = torch.zeros((1, Hq, qb, -(-(-(-nk[b] // 64)) // 64)), dtype=torch.int64,
                           device="cuda")
        _lib.bsfa_gate_masks(q, k, dtab, 0, mask, block_q=Bq)
        torch.cuda.synchronize()
        m = np.ascontiguousarray(mask.cpu().numpy()).view(np.uint8)
        bits = np.unpackbits(m, axis=-1, bitorder="little").astype(bool)
        for i in range(qb):
            n_off = oracle.key_block_range(i, nq[b], Bq, 64, nk[b] - nq[b])[0]
            keep[b, :, i, :n_off] = bits[0, :, i, :n_off]
            pruned += int((~bits[0, :, i, :n_off]).sum())
    assert pruned > 0
    r = oracle.oracle_prefill_varlen(Qh, Kh, Vh, cu_q, cu_k, block_q=Bq, block_k=64,
                                     mode="absolute", table=T, mean_correction=True,
                                     forced_keep=keep, band=BAND)
    err = np.abs(O.cpu().numpy() - r.out)
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (err.max(), err.mean())


@pytest.mark.parametrize("N,Bq", [(64, 64), (100, 64), (130, 128), (1, 64)])
def test_short_sequences(N, Bq):
    # at most one off-diagonal block: corrected and plain calls agree where nothing is pruned,
    # and the corrected one matches the oracle where the single block is pruned (T = +inf)
    Hq, Hkv, d = 2, 1, 64
    g = torch.Generator().manual_seed(36)
    Q, K, V = (torch.randn(1, N, h, d, generator=g) for h in (Hq, Hkv, Hkv))
    (Qd, Kd, Vd), (Qh, Kh, Vh) = bf16_pair(Q, K, V)
    T = np.full((1, Hq, 4), np.inf, np.float32)
    tab = make_table(T, Bq, d, [1])
    O = _lib.bsfa_prefill(Qd, Kd, Vd, block_q=Bq, gate_mode="absolute",
                          table=tab.to_device("cuda"), out_dtype=torch.float32,
                          mean_correction=True)
    torch.cuda.synchronize()
    r = oracle.oracle_prefill(Qh, Kh, Vh, block_q=Bq, block_k=64, mode="absolute", table=T,
                              mean_correction=True)
    err = np.abs(O.cpu().numpy() - r.out)
    assert np.isfinite(O.cpu().numpy()).all()
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (err.max(), err.mean())
