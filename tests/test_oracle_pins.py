"""Pins for the CPU oracle: each check ties it to something other than itself.

Sources: "Block Sparse Flash Attention" (paper notes), Method (Key Designs 1-3, A Worked
Example); "Skipping attention blocks was the easy part" (BLASST blog), "Vote, then skip".
References are torch's scaled_dot_product_attention (float64, CPU, explicit masks), brute-force
float64 block maxima from one full score matrix, values printed on the pages, and closed forms.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import (GATE_ABSOLUTE, GATE_DENSE, GATE_RELATIVE, calibrate, key_block_range,
                    kth_highest, oracle_prefill)
from pins_util import (block_mask_to_token_mask, brute_block_max, causal_mask,
                       diagonal_region_mask, first_offdiag_blocks, full_scores,
                       quantized_normal, sdpa_masked)


def _rand(seed, B, N, Hq, Hkv, d):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, N, Hq, d)).astype(np.float32),
            rng.standard_normal((B, N, Hkv, d)).astype(np.float32),
            rng.standard_normal((B, N, Hkv, d)).astype(np.float32))


def _const_table(value, Hq, t_len, n_budgets=1):
    return np.full((n_budgets, Hq, t_len), value, dtype=np.float32)


# ---------------------------------------------------------------------------------------------
# Block structure
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("N,Bq,Bk", [(384, 64, 64), (1000, 128, 64), (200, 64, 32), (300, 32, 64),
                                     (129, 128, 64), (1000, 128, 128)])
def test_block_ranges_match_brute_force(N, Bq, Bk):
    noff = first_offdiag_blocks(N, Bq, Bk)
    nqb = -(-N // Bq)
    for i in range(nqb):
        n_off, n_end = key_block_range(i, N, Bq, Bk)
        assert n_off == noff[i]
        last_row = min((i + 1) * Bq, N) - 1
        # n_end: one past the last key block holding a key <= the block's last row
        assert n_end == max(j for j in range(-(-N // Bk)) if j * Bk <= last_row) + 1


def test_block_ranges_named_tiles():
    # Bq = Bk: diagonal region is block i alone; Bq = 2 Bk: blocks 2i and 2i + 1
    assert [key_block_range(i, 1024, 64, 64) for i in (0, 5)] == [(0, 1), (5, 6)]
    assert [key_block_range(i, 1024, 128, 64) for i in (0, 3)] == [(0, 2), (6, 8)]


# ---------------------------------------------------------------------------------------------
# The worked example printed on the page
# ---------------------------------------------------------------------------------------------
def _worked_example_problem(maxima):
    """Embed the page's example: query block 5 sees 5 off-diagonal key blocks (Bq = Bk = 64,
    d = 64, scale 1/8). Query row 320 is 8 e0, the other rows of block 5 are zero; key block j
    holds one key with e0-component maxima[j] and zeros elsewhere, so the tile maxima are
    exactly the printed values."""
    N, d = 384, 64
    rng = np.random.default_rng(11)
    Q = np.zeros((1, N, 1, d), np.float32)
    K = np.zeros((1, N, 1, d), np.float32)
    V = rng.standard_normal((1, N, 1, d)).astype(np.float32)
    Q[0, 320, 0, 0] = 8.0
    for j, v in enumerate(maxima):
        K[0, 64 * j + 7, 0, 0] = v
    K[0, 320:, 0, :] = rng.standard_normal((64, d)).astype(np.float32) * 0.25
    return Q, K, V


def test_worked_example_from_page(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "worked_example.json")))
    maxima = ex["block_maxima"]
    Q, K, V = _worked_example_problem(maxima)
    table = _const_table(ex["threshold"], 1, 6)
    r = oracle_prefill(Q, K, V, block_q=64, block_k=64, mode=GATE_ABSOLUTE, table=table)
    np.testing.assert_array_equal(r.stat[0, 0, 5, :5], maxima)          # exact tile maxima
    kept = [maxima[j] for j in range(5) if r.keep[0, 0, 5, j]]
    skipped = [maxima[j] for j in range(5) if not r.keep[0, 0, 5, j]]
    assert sorted(kept) == sorted(ex["kept_maxima"])
    assert sorted(skipped) == sorted(ex["skipped_maxima"])
    assert r.kept_counts[0, 0, 5] == ex["kept_count"]
    assert r.keep[0, 0, 5, 5]                                            # diagonal extra
    # renormalisation over kept + diagonal, skipped blocks out of the denominator; the block
    # scoring 5 raises the running max after 4 was accumulated (rescale path)
    ref = sdpa_masked(Q, K, V, block_mask_to_token_mask(r.keep, 384, 64, 64), scale=0.125)
    np.testing.assert_allclose(r.out[0, 320:], ref[0, 320:], rtol=0, atol=2e-6)


@pytest.mark.parametrize("T,expected", [(4.0, 2), (3.5, 3), (-math.inf, 5), (math.inf, 0),
                                        (5.0, 1), (5.0000005, 0)])
def test_worked_example_threshold_edges(T, expected):
    # ">=" reading: a block whose max equals T is kept
    maxima = [1.0, 4.0, 2.0, 5.0, 3.5]
    Q, K, V = _worked_example_problem(maxima)
    r = oracle_prefill(Q, K, V, block_q=64, block_k=64, mode=GATE_ABSOLUTE,
                       table=_const_table(T, 1, 6))
    assert r.kept_counts[0, 0, 5] == expected


# ---------------------------------------------------------------------------------------------
# Special cases that reduce to library attention
# ---------------------------------------------------------------------------------------------
CASES = [  # B, N, Hq, Hkv, d, Bq, Bk
    (1, 256, 2, 1, 32, 64, 64),
    (2, 200, 4, 2, 16, 64, 32),     # batch, GQA, ragged tail
    (1, 300, 2, 2, 8, 128, 64),     # Bq = 2 Bk, ragged
    (1, 130, 2, 1, 16, 32, 64),     # Bq < Bk
    (1, 400, 2, 1, 16, 128, 128),   # the wide key tile, ragged
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("mode", ["dense", "abs_minus_inf", "rel_lambda0"])
def test_no_skip_equals_causal_attention(case, mode):
    B, N, Hq, Hkv, d, Bq, Bk = case
    Q, K, V = _rand(1, B, N, Hq, Hkv, d)
    kw = dict(block_q=Bq, block_k=Bk)
    if mode == "dense":
        r = oracle_prefill(Q, K, V, mode=GATE_DENSE, **kw)
    elif mode == "abs_minus_inf":
        r = oracle_prefill(Q, K, V, mode=GATE_ABSOLUTE, table=_const_table(-math.inf, Hq, 3), **kw)
    else:
        r = oracle_prefill(Q, K, V, mode=GATE_RELATIVE, log_lambda=-math.inf, **kw)
    ref = sdpa_masked(Q, K, V, causal_mask(B, Hq, N))
    np.testing.assert_allclose(r.out, ref, rtol=0, atol=3e-6)
    noff = first_offdiag_blocks(N, Bq, Bk)
    np.testing.assert_array_equal(r.kept_counts, np.broadcast_to(noff, r.kept_counts.shape))


@pytest.mark.parametrize("case", CASES)
def test_plus_inf_threshold_is_diagonal_only(case):
    B, N, Hq, Hkv, d, Bq, Bk = case
    Q, K, V = _rand(2, B, N, Hq, Hkv, d)
    r = oracle_prefill(Q, K, V, block_q=Bq, block_k=Bk, mode=GATE_ABSOLUTE,
                       table=_const_table(math.inf, Hq, 2))
    ref = sdpa_masked(Q, K, V, diagonal_region_mask(B, Hq, N, Bq, Bk))
    np.testing.assert_allclose(r.out, ref, rtol=0, atol=3e-6)
    assert (r.kept_counts == 0).all()


def test_float64_run_matches_library_tightly():
    Q, K, V = _rand(3, 1, 192, 2, 1, 16)
    r = oracle_prefill(Q, K, V, block_q=64, block_k=32, mode=GATE_DENSE, dtype=np.float64)
    ref = sdpa_masked(Q, K, V, causal_mask(1, 2, 192))
    np.testing.assert_allclose(r.out, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------------------------
# General thresholds: keep rule against brute force, aggregation against masked attention
# ---------------------------------------------------------------------------------------------
def _midpoint_table(bm, Hq, nqb, rng):
    """Per-(h, i) thresholds placed between two distinct brute-force block maxima, so the
    keep decision has no near-ties."""
    T = np.full((1, Hq, nqb), -np.inf, dtype=np.float32)
    for h in range(Hq):
        for i in range(nqb):
            v = np.unique(bm[:, h, i][~np.isnan(bm[:, h, i])])
            if len(v) >= 2:
                a = rng.integers(0, len(v) - 1)
                T[0, h, i] = np.float32(0.5 * (v[a] + v[a + 1]))
    return T


@pytest.mark.parametrize("case", CASES)
def test_keep_rule_and_renormalisation(case):
    B, N, Hq, Hkv, d, Bq, Bk = case
    Q, K, V = _rand(4, B, N, Hq, Hkv, d)
    bm = brute_block_max(Q, K, Bq, Bk)
    nqb = -(-N // Bq)
    T = _midpoint_table(bm[:1], Hq, nqb, np.random.default_rng(5))
    r = oracle_prefill(Q, K, V, block_q=Bq, block_k=Bk, mode=GATE_ABSOLUTE, table=T)
    noff = first_offdiag_blocks(N, Bq, Bk)
    exp_keep = np.zeros_like(r.keep)
    for i in range(nqb):
        exp_keep[:, :, i, :noff[i]] = bm[:, :, i, :noff[i]] >= T[0][None, :, i, None]
        n_end = key_block_range(i, N, Bq, Bk)[1]
        exp_keep[:, :, i, noff[i]:n_end] = True
        np.testing.assert_allclose(r.stat[:, :, i, :noff[i]], bm[:, :, i, :noff[i]],
                                   rtol=1e-6, atol=1e-6)
    np.testing.assert_array_equal(r.keep, exp_keep)
    np.testing.assert_array_equal(r.kept_counts, exp_keep[..., :].sum(-1) - np.array(
        [key_block_range(i, N, Bq, Bk)[1] - noff[i] for i in range(nqb)]))
    ref = sdpa_masked(Q, K, V, block_mask_to_token_mask(r.keep, N, Bq, Bk))
    np.testing.assert_allclose(r.out, ref, rtol=0, atol=3e-6)


def test_threshold_reuse_past_calibrated_length():
    B, N, Hq, Hkv, d, Bq, Bk = 1, 512, 2, 1, 16, 64, 32
    Q, K, V = _rand(6, B, N, Hq, Hkv, d)
    bm = brute_block_max(Q, K, Bq, Bk)
    t_len = 3
    rng = np.random.default_rng(7)
    T = np.empty((1, Hq, t_len), np.float32)
    for h in range(Hq):
        for c in range(t_len):
            T[0, h, c] = np.float32(rng.uniform(0.5, 2.5))
    T[0, :, 0] = -np.inf            # first and last calibrated columns far apart, so a wrong
    T[0, :, t_len - 1] = np.float32(np.nanmedian(bm))   # column choice past T_len matters
    r = oracle_prefill(Q, K, V, block_q=Bq, block_k=Bk, mode=GATE_ABSOLUTE, table=T)
    noff = first_offdiag_blocks(N, Bq, Bk)
    for h in range(Hq):
        for i in range(N // Bq):
            thr = T[0, h, min(i, t_len - 1)]
            assert r.kept_counts[0, h, i] == int((bm[0, h, i, :noff[i]] >= thr).sum())
    assert (r.kept_counts[0, :, t_len:] < np.array(noff[t_len:])[None, :]).any()


def test_budget_slice_selects_table_slice():
    Q, K, V = _rand(8, 1, 256, 1, 1, 16)
    T = np.stack([np.full((1, 4), -np.inf), np.full((1, 4), np.inf)]).astype(np.float32)
    r0 = oracle_prefill(Q, K, V, block_q=64, block_k=64, mode=GATE_ABSOLUTE, table=T,
                        budget_slice=0)
    r1 = oracle_prefill(Q, K, V, block_q=64, block_k=64, mode=GATE_ABSOLUTE, table=T,
                        budget_slice=1)
    assert list(r0.kept_counts[0, 0]) == [0, 1, 2, 3]
    assert list(r1.kept_counts[0, 0]) == [0, 0, 0, 0]


def test_skipped_values_never_read():
    # a rejected block loads no V: poisoning the V rows of skipped blocks changes nothing
    B, N, Hq, Hkv, d, Bq, Bk = 1, 256, 1, 1, 16, 64, 32
    Q, K, V = _rand(9, B, N, Hq, Hkv, d)
    bm = brute_block_max(Q, K, Bq, Bk)
    T = _midpoint_table(bm, Hq, N // Bq, np.random.default_rng(3))
    r = oracle_prefill(Q, K, V, block_q=Bq, block_k=Bk, mode=GATE_ABSOLUTE, table=T)
    # poison the V rows of every block the last query block skips; its output must not change
    i = N // Bq - 1
    Vp = V.copy()
    n_poisoned = 0
    for j in range(first_offdiag_blocks(N, Bq, Bk)[i]):
        if not r.keep[0, 0, i, j]:
            Vp[0, j * Bk:(j + 1) * Bk] = np.nan
            n_poisoned += 1
    assert n_poisoned > 0
    r2 = oracle_prefill(Q, K, Vp, block_q=Bq, block_k=Bk, mode=GATE_ABSOLUTE, table=T,
                        query_blocks=[i])
    np.testing.assert_array_equal(r.out[0, i * Bq:], r2.out[0, i * Bq:])
    np.testing.assert_array_equal(r.kept_counts[0, 0, i], r2.kept_counts[0, 0, i])


def test_gqa_equals_repeated_kv():
    Q, K, V = _rand(10, 1, 256, 4, 2, 16)
    T = _const_table(1.0, 4, 4)
    a = oracle_prefill(Q, K, V, block_q=64, block_k=32, mode=GATE_ABSOLUTE, table=T)
    b = oracle_prefill(Q, np.repeat(K, 2, axis=2), np.repeat(V, 2, axis=2), block_q=64,
                       block_k=32, mode=GATE_ABSOLUTE, table=T)
    np.testing.assert_array_equal(a.out, b.out)
    np.testing.assert_array_equal(a.kept_counts, b.kept_counts)


def test_forced_keep_applies_inside_band_only():
    Q, K, V = _rand(12, 1, 256, 1, 1, 16)
    bm = brute_block_max(Q, K, 64, 32)
    T = np.full((1, 1, 4), np.float32(bm[0, 0, 3, 2]), dtype=np.float32)   # exact tie at (3, 2)
    base = oracle_prefill(Q, K, V, block_q=64, block_k=32, mode=GATE_ABSOLUTE, table=T)
    forced = ~base.keep
    r = oracle_prefill(Q, K, V, block_q=64, block_k=32, mode=GATE_ABSOLUTE, table=T,
                       forced_keep=forced, band=1e-2)
    inband = np.abs(base.margin) <= 1e-2
    np.testing.assert_array_equal(r.keep[inband], forced[inband])
    outband = ~inband & ~np.isnan(base.margin)
    np.testing.assert_array_equal(r.keep[outband], base.keep[outband])


# ---------------------------------------------------------------------------------------------
# Relative gate
# ---------------------------------------------------------------------------------------------
def _relative_hand_case():
    """Query block 2 (Bq = Bk = 64, d = 16, scale 1/4): off-diagonal block 0 scores 0 for every
    pair, block 1 scores -10 for every pair."""
    N, d = 192, 16
    Q = np.zeros((1, N, 1, d), np.float32)
    K = np.zeros((1, N, 1, d), np.float32)
    V = np.random.default_rng(0).standard_normal((1, N, 1, d)).astype(np.float32)
    Q[0, 128:, 0, 0] = 4.0
    K[0, 64:128, 0, 0] = -10.0          # (4 * -10) / 4 = -10
    K[0, 128:, 0, 0] = 0.0
    return Q, K, V


@pytest.mark.parametrize("lam,kept_block1", [(1e-3, False), (1e-5, True), (0.0, True)])
def test_relative_gate_hand_case(lam, kept_block1):
    Q, K, V = _relative_hand_case()
    ll = math.log(lam) if lam > 0 else -math.inf
    r = oracle_prefill(Q, K, V, block_q=64, block_k=64, mode=GATE_RELATIVE, log_lambda=ll,
                       scale=0.25)
    assert r.keep[0, 0, 2, 0]                         # first block: running max is -inf
    assert r.keep[0, 0, 2, 1] == kept_block1
    assert r.stat[0, 0, 2, 1] == -10.0


@pytest.mark.parametrize("lam", [1e-4, 1e-3, 1e-2, 1e-1])
def test_relative_gate_bound_on_dense_weights(lam):
    # every dense softmax weight inside a skipped block is below lambda
    B, N, Hq, Hkv, d, Bq, Bk = 1, 512, 2, 1, 16, 64, 32
    Q, K, V = _rand(13, B, N, Hq, Hkv, d)
    Q *= 6.0
    for j in range(1, N // Bk, 2):
        K[:, j * Bk:(j + 1) * Bk] *= 0.05          # weak key blocks that the gate can drop
    r = oracle_prefill(Q, K, V, block_q=Bq, block_k=Bk, mode=GATE_RELATIVE,
                       log_lambda=math.log(lam))
    S = full_scores(Q, K)
    S = np.where(np.tril(np.ones((N, N), bool)), S, -np.inf)
    P = np.exp(S - S.max(-1, keepdims=True))
    P /= P.sum(-1, keepdims=True)
    n_skipped = 0
    for h in range(Hq):
        for i in range(N // Bq):
            for j in range(first_offdiag_blocks(N, Bq, Bk)[i]):
                if not r.keep[0, h, i, j]:
                    n_skipped += 1
                    assert P[0, h, i * Bq:(i + 1) * Bq, j * Bk:(j + 1) * Bk].max() < lam * (1 + 1e-5)
    assert n_skipped > 0
    ref = sdpa_masked(Q, K, V, block_mask_to_token_mask(r.keep, N, Bq, Bk))
    np.testing.assert_allclose(r.out, ref, rtol=0, atol=3e-6)


# ---------------------------------------------------------------------------------------------
# Calibration
# ---------------------------------------------------------------------------------------------
def test_kth_highest_hand_values():
    m = np.array([5.0, 3.0, 3.0, 1.0, 9.0])
    assert kth_highest(m, 4, 1) == 5.0
    assert kth_highest(m, 4, 2) == 3.0
    assert kth_highest(m, 4, 3) == 3.0
    assert kth_highest(m, 4, 4) == 1.0          # n_off == k: the smallest candidate, not -inf
    assert kth_highest(m, 4, 5) == -math.inf    # fewer than k candidates
    assert kth_highest(m, 5, 1) == 9.0


def _exact_sample(seed, N=512, Hq=2, Hkv=1, d=32):
    rng = np.random.default_rng(seed)
    return (quantized_normal(rng, (1, N, Hq, d)), quantized_normal(rng, (1, N, Hkv, d)),
            rng.standard_normal((1, N, Hkv, d)).astype(np.float32))


@pytest.mark.parametrize("k", [1, 3, 6])
def test_calibrate_on_one_sample_keeps_exactly_k(k):
    Bq, Bk, N = 64, 32, 512
    Q, K, V = _exact_sample(21)
    bm = brute_block_max(Q, K, Bq, Bk, scale=0.125)
    T = calibrate([(Q, K)], block_q=Bq, block_k=Bk, budgets=[k], scale=0.125)
    r = oracle_prefill(Q, K, V, block_q=Bq, block_k=Bk, mode=GATE_ABSOLUTE, table=T, scale=0.125)
    noff = first_offdiag_blocks(N, Bq, Bk)
    for h in range(2):
        for i in range(N // Bq):
            vals = bm[0, h, i, :noff[i]]
            assert len(np.unique(vals)) == len(vals)          # premise: distinct maxima
            if noff[i] >= k:
                assert r.kept_counts[0, h, i] == k
                assert T[0, h, i] == np.sort(vals)[::-1][k - 1]
            else:
                assert T[0, h, i] == -np.inf
                assert r.kept_counts[0, h, i] == noff[i]


def test_calibrate_averages_samples():
    Bq, Bk, N, k = 64, 32, 512, 2
    s1, s2 = _exact_sample(31), _exact_sample(32)
    T = calibrate([s1[:2], s2[:2]], block_q=Bq, block_k=Bk, budgets=[k, 5], scale=0.125)
    noff = first_offdiag_blocks(N, Bq, Bk)
    b1 = brute_block_max(s1[0], s1[1], Bq, Bk, scale=0.125)
    b2 = brute_block_max(s2[0], s2[1], Bq, Bk, scale=0.125)
    for kk, kv in enumerate([k, 5]):
        for h in range(2):
            for i in range(N // Bq):
                if noff[i] < kv:
                    assert T[kk, h, i] == -np.inf
                    continue
                t1 = np.sort(b1[0, h, i, :noff[i]])[::-1][kv - 1]
                t2 = np.sort(b2[0, h, i, :noff[i]])[::-1][kv - 1]
                assert T[kk, h, i] == np.float32(0.5 * (t1 + t2))


def test_calibrate_batch_entries_are_samples():
    s1, s2 = _exact_sample(41), _exact_sample(42)
    Qb = np.concatenate([s1[0], s2[0]])
    Kb = np.concatenate([s1[1], s2[1]])
    a = calibrate([(Qb, Kb)], block_q=64, block_k=32, budgets=[3], scale=0.125)
    b = calibrate([s1[:2], s2[:2]], block_q=64, block_k=32, budgets=[3], scale=0.125)
    np.testing.assert_array_equal(a, b)


def test_predicted_density_closed_form():
    # sum_i min(n_off(i), k) / sum_i n_off(i) for Bq = 2 Bk: n_off(i) = 2 i
    for nqb, k in [(128, 32), (256, 16), (256, 64), (256, 256), (1024, 64)]:
        noff = [key_block_range(i, nqb * 128, 128, 64)[0] for i in range(nqb)]
        num = sum(min(x, k) for x in noff)
        den = sum(noff)
        # closed form: 2 * sum_{i < k/2} i + k * (#i >= k/2) over the triangle sum nqb (nqb - 1)
        h = min(k // 2, nqb)
        closed = (h * (h - 1) + k * (nqb - h)) / (nqb * (nqb - 1))
        assert abs(num / den - closed) < 1e-12


def test_oracle_module_header_marks_test_infrastructure():
    doc = oracle.bsfa_oracle.__doc__
    assert "TEST INFRASTRUCTURE ONLY" in doc


# ---------------------------------------------------------------------------------------------
# Chunked prefill: a chunk of query rows after a prefix of keys
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("Nq,P,Bq,Bk", [(256, 128, 64, 64), (300, 256, 128, 64), (200, 70, 64, 64),
                                        (129, 1, 128, 64), (64, 1000, 64, 32)])
def test_block_ranges_with_prefix_match_brute_force(Nq, P, Bq, Bk):
    Nk = Nq + P
    nkb = -(-Nk // Bk)
    for i in range(-(-Nq // Bq)):
        n_off, n_end = key_block_range(i, Nq, Bq, Bk, P)
        first, last = P + i * Bq, P + min((i + 1) * Bq, Nq) - 1     # absolute rows
        # blocks whose every key precedes the first row, and blocks holding a visible key
        assert n_off == sum(1 for j in range(nkb) if min((j + 1) * Bk, Nk) - 1 < first)
        assert n_end == sum(1 for j in range(nkb) if j * Bk <= last)


@pytest.mark.parametrize("B,Nq,P,Hq,Hkv,d,Bq,Bk", [(1, 200, 128, 2, 1, 16, 64, 64),
                                                   (2, 130, 70, 4, 2, 8, 128, 64),
                                                   (1, 64, 333, 2, 2, 16, 64, 32)])
def test_prefix_dense_equals_masked_attention(B, Nq, P, Hq, Hkv, d, Bq, Bk):
    # any prefix (aligned to the tiles or not): row r of the chunk sees keys 0 .. P + r
    rng = np.random.default_rng(31)
    Q = rng.standard_normal((B, Nq, Hq, d)).astype(np.float32)
    K = rng.standard_normal((B, Nq + P, Hkv, d)).astype(np.float32)
    V = rng.standard_normal((B, Nq + P, Hkv, d)).astype(np.float32)
    r = oracle_prefill(Q, K, V, block_q=Bq, block_k=Bk, mode=GATE_DENSE)
    mask = np.arange(Nq + P)[None, :] <= (P + np.arange(Nq))[:, None]
    ref = sdpa_masked(Q, K, V, np.broadcast_to(mask, (B, Hq, Nq, Nq + P)).copy())
    np.testing.assert_allclose(r.out, ref, rtol=0, atol=3e-6)
    for i in range(-(-Nq // Bq)):
        assert (r.kept_counts[:, :, i] == key_block_range(i, Nq, Bq, Bk, P)[0]).all()


@pytest.mark.parametrize("mode", ["dense", "absolute", "relative"])
@pytest.mark.parametrize("P", [128, 256])
def test_chunk_equals_rows_of_full_prefill(mode, P):
    # with the prefix on the query-block grid, every query block of the chunk sees the same
    # keys, thresholds and traversal as the same block of the whole prefill: identical results
    B, N, Hq, Hkv, d, Bq, Bk = 1, 512, 4, 2, 16, 64, 64
    Q, K, V = _rand(32, B, N, Hq, Hkv, d)
    Q = Q * 2.0
    nqb = N // Bq
    kw = dict(block_q=Bq, block_k=Bk, mode=mode)
    if mode == "absolute":
        rng = np.random.default_rng(5)
        kw["table"] = _midpoint_table(brute_block_max(Q, K, Bq, Bk), Hq, nqb, rng)
    elif mode == "relative":
        # keys after the first block weaker, so that later blocks trail the running max
        K = K.copy()
        K[:, 64:] *= 0.3
        kw["log_lambda"] = math.log(0.3)
    full = oracle_prefill(Q, K, V, **kw)
    chunk = oracle_prefill(Q[:, P:], K, V, **kw)
    i0 = P // Bq
    np.testing.assert_array_equal(chunk.out, full.out[:, P:])
    np.testing.assert_array_equal(chunk.kept_counts, full.kept_counts[:, :, i0:])
    np.testing.assert_array_equal(chunk.keep, full.keep[:, :, i0:])
    np.testing.assert_array_equal(np.isnan(chunk.stat), np.isnan(full.stat[:, :, i0:]))
    fin = ~np.isnan(chunk.stat)
    np.testing.assert_array_equal(chunk.stat[fin], full.stat[:, :, i0:][fin])
    if mode != "dense":
        assert 0 < chunk.kept_counts.sum() < sum(key_block_range(i, N - P, Bq, Bk, P)[0]
                                                 for i in range(nqb - i0)) * B * Hq


def test_absolute_gate_rejects_prefix_off_the_block_grid():
    Q, K, V = _rand(33, 1, 192, 1, 1, 8)
    with pytest.raises(ValueError):
        oracle_prefill(Q[:, 100:], K, V, block_q=64, block_k=64, mode=GATE_ABSOLUTE,
                       table=_const_table(0.0, 1, 3))


# ---------------------------------------------------------------------------------------------
# Variable-length batches (sequences packed along the token axis)
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("mode", ["dense", "absolute", "relative"])
def test_varlen_of_equal_sequences_equals_the_batch(mode):
    # packing a batch of equal-length sequences changes nothing
    B, N, Hq, Hkv, d, Bq, Bk = 3, 192, 2, 1, 16, 64, 64
    Q, K, V = _rand(34, B, N, Hq, Hkv, d)
    kw = dict(block_q=Bq, block_k=Bk, mode=mode)
    if mode == "absolute":
        kw["table"] = _midpoint_table(brute_block_max(Q, K, Bq, Bk), Hq, N // Bq,
                                      np.random.default_rng(6))
    elif mode == "relative":
        kw["log_lambda"] = math.log(0.3)
    batch = oracle_prefill(Q, K, V, **kw)
    cu = [0, N, 2 * N, 3 * N]
    var = oracle.oracle_prefill_varlen(Q.reshape(B * N, Hq, d), K.reshape(B * N, Hkv, d),
                                       V.reshape(B * N, Hkv, d), cu, cu, **kw)
    np.testing.assert_array_equal(var.out, batch.out.reshape(B * N, Hq, d))
    np.testing.assert_array_equal(var.kept_counts, batch.kept_counts)
    np.testing.assert_array_equal(var.keep, batch.keep)


def test_varlen_mixed_lengths_and_prefixes():
    # sequences of different lengths, one with a prefix, one empty: each equals its own call,
    # and the padding past each sequence's blocks stays unwritten
    rng = np.random.default_rng(35)
    Hq, Hkv, d, Bq, Bk = 2, 1, 8, 64, 64
    nq, nk = [100, 0, 256, 64], [100, 0, 384, 64]
    cu_q, cu_k = np.cumsum([0] + nq), np.cumsum([0] + nk)
    Q = rng.standard_normal((cu_q[-1], Hq, d)).astype(np.float32)
    K = rng.standard_normal((cu_k[-1], Hkv, d)).astype(np.float32)
    V = rng.standard_normal((cu_k[-1], Hkv, d)).astype(np.float32)
    r = oracle.oracle_prefill_varlen(Q, K, V, cu_q, cu_k, block_q=Bq, block_k=Bk, mode="dense")
    for b in range(4):
        if nq[b] == 0:
            assert (r.kept_counts[b] == -1).all()
            continue
        one = oracle_prefill(Q[None, cu_q[b]:cu_q[b + 1]], K[None, cu_k[b]:cu_k[b + 1]],
                             V[None, cu_k[b]:cu_k[b + 1]], block_q=Bq, block_k=Bk, mode="dense")
        np.testing.assert_array_equal(r.out[cu_q[b]:cu_q[b + 1]], one.out[0])
        qb = one.kept_counts.shape[2]
        np.testing.assert_array_equal(r.kept_counts[b, :, :qb], one.kept_counts[0])
        assert (r.kept_counts[b, :, qb:] == -1).all()
    # and the prefixed sequence is plain masked attention over its keys
    b = 2
    mask = np.arange(nk[b])[None, :] <= (nk[b] - nq[b] + np.arange(nq[b]))[:, None]
    ref = sdpa_masked(Q[None, cu_q[b]:cu_q[b + 1]], K[None, cu_k[b]:cu_k[b + 1]],
                      V[None, cu_k[b]:cu_k[b + 1]], np.broadcast_to(mask, (1, Hq) + mask.shape).copy())
    np.testing.assert_allclose(r.out[None, cu_q[b]:cu_q[b + 1]], ref, rtol=0, atol=3e-6)


def test_gather_pages_inverts_a_paged_layout():
    # scatter packed sequences into shuffled pages by hand, then gather them back
    rng = np.random.default_rng(36)
    page, H, d = 64, 2, 4
    lens = [130, 0, 64, 257]
    K = rng.standard_normal((sum(lens), H, d)).astype(np.float32)
    n_pages = [-(-n // page) for n in lens]
    free = list(rng.permutation(sum(n_pages) + 3))        # pool with unused pages
    pool = np.full((len(free), page, H, d), np.nan, np.float32)
    table = np.zeros((len(lens), max(n_pages)), np.int32)
    off = 0
    for b, n in enumerate(lens):
        for j in range(n_pages[b]):
            pg = free.pop()
            table[b, j] = pg
            m = min(page, n - j * page)
            pool[pg, :m] = K[off + j * page: off + j * page + m]
        off += n
    G, cu = oracle.gather_pages(pool, table, lens)
    np.testing.assert_array_equal(cu, np.cumsum([0] + lens))
    np.testing.assert_array_equal(G, K)


# ---------------------------------------------------------------------------------------------
# Mean correction ("FlashPrefill V2: Block-Sparse Prefill Attention for Long-Context LLM
# Serving", mean correction): a pruned block contributes |B| e^{s(q, kbar)} vbar to the
# numerator and |B| e^{s(q, kbar)} to the denominator.
# ---------------------------------------------------------------------------------------------
def _block_constant_keys(K, Bk, rng, noise=0.0):
    """K with every key of a block of Bk keys equal to one random key (plus noise * N(0, 1))."""
    K = K.copy()
    Nk = K.shape[1]
    for j0 in range(0, Nk, Bk):
        K[:, j0:j0 + Bk] = K[:, j0:j0 + 1]
    if noise:
        K = (K + noise * rng.standard_normal(K.shape)).astype(K.dtype)
    return K


MEAN_CASES = [   # B, Nq, P, Hq, Hkv, d, Bq, Bk
    (1, 256, 0, 2, 1, 32, 64, 64),
    (2, 300, 0, 4, 2, 16, 128, 64),     # batch, GQA, ragged tail
    (1, 200, 128, 2, 1, 16, 64, 32),    # a prefix before the chunk
    (1, 400, 0, 2, 1, 16, 128, 128),    # the wide key block
]


@pytest.mark.parametrize("case", MEAN_CASES)
@pytest.mark.parametrize("table", ["plus_inf", "midpoint"])
def test_mean_correction_is_exact_for_block_constant_keys(case, table):
    # Keys equal within each block: sum_j e^{s_j} v_j = |B| e^{s(q, k)} vbar exactly, so the
    # corrected output equals full causal attention whatever is pruned.
    B, Nq, P, Hq, Hkv, d, Bq, Bk = case
    rng = np.random.default_rng(11)
    Q = rng.standard_normal((B, Nq, Hq, d)).astype(np.float32)
    K = _block_constant_keys(rng.standard_normal((B, P + Nq, Hkv, d)).astype(np.float32), Bk, rng)
    V = rng.standard_normal((B, P + Nq, Hkv, d)).astype(np.float32)
    nqb = -(-Nq // Bq)
    t_len = P // Bq + nqb
    ref = oracle_prefill(Q, K, V, block_q=Bq, block_k=Bk, mode=GATE_DENSE, dtype=np.float64)
    n_off = np.array([key_block_range(i, Nq, Bq, Bk, P)[0] for i in range(nqb)])
    if table == "plus_inf":
        T = _const_table(math.inf, Hq, t_len)
    else:   # the median off-diagonal block maximum: about half the blocks pruned
        off = np.arange(ref.stat.shape[3])[None, :] < n_off[:, None]
        T = _const_table(np.median(ref.stat[:, :, off]), Hq, t_len)
    kw = dict(block_q=Bq, block_k=Bk, mode=GATE_ABSOLUTE, table=T, dtype=np.float64)
    r = oracle_prefill(Q, K, V, mean_correction=True, **kw)
    plain = oracle_prefill(Q, K, V, **kw)
    assert (plain.kept_counts < n_off).any()    # something was pruned
    np.testing.assert_allclose(ref.out, sdpa_masked_prefix(Q, K, V, P), rtol=0, atol=1e-10)
    np.testing.assert_allclose(r.out, ref.out, rtol=0, atol=1e-10)
    assert np.abs(plain.out - ref.out).max() > 1e-3    # the correction is what closes the gap
    np.testing.assert_array_equal(r.keep, plain.keep)   # it never changes a decision


def sdpa_masked_prefix(Q, K, V, P):
    """Causal attention of Nq query rows at absolute positions P .. P + Nq - 1 (float64)."""
    B, Nq, Hq, d = Q.shape
    Nk = K.shape[1]
    rows = P + np.arange(Nq)[:, None]
    mask = np.broadcast_to(np.arange(Nk)[None, :] <= rows, (B, Hq, Nq, Nk))
    return sdpa_masked(Q, K, V, mask)


@pytest.mark.parametrize("case", MEAN_CASES)
def test_mean_correction_closed_form(case):
    # Written as one sum per row over the kept keys and the pruned blocks' stand-ins (no online
    # softmax): numerator sum e^{s} v + sum_J |B_J| e^{sbar_J} vbar_J, denominator likewise.
    B, Nq, P, Hq, Hkv, d, Bq, Bk = case
    rng = np.random.default_rng(12)
    Q = rng.standard_normal((B, Nq, Hq, d))
    K = rng.standard_normal((B, P + Nq, Hkv, d))
    V = rng.standard_normal((B, P + Nq, Hkv, d))
    Nk = P + Nq
    sc = 1.0 / math.sqrt(d)
    nqb = -(-Nq // Bq)
    t_len = P // Bq + nqb
    n_off = np.array([key_block_range(i, Nq, Bq, Bk, P)[0] for i in range(nqb)])
    dense = oracle_prefill(Q, K, V, block_q=Bq, block_k=Bk, mode=GATE_DENSE, dtype=np.float64)
    med = np.median(dense.stat[:, :, np.arange(dense.stat.shape[3])[None, :] < n_off[:, None]])
    T = (med + 0.3 * rng.standard_normal((1, Hq, t_len))).astype(np.float32)
    r = oracle_prefill(Q, K, V, block_q=Bq, block_k=Bk, mode=GATE_ABSOLUTE, table=T,
                       mean_correction=True, dtype=np.float64)
    assert (r.kept_counts < n_off).any() and (r.kept_counts > 0).any()
    G = Hq // Hkv
    out = np.empty_like(Q)
    for b in range(B):
        for h in range(Hq):
            k, v = K[b, :, h // G], V[b, :, h // G]
            for row in range(Nq):
                i, arow = row // Bq, P + row
                n_off = (P + i * Bq) // Bk
                logits, vals = [], []
                for j in range(-(-Nk // Bk)):
                    c0, c1 = j * Bk, min((j + 1) * Bk, Nk)
                    if j >= n_off or r.keep[b, h, i, j]:
                        cols = np.arange(c0, min(c1, arow + 1))
                        logits += list(sc * (k[cols] @ Q[b, row, h]))
                        vals += list(v[cols])
                    else:
                        logits.append(math.log(c1 - c0) + sc * (k[c0:c1].mean(0) @ Q[b, row, h]))
                        vals.append(v[c0:c1].mean(0))
                w = np.exp(np.array(logits) - max(logits))
                out[b, row, h] = (w[:, None] * np.array(vals)).sum(0) / w.sum()
    np.testing.assert_allclose(r.out, out, rtol=0, atol=1e-12)


def test_mean_correction_error_vanishes_with_within_block_spread():
    # Keys = block constant + eps * noise: the stand-in's error is first order in eps (the
    # within-block covariance of e^{s} and v), the uncorrected output's is not small at all.
    B, N, Hq, Hkv, d, Bq, Bk = 1, 512, 2, 1, 32, 64, 64
    rng = np.random.default_rng(13)
    Q = rng.standard_normal((B, N, Hq, d))
    K0 = rng.standard_normal((B, N, Hkv, d))
    V = rng.standard_normal((B, N, Hkv, d))
    T = _const_table(math.inf, Hq, N // Bq)
    errs = []
    for eps in (1e-2, 1e-3):
        K = _block_constant_keys(K0, Bk, np.random.default_rng(14), noise=eps)
        dense = oracle_prefill(Q, K, V, block_q=Bq, block_k=Bk, mode=GATE_DENSE, dtype=np.float64)
        kw = dict(block_q=Bq, block_k=Bk, mode=GATE_ABSOLUTE, table=T, dtype=np.float64)
        corr = oracle_prefill(Q, K, V, mean_correction=True, **kw)
        plain = oracle_prefill(Q, K, V, **kw)
        errs.append((np.abs(corr.out - dense.out).max(), np.abs(plain.out - dense.out).max()))
    (c1, p1), (c2, p2) = errs
    assert c1 < 0.05 * p1 and c2 < 0.2 * c1 and p2 > 0.5 * p1


@pytest.mark.parametrize("mode", ["dense", "abs_minus_inf"])
def test_mean_correction_changes_nothing_when_nothing_is_pruned(mode):
    Q, K, V = _rand(15, 1, 300, 2, 1, 16)
    kw = dict(block_q=64, block_k=64)
    if mode == "dense":
        kw["mode"] = GATE_DENSE
    else:
        kw.update(mode=GATE_ABSOLUTE, table=_const_table(-math.inf, 2, 5))
    a = oracle_prefill(Q, K, V, mean_correction=True, **kw)
    b = oracle_prefill(Q, K, V, **kw)
    np.testing.assert_array_equal(a.out, b.out)


def test_mean_correction_refuses_the_relative_gate():
    Q, K, V = _rand(16, 1, 128, 1, 1, 16)
    with pytest.raises(ValueError):
        oracle_prefill(Q, K, V, block_q=64, block_k=64, mode=GATE_RELATIVE, log_lambda=-1.0,
                       mean_correction=True)


# ---------------------------------------------------------------------------------------------
# FP8 (E4M3) gate scores
# ---------------------------------------------------------------------------------------------
def _e4m3_positive_grid():
    """Every finite positive E4M3 value from the format's definition: subnormals m 2^-9
    (m = 1..7) and normals 2^e (1 + m/8), e = -6..8, without the top code (e = 8, m = 7)."""
    vals = [m * 2.0 ** -9 for m in range(1, 8)]
    vals += [2.0 ** e * (1 + m / 8) for e in range(-6, 9) for m in range(8)
             if not (e == 8 and m == 7)]
    return np.array(sorted(vals))


def test_e4m3_grid_fixed_points_and_ties_to_even():
    grid = _e4m3_positive_grid()
    assert len(grid) == 126 and grid[-1] == 448.0
    full = np.concatenate([-grid[::-1], [0.0], grid])
    np.testing.assert_array_equal(oracle.quantize_e4m3(full), full.astype(np.float32))
    # a midpoint goes to the neighbour whose last mantissa bit is 0
    mids = 0.5 * (grid[:-1] + grid[1:])
    got = oracle.quantize_e4m3(mids)
    k = np.arange(len(mids))
    even_lo = (k % 2 == 0)          # grid[k] has an even code when k is even (k = code - 1)
    # code of grid[k] is k + 1: even code when k is odd
    want = np.where((k + 1) % 2 == 0, grid[:-1], grid[1:])
    np.testing.assert_array_equal(got, want.astype(np.float32))
    assert even_lo.any()
    # just off the midpoint: plain nearest
    np.testing.assert_array_equal(oracle.quantize_e4m3(mids * (1 + 1e-6)), grid[1:].astype(np.float32))
    np.testing.assert_array_equal(oracle.quantize_e4m3(mids * (1 - 1e-6)), grid[:-1].astype(np.float32))


def test_e4m3_matches_torch_float8_conversion():
    rng = np.random.default_rng(40)
    x = np.concatenate([rng.uniform(-448, 448, 100000),
                        rng.standard_normal(100000) * 0.01,
                        np.linspace(-2.0 ** -5, 2.0 ** -5, 20001)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).float().numpy()
    np.testing.assert_array_equal(oracle.quantize_e4m3(x), ref)


def test_q_rows_and_k_tiles_quantisation():
    rng = np.random.default_rng(41)
    Q = rng.standard_normal((2, 70, 3, 32)).astype(np.float32)
    Q[1, 5, 2] = 0.0                                     # an all-zero row
    K = rng.standard_normal((2, 150, 2, 32)).astype(np.float32)
    K[0, 64:128, 1] = 0.0                                # an all-zero tile of one head
    for X, (codes, scale), axes in ((Q, oracle.quantize_q_rows(Q), None),
                                    (K, oracle.quantize_k_tiles(K), "tiles")):
        assert np.abs(codes).max() <= 448
        if axes is None:
            amax = np.abs(X).max(-1)
            deq = codes * scale[..., None]
            # the largest element of each nonzero row becomes +-448 exactly
            nz = amax > 0
            np.testing.assert_array_equal(np.abs(codes).max(-1)[nz], 448.0)
            np.testing.assert_array_equal(scale, np.where(nz, amax / np.float32(448), 0))
            assert (codes[~nz] == 0).all()
        else:
            nt = -(-X.shape[1] // 64)
            assert scale.shape == (2, nt, 2)
            for t in range(nt):
                blk = np.abs(X[:, t * 64:(t + 1) * 64]).max(axis=(1, 3))
                np.testing.assert_array_equal(scale[:, t], blk / np.float32(448))
            deq = codes * np.repeat(scale, 64, axis=1)[:, :X.shape[1], :, None]
            assert (codes[0, 64:128, 1] == 0).all() and scale[0, 1, 1] == 0
        # relative error 2^-4 for values in E4M3's normal range, absolute 2^-10 * scale below
        s_b = scale[..., None] if axes is None else np.repeat(scale, 64, axis=1)[:, :X.shape[1], :, None]
        bound = np.maximum(np.abs(X) * 2.0 ** -4, 2.0 ** -10 * s_b) * (1 + 1e-6)
        assert (np.abs(deq - X) <= bound).all()


def _representable_inputs(rng, B, N, Hq, Hkv, d):
    """Q rows and K tiles whose FP8 copies are exact: E4M3 values times a power of two, with one
    element of each row / tile at +-448 times that power (so amax / 448 is the power)."""
    grid = _e4m3_positive_grid()
    def draw(shape):
        v = rng.choice(grid[40:], size=shape) * rng.choice([-1.0, 1.0], size=shape)
        return v.astype(np.float32)
    Q = draw((B, N, Hq, d))
    Q[..., 0] = 448.0
    Q *= (2.0 ** rng.integers(-9, -5, size=(B, N, Hq, 1))).astype(np.float32)
    K = draw((B, N, Hkv, d))
    for t in range(-(-N // 64)):
        K[:, t * 64, :, 0] = -448.0
        K[:, t * 64:(t + 1) * 64] *= (2.0 ** rng.integers(-9, -5, size=(B, 1, Hkv, 1))).astype(np.float32)
    return Q, K


def test_fp8_gate_equals_exact_gate_on_representable_inputs():
    rng = np.random.default_rng(42)
    B, N, Hq, Hkv, d, Bq, Bk = 1, 520, 4, 2, 32, 128, 64
    Q, K = _representable_inputs(rng, B, N, Hq, Hkv, d)
    V = rng.standard_normal((B, N, Hkv, d)).astype(np.float32)
    q8, qs = oracle.quantize_q_rows(Q)
    np.testing.assert_array_equal(q8 * qs[..., None], Q)
    k8, ks = oracle.quantize_k_tiles(K)
    np.testing.assert_array_equal(k8 * np.repeat(ks, 64, axis=1)[:, :N, :, None], K)
    bm = brute_block_max(Q, K, Bq, Bk)
    T = _midpoint_table(bm, Hq, -(-N // Bq), np.random.default_rng(43))
    kw = dict(block_q=Bq, block_k=Bk, mode=GATE_ABSOLUTE, table=T, dtype=np.float64)
    a = oracle_prefill(Q, K, V, gate_dtype="fp8", **kw)
    b = oracle_prefill(Q, K, V, **kw)
    np.testing.assert_array_equal(a.keep, b.keep)
    np.testing.assert_allclose(a.stat, b.stat, rtol=1e-12, atol=0)
    np.testing.assert_array_equal(a.out, b.out)


@pytest.mark.parametrize("Bk", [64, 128])
def test_fp8_block_maxima_brute_force(Bk):
    # one full score matrix of the dequantised copies, then block maxima
    rng = np.random.default_rng(44)
    B, N, Hq, Hkv, d, Bq = 1, 600, 4, 2, 32, 128
    Q = rng.standard_normal((B, N, Hq, d)).astype(np.float32)
    K = rng.standard_normal((B, N, Hkv, d)).astype(np.float32)
    V = rng.standard_normal((B, N, Hkv, d)).astype(np.float32)
    q8, qs = oracle.quantize_q_rows(Q)
    k8, ks = oracle.quantize_k_tiles(K)
    Qd = (q8 * qs[..., None]).astype(np.float64)
    Kd = (k8 * np.repeat(ks, 64, axis=1)[:, :N, :, None]).astype(np.float64)
    bm = brute_block_max(Qd, Kd, Bq, Bk)
    sm = oracle.off_diagonal_block_maxima(Q, K, block_q=Bq, block_k=Bk, gate_dtype="fp8",
                                          dtype=np.float64)
    sm32 = oracle.off_diagonal_block_maxima(Q, K, block_q=Bq, block_k=Bk, gate_dtype="fp8")
    T = _const_table(math.inf, Hq, 8)
    r = oracle_prefill(Q, K, V, block_q=Bq, block_k=Bk, mode=GATE_ABSOLUTE, table=T,
                       gate_dtype="fp8", dtype=np.float64)
    for i in range(-(-N // Bq)):
        n_off = key_block_range(i, N, Bq, Bk)[0]
        # (the oracle holds the softmax scale in float32, as the device does: 2^-24 relative)
        np.testing.assert_allclose(sm[:, :, i, :n_off], bm[:, :, i, :n_off], rtol=2e-7, atol=0)
        # the default float32 run: float32 operands and sums
        np.testing.assert_allclose(sm32[:, :, i, :n_off], bm[:, :, i, :n_off], rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(r.stat[:, :, i, :n_off], bm[:, :, i, :n_off], rtol=2e-7,
                                   atol=0)


def test_fp8_block_maxima_within_the_quantisation_bound():
    rng = np.random.default_rng(45)
    B, N, Hq, Hkv, d, Bq, Bk = 1, 512, 2, 1, 64, 64, 64
    Q = rng.standard_normal((B, N, Hq, d)).astype(np.float32) * 1.5
    K = rng.standard_normal((B, N, Hkv, d)).astype(np.float32)
    sc = 1 / math.sqrt(d)
    exact = oracle.off_diagonal_block_maxima(Q, K, block_q=Bq, block_k=Bk, dtype=np.float64)
    fp8 = oracle.off_diagonal_block_maxima(Q, K, block_q=Bq, block_k=Bk, gate_dtype="fp8")
    _, qs = oracle.quantize_q_rows(Q)
    _, ks = oracle.quantize_k_tiles(K)
    # per element error <= max(2^-4 |x|, 2^-10 scale): bound sum_d |dq||k| + |q||dk| + |dq||dk|
    eq = np.maximum(np.abs(Q) * 2.0 ** -4, 2.0 ** -10 * qs[..., None])
    ek = np.maximum(np.abs(K) * 2.0 ** -4, 2.0 ** -10 * np.repeat(ks, 64, axis=1)[:, :N, :, None])
    for i in range(N // Bq):
        for h in range(Hq):
            q, dq = np.abs(Q[0, i * Bq:(i + 1) * Bq, h]), eq[0, i * Bq:(i + 1) * Bq, h]
            k, dk = np.abs(K[0, :i * Bq, 0]), ek[0, :i * Bq, 0]
            if i == 0:
                continue
            bound = (dq @ k.T + q @ dk.T + dq @ dk.T) * sc
            bmax = bound.reshape(Bq, i, Bk).max(axis=(0, 2))
            diff = np.abs(fp8[0, h, i, :i] - exact[0, h, i, :i])
            assert (diff <= bmax * (1 + 1e-6) + 1e-9).all()
            assert diff.max() > 0                                 # it is not the exact gate


@pytest.mark.parametrize("k", [1, 3])
def test_fp8_calibration_keeps_exactly_k_under_the_fp8_gate(k):
    Q, K, V = _exact_sample(46)
    Bq, Bk = 64, 64
    T = calibrate([(Q, K)], block_q=Bq, block_k=Bk, budgets=[k], gate_dtype="fp8")
    # FP8 maxima are not float32 numbers: the stored threshold may round above the k-th
    # maximum itself, so take it one float32 step lower
    T = np.nextafter(T, np.float32(-np.inf)).astype(np.float32)
    r = oracle_prefill(Q, K, V, block_q=Bq, block_k=Bk, mode=GATE_ABSOLUTE, table=T,
                       gate_dtype="fp8")
    N = Q.shape[1]
    for i in range(-(-N // Bq)):
        n_off = key_block_range(i, N, Bq, Bk)[0]
        want = k if n_off >= k else n_off
        assert (r.kept_counts[:, :, i] == want).all(), (i, r.kept_counts[:, :, i])


def test_fp8_gate_refuses_the_relative_gate():
    Q, K, V = _rand(47, 1, 128, 1, 1, 16)
    with pytest.raises(ValueError):
        oracle_prefill(Q, K, V, block_q=64, block_k=64, mode=GATE_RELATIVE, log_lambda=-1.0,
                       gate_dtype="fp8")
