"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same seeded inputs.

Bar: keep decisions bit-exact outside the 1e-2 near-tie band, kept counts exact, output
max-abs <= 1e-2 and mean-abs <= 1e-3 (bf16 inputs, float32 oracle). Bitwise identities:
DENSE == ABSOLUTE(T = -inf) == RELATIVE(lambda = 0); NaN in the V rows of skipped blocks
changes nothing; back-to-back launches agree bit for bit.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from block_sparse_long_amd import _lib, synth
from block_sparse_long_amd.table import ThresholdTable
from gpu_util import (BAND, MAX_ABS, MEAN_ABS, bf16_pair, check_parity, make_table,
                      quantile_table, run_device)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded():
    _cuda()
    _lib.load_library()


def golden_table(name):
    return ThresholdTable.load(os.path.join(GOLDEN, f"thresholds_{name}.bin"))


# ---------------------------------------------------------------------------------------------
# Tiny single-head workload (1K, d = 64, 64x64 tiles, k = 4 calibrated on seeds 1-4)
# ---------------------------------------------------------------------------------------------
@pytest.fixture(scope="module")
def tiny():
    Q, K, V = synth.make_inputs("tiny_1k", 0)
    (Qd, Kd, Vd), (Qh, Kh, Vh) = bf16_pair(Q, K, V)
    return Qd, Kd, Vd, Qh, Kh, Vh


def test_tiny_absolute_k4(tiny):
    Qd, Kd, Vd, Qh, Kh, Vh = tiny
    tab = golden_table("tiny_1k")
    dev = run_device(Qd, Kd, Vd, block_q=64, mode="absolute", table=tab)
    r = check_parity(dev, Qh, Kh, Vh, block_q=64, mode="absolute", table=tab)
    assert 0 < dev["total"] < sum(oracle.key_block_range(i, 1024, 64, 64)[0] for i in range(16))
    print(f"tiny k=4 kept {dev['total']} of 120 off-diagonal blocks")


@pytest.mark.parametrize("T,expect", [(-math.inf, "all"), (math.inf, "none")])
def test_tiny_threshold_limits(tiny, T, expect):
    Qd, Kd, Vd, Qh, Kh, Vh = tiny
    tab = make_table(np.full((1, 1, 16), T), 64, 64)
    dev = run_device(Qd, Kd, Vd, block_q=64, mode="absolute", table=tab)
    check_parity(dev, Qh, Kh, Vh, block_q=64, mode="absolute", table=tab)
    assert dev["total"] == (120 if expect == "all" else 0)


def test_tiny_dense(tiny):
    Qd, Kd, Vd, Qh, Kh, Vh = tiny
    dev = run_device(Qd, Kd, Vd, block_q=64, mode="dense")
    check_parity(dev, Qh, Kh, Vh, block_q=64, mode="dense")


# ---------------------------------------------------------------------------------------------
# Mid-size cases covering every workgroup shape, ragged tails and GQA
# ---------------------------------------------------------------------------------------------
SHAPES = {  # name: (B, N, Hq, Hkv, d, Bq)
    "llama_like_ragged": (1, 1000, 8, 2, 128, 128),       # 4 waves: 1 head x 128 rows
    "d128_bq64_g4": (1, 700, 8, 2, 128, 64),              # 4 waves: 2 heads x 64 rows
    "d64_bq128_g1": (1, 515, 2, 2, 64, 128),              # 4 waves: 1 head x 128 rows
    "d64_bq64_g2": (2, 333, 4, 2, 64, 64),                # 4 waves: 2 heads, batch 2
    "d64_bq64_g1": (1, 200, 1, 1, 64, 64),                # 2 waves: 1 head x 64 rows
    "d128_bq64_g1": (1, 130, 2, 2, 128, 64),              # 2 waves, d = 128
    "g8": (1, 384, 16, 2, 128, 128),                      # G = 8: 8 workgroups per KV group
}


def _mid_inputs(name, seed):
    B, N, Hq, Hkv, d, Bq = SHAPES[name]
    if B == 1 and Hq % Hkv == 0 and N > 8:
        Q, K, V = synth.structured(seed, N, heads_q=Hq, heads_kv=Hkv, d=d, needles=4)
    else:
        Q, K, V = synth.uniform_mix(seed, B, N, Hq, Hkv, d)
        Q = Q * 1.5
    return Q, K, V


@pytest.fixture(scope="module")
def mid_tables():
    cache = {}

    def get(name, budgets=(2, 4)):
        key = (name, tuple(budgets))
        if key not in cache:
            B, N, Hq, Hkv, d, Bq = SHAPES[name]
            samples = []
            for s in (101, 102):
                Q, K, _ = _mid_inputs(name, s)
                _, (Qh, Kh) = bf16_pair(Q, K)
                samples.append((Qh, Kh))
            T = oracle.calibrate(samples, block_q=Bq, block_k=64, budgets=list(budgets),
                                 scale=float(np.float32(1 / math.sqrt(d))))
            cache[key] = make_table(T, Bq, d, list(budgets))
        return cache[key]
    return get


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("mode", ["dense", "absolute", "relative"])
def test_mid_parity(name, mode, mid_tables):
    B, N, Hq, Hkv, d, Bq = SHAPES[name]
    Q, K, V = _mid_inputs(name, 7)
    (Qd, Kd, Vd), (Qh, Kh, Vh) = bf16_pair(Q, K, V)
    kw = {}
    if mode == "absolute":
        kw = dict(table=mid_tables(name), budget_slice=1)
    elif mode == "relative":
        kw = dict(log_lambda=math.log(1e-3))
    dev = run_device(Qd, Kd, Vd, block_q=Bq, mode=mode, **kw)
    check_parity(dev, Qh, Kh, Vh, block_q=Bq, mode=mode, **kw)


@pytest.mark.parametrize("lam", [1e-4, 1e-2, 1e-1])
def test_relative_gate_lambdas(lam):
    B, N, Hq, Hkv, d, Bq = SHAPES["llama_like_ragged"]
    Q, K, V = _mid_inputs("llama_like_ragged", 8)
    (Qd, Kd, Vd), (Qh, Kh, Vh) = bf16_pair(Q, K, V)
    dev = run_device(Qd, Kd, Vd, block_q=Bq, mode="relative", log_lambda=math.log(lam))
    check_parity(dev, Qh, Kh, Vh, block_q=Bq, mode="relative", log_lambda=math.log(lam))


def test_budget_slices_switch_per_call(mid_tables):
    B, N, Hq, Hkv, d, Bq = SHAPES["llama_like_ragged"]
    tab = mid_tables("llama_like_ragged", budgets=(1, 2, 4))
    Q, K, V = _mid_inputs("llama_like_ragged", 9)
    (Qd, Kd, Vd), (Qh, Kh, Vh) = bf16_pair(Q, K, V)
    totals = []
    for sl in range(3):
        dev = run_device(Qd, Kd, Vd, block_q=Bq, mode="absolute", table=tab, budget_slice=sl)
        check_parity(dev, Qh, Kh, Vh, block_q=Bq, mode="absolute", table=tab, budget_slice=sl)
        totals.append(dev["total"])
    assert totals[0] <= totals[1] <= totals[2]


# ---------------------------------------------------------------------------------------------
# Bitwise identities
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["llama_like_ragged", "d64_bq64_g2", "d64_bq64_g1"])
def test_dense_equals_minus_inf_and_lambda_zero_bitwise(name):
    B, N, Hq, Hkv, d, Bq = SHAPES[name]
    Q, K, V = _mid_inputs(name, 10)
    (Qd, Kd, Vd), _ = bf16_pair(Q, K, V)
    nqb = -(-N // Bq)
    dense = run_device(Qd, Kd, Vd, block_q=Bq, mode="dense", dbg=False)["O"]
    dense16 = run_device(Qd, Kd, Vd, block_q=Bq, mode="dense", dbg=False,
                         out_dtype=torch.bfloat16)["O"]
    assert torch.equal(dense16, dense.to(torch.bfloat16))     # bf16 out = RNE(fp32 out)
    tab = make_table(np.full((1, Hq, nqb), -np.inf), Bq, d)
    absm = run_device(Qd, Kd, Vd, block_q=Bq, mode="absolute", table=tab)
    rel0 = run_device(Qd, Kd, Vd, block_q=Bq, mode="relative", log_lambda=-math.inf)
    assert torch.equal(dense, absm["O"])
    assert torch.equal(dense, rel0["O"])
    n_off_total = B * Hq * sum(oracle.key_block_range(i, N, Bq, 64)[0] for i in range(nqb))
    assert absm["total"] == rel0["total"] == n_off_total


@pytest.mark.parametrize("mode,Bq", [("dense", 128), ("relative", 128), ("absolute", 128),
                                     ("dense", 64)])
def test_ticket_order_with_heaviest_first_tail_bitwise(mode, Bq):
    # 8100 tokens (ragged), 32 query / 8 KV heads: more units than resident workgroups, so a
    # ticket launch takes the query blocks above a cut KV head by KV head and those below it
    # last, heaviest first (Bq = 128: 64 blocks, cut about 46; Bq = 64: 127 blocks, cut about
    # 91). Every unit still runs exactly once: output, counts and statistics equal those of one
    # workgroup per unit (the absolute gate: its two launches, the walk taking tickets, equal
    # the one launch without a workspace)
    N, Hq, Hkv, d = 8100, 32, 8, 128
    Q, K, V = synth.structured(21, N, heads_q=Hq, heads_kv=Hkv, d=d, needles=4)
    (Qd, Kd, Vd), (Qh, Kh, _) = bf16_pair(Q, K, V)
    kw = dict(block_q=Bq, mode=mode)
    if mode == "relative":
        kw["log_lambda"] = math.log(3e-2)
    if mode == "absolute":
        kw["table"] = quantile_table(Qh, Kh, Bq, 64)
    need = _lib.bsfa_prefill_workspace_bytes(Qd, Kd, block_q=Bq, gate_mode=mode)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    none = torch.empty(0, dtype=torch.uint8, device="cuda")
    one = run_device(Qd, Kd, Vd, workspace=none, **kw)
    tk = run_device(Qd, Kd, Vd, workspace=ws, **kw)
    assert torch.equal(tk["O"], one["O"])
    np.testing.assert_array_equal(tk["counts"], one["counts"])
    assert tk["total"] == one["total"]
    np.testing.assert_array_equal(np.nan_to_num(tk["stat"], nan=7.0),
                                  np.nan_to_num(one["stat"], nan=7.0))
    if mode != "dense":   # the gate skipped some blocks and kept others
        nqb = -(-N // Bq)
        n_off = Hq * sum(oracle.key_block_range(i, N, Bq, 64)[0] for i in range(nqb))
        assert 0 < tk["total"] < n_off


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("mode,lam", [("dense", 0.0), ("relative", 0.0), ("relative", 3e-2)])
def test_ticket_launch_equals_one_workgroup_per_unit_bitwise(name, mode, lam):
    # dense and the relative gate: with a workspace the resident workgroups take their units
    # from a counter in it, without one each unit runs in a workgroup of its own. The order of
    # the units changes nothing: output, counts and statistics agree bit for bit, also on a
    # second call through the same workspace (each call zeroes its counter)
    B, N, Hq, Hkv, d, Bq = SHAPES[name]
    Q, K, V = _mid_inputs(name, 12)
    (Qd, Kd, Vd), _ = bf16_pair(Q, K, V)
    ll = math.log(lam) if lam > 0 else -math.inf
    assert _lib.bsfa_prefill_workspace_bytes(Qd, Kd, block_q=Bq, gate_mode=mode) == 256
    ws = torch.full((256,), 0xA5, dtype=torch.uint8, device="cuda")
    none = torch.empty(0, dtype=torch.uint8, device="cuda")
    kw = dict(block_q=Bq, mode=mode, log_lambda=ll)
    one = run_device(Qd, Kd, Vd, workspace=none, **kw)
    for _ in range(2):
        tk = run_device(Qd, Kd, Vd, workspace=ws, **kw)
        assert torch.equal(tk["O"], one["O"])
        np.testing.assert_array_equal(tk["counts"], one["counts"])
        assert tk["total"] == one["total"]
        np.testing.assert_array_equal(np.nan_to_num(tk["stat"], nan=7.0),
                                      np.nan_to_num(one["stat"], nan=7.0))


def test_poisoned_skipped_values_bitwise(mid_tables):
    # a skipped block loads no V and adds nothing: with NaN in the V rows of key block j0,
    # every (head, query block) that skips j0 (outside the near-tie band) keeps a
    # bit-identical output; the rows that keep j0 are not compared
    B, N, Hq, Hkv, d, Bq = SHAPES["llama_like_ragged"]
    tab = mid_tables("llama_like_ragged")
    Q, K, V = _mid_inputs("llama_like_ragged", 11)
    (Qd, Kd, Vd), _ = bf16_pair(Q, K, V)
    ref = run_device(Qd, Kd, Vd, block_q=Bq, mode="absolute", table=tab, budget_slice=0)
    G = Hq // Hkv
    stat = ref["stat"]
    nqb = stat.shape[2]
    checked = 0
    for j0 in (1, 3, 6):
        g0 = 0
        Vp = Vd.clone()
        Vp[:, j0 * 64:(j0 + 1) * 64, g0, :] = float("nan")
        pois = run_device(Qd, Kd, Vp, block_q=Bq, mode="absolute", table=tab, budget_slice=0)
        np.testing.assert_array_equal(ref["counts"], pois["counts"])
        for h in range(g0 * G, (g0 + 1) * G):
            for i in range(nqb):
                n_off = oracle.key_block_range(i, N, Bq, 64)[0]
                thr = tab.T[0][h, min(i, tab.t_len - 1)]
                if j0 < n_off and stat[0, h, i, j0] < thr - 2e-2:
                    rows = slice(i * Bq, min((i + 1) * Bq, N))
                    assert torch.equal(ref["O"][:, rows, h], pois["O"][:, rows, h]), (j0, h, i)
                    checked += 1
                elif j0 < n_off and stat[0, h, i, j0] >= thr:
                    rows = slice(i * Bq, min((i + 1) * Bq, N))
                    assert torch.isnan(pois["O"][:, rows, h]).any()     # kept: V was read
    assert checked >= 8


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("dbg", [True, False])
def test_absolute_gate_sweep_and_single_launch_agree_bitwise(name, dbg, mid_tables):
    # with a workspace the keep masks come from the separate gate sweep, without one from the
    # softmax kernel's own first pass: same decisions, same output bits. The table is handed
    # over without its budgets, so that the call with a workspace takes two launches whatever
    # share of blocks the budget keeps; with its budgets recorded, a budget that keeps most
    # blocks, or a call this small, makes the library take one launch, with the same bits.
    B, N, Hq, Hkv, d, Bq = SHAPES[name]
    tab = mid_tables(name)
    Q, K, V = _mid_inputs(name, 14)
    (Qd, Kd, Vd), _ = bf16_pair(Q, K, V)
    need = _lib.bsfa_prefill_workspace_bytes(Qd, Kd, block_q=Bq)
    ws = torch.full((need + 64,), 0xA5, dtype=torch.uint8, device="cuda")   # stale contents
    none = torch.empty(0, dtype=torch.uint8, device="cuda")
    for sl in (0, 1):
        a = run_device(Qd, Kd, Vd, block_q=Bq, mode="absolute", table=tab, budget_slice=sl,
                       dbg=dbg, workspace=ws, record_budgets=False)
        b = run_device(Qd, Kd, Vd, block_q=Bq, mode="absolute", table=tab, budget_slice=sl,
                       dbg=dbg, workspace=none)
        c = run_device(Qd, Kd, Vd, block_q=Bq, mode="absolute", table=tab, budget_slice=sl,
                       dbg=dbg, workspace=ws, record_budgets=True)
        for x in (a, c):
            assert torch.equal(x["O"], b["O"])
            np.testing.assert_array_equal(x["counts"], b["counts"])
            assert x["total"] == b["total"]
            if dbg:
                np.testing.assert_array_equal(x["stat"], b["stat"])


def test_full_size_two_launch_call_equals_single_launch_bitwise():
    # at 32K (256 query blocks): the absolute gate with a workspace (gate sweep, then the walk)
    # gives the single launch's output, counts and statistics, and the masks it leaves in the
    # workspace (bf16 and FP8 scores) are those of a separate gate-mask launch
    name = "llama_32k_sweep"
    c = synth.CONFIGS[name]
    Bq, N, Hq = c["block_q"], c["n"], c["heads_q"]
    nqb = -(-N // Bq)
    print(f"case {name} two launches vs one", flush=True)
    Q, K, V = synth.make_inputs(name, 3)
    Qd, Kd, Vd = (x.to("cuda") for x in synth.to_bf16(Q, K, V))
    tab = ThresholdTable.load(os.path.join(GOLDEN, f"thresholds_{name}.bin"))
    dtab = tab.to_device("cuda")
    none = torch.empty(0, dtype=torch.uint8, device="cuda")
    a = run_device(Qd, Kd, Vd, block_q=Bq, mode="absolute", table=tab, budget_slice=1,
                   dbg=True)
    b = run_device(Qd, Kd, Vd, block_q=Bq, mode="absolute", table=tab, budget_slice=1,
                   dbg=True, workspace=none)
    assert torch.equal(a["O"], b["O"])
    np.testing.assert_array_equal(a["counts"], b["counts"])
    assert a["total"] == b["total"]
    np.testing.assert_array_equal(a["stat"], b["stat"])
    # k = 256 keeps most blocks: with a workspace the library takes one launch whose
    # workgroups draw units from the workspace's counter; the same bits as without one
    a = run_device(Qd, Kd, Vd, block_q=Bq, mode="absolute", table=tab, budget_slice=2,
                   dbg=False, record_budgets=True)
    b = run_device(Qd, Kd, Vd, block_q=Bq, mode="absolute", table=tab, budget_slice=2,
                   dbg=False, workspace=none)
    assert torch.equal(a["O"], b["O"])
    np.testing.assert_array_equal(a["counts"], b["counts"])
    # query blocks whose thresholds are finite for every head (the others keep all without a
    # mask)
    T = tab.T[1]
    qbs = [i for i in range(nqb) if np.isfinite(T[:, min(i, T.shape[1] - 1)]).all()]
    assert len(qbs) > nqb // 2
    for gd in ("bf16", "fp8"):
        need = _lib.bsfa_prefill_workspace_bytes(Qd, Kd, block_q=Bq, gate_dtype=gd)
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
        O = torch.empty_like(Qd)
        _lib.bsfa_prefill(Qd, Kd, Vd, O, block_q=Bq, gate_mode="absolute", table=dtab,
                          budget_slice=1, workspace=ws, gate_dtype=gd)
        ref = _lib.bsfa_gate_masks(Qd, Kd, dtab, 1, block_q=Bq, gate_dtype=gd)
        torch.cuda.synchronize()
        ref = ref.cpu().numpy()
        got = ws[:ref.size * 8].view(torch.int64).view(ref.shape).cpu().numpy()
        for i in qbs:
            words = -(-(i * Bq // 64) // 64)
            np.testing.assert_array_equal(got[:, :, i, :words], ref[:, :, i, :words],
                                          err_msg=f"{gd} query block {i}")


def _unpack_masks(mask, nkb):
    m = np.ascontiguousarray(mask.cpu().numpy()).view(np.uint8)
    bits = np.unpackbits(m, axis=-1, bitorder="little").astype(bool)
    return bits[..., :nkb], bits[..., nkb:]


@pytest.mark.parametrize("name", list(SHAPES))
def test_gate_masks_match_oracle_decisions(name, mid_tables):
    # the keep decisions alone: the mask bits are the device's own fp32 comparison of its dumped
    # maxima with the threshold, the oracle's outside the near-tie band, and zero elsewhere
    B, N, Hq, Hkv, d, Bq = SHAPES[name]
    tab = mid_tables(name)
    dtab = tab.to_device("cuda")
    Q, K, V = _mid_inputs(name, 15)
    (Qd, Kd, Vd), (Qh, Kh, Vh) = bf16_pair(Q, K, V)
    nqb, nkb = -(-N // Bq), -(-N // 64)
    W = -(-nkb // 64)
    for sl in (0, 1):
        mask = torch.full((B, Hq, nqb, W), -0x5A5A5A5A5A5A5A5B, dtype=torch.int64, device="cuda")
        stat = torch.full((B, Hq, nqb, nkb), float("nan"), dtype=torch.float32, device="cuda")
        _lib.bsfa_gate_masks(Qd, Kd, dtab, sl, mask, block_q=Bq, debug_block_stat=stat)
        torch.cuda.synchronize()
        bits, pad = _unpack_masks(mask, nkb)
        assert not pad.any()
        st = stat.cpu().numpy()
        r = oracle.oracle_prefill(Qh, Kh, Vh, block_q=Bq, block_k=64, mode="absolute",
                                  table=tab.T, budget_slice=sl)
        for i in range(nqb):
            n_off = oracle.key_block_range(i, N, Bq, 64)[0]
            assert not bits[:, :, i, n_off:].any()
            thr = tab.T[sl][:, min(i, tab.t_len - 1)].astype(np.float32)
            dev = st[:, :, i, :n_off] >= thr[None, :, None]
            np.testing.assert_array_equal(bits[:, :, i, :n_off], dev)
            mg = r.margin[:, :, i, :n_off]
            outside = np.abs(mg) > BAND
            np.testing.assert_array_equal(bits[:, :, i, :n_off][outside],
                                          r.keep[:, :, i, :n_off][outside])
            fin = np.isfinite(r.stat[:, :, i, :n_off])
            np.testing.assert_allclose(st[:, :, i, :n_off][fin], r.stat[:, :, i, :n_off][fin],
                                       rtol=1e-5, atol=2e-3)


@pytest.mark.parametrize("name", list(SHAPES))
def test_gate_masks_through_a_workspace_match_the_mask_buffer(name, mid_tables):
    # a buffer of bsfa_prefill's workspace size makes the sweep take its units from the
    # workspace's counter (the order bsfa_prefill uses); masks and statistics are the same bits
    B, N, Hq, Hkv, d, Bq = SHAPES[name]
    dtab = mid_tables(name).to_device("cuda")
    Q, K, V = _mid_inputs(name, 17)
    (Qd, Kd, Vd), _ = bf16_pair(Q, K, V)
    nqb, nkb = -(-N // Bq), -(-N // 64)
    need = _lib.bsfa_prefill_workspace_bytes(Qd, Kd, block_q=Bq)
    for sl in (0, 1):
        out = []
        for buf in (None, torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")):
            stat = torch.full((B, Hq, nqb, nkb), float("nan"), dtype=torch.float32,
                              device="cuda")
            for _ in range(2):   # the second call finds the counter as the first left it
                m = _lib.bsfa_gate_masks(Qd, Kd, dtab, sl, buf, block_q=Bq,
                                         debug_block_stat=stat)
            torch.cuda.synchronize()
            out.append((m.cpu().numpy().copy(), stat.cpu().numpy()))
        np.testing.assert_array_equal(out[0][0], out[1][0])
        np.testing.assert_array_equal(out[0][1], out[1][1])


def test_gate_masks_minus_inf_keeps_all_and_writes_every_word():
    B, N, Hq, Hkv, d, Bq = SHAPES["llama_like_ragged"]
    Q, K, V = _mid_inputs("llama_like_ragged", 16)
    (Qd, Kd, Vd), _ = bf16_pair(Q, K, V)
    nqb, nkb = -(-N // Bq), -(-N // 64)
    tab = make_table(np.full((1, Hq, nqb), -np.inf), Bq, d).to_device("cuda")
    mask = torch.full((B, Hq, nqb, -(-nkb // 64)), -1, dtype=torch.int64, device="cuda")
    _lib.bsfa_gate_masks(Qd, Kd, tab, 0, mask, block_q=Bq)
    torch.cuda.synchronize()
    bits, pad = _unpack_masks(mask, nkb)
    assert not pad.any()
    for i in range(nqb):
        n_off = oracle.key_block_range(i, N, Bq, 64)[0]
        assert bits[:, :, i, :n_off].all() and not bits[:, :, i, n_off:].any()


# ---------------------------------------------------------------------------------------------
# Chunked prefill: query rows after a prefix of cached keys (K and V longer than Q)
# ---------------------------------------------------------------------------------------------
PREFIX_CASES = [   # (shape, prefix, modes)
    ("llama_like_ragged", 256, ("dense", "absolute", "relative")),   # aligned to Bq = 128
    ("llama_like_ragged", 100, ("dense", "relative")),               # off the tile grid
    ("d64_bq64_g2", 128, ("dense", "absolute", "relative")),          # batch 2, Bq = 64
    ("d128_bq64_g4", 64, ("absolute",)),
    ("g8", 256, ("absolute", "relative")),
]


@pytest.mark.parametrize("name,prefix,modes", PREFIX_CASES)
def test_prefix_parity(name, prefix, modes, mid_tables):
    B, N, Hq, Hkv, d, Bq = SHAPES[name]
    Q, K, V = _mid_inputs(name, 17)
    (Qd, Kd, Vd), (Qh, Kh, Vh) = bf16_pair(Q[:, prefix:].contiguous(), K, V)
    for mode in modes:
        kw = {}
        if mode == "absolute":
            kw = dict(table=mid_tables(name), budget_slice=1)
        elif mode == "relative":
            kw = dict(log_lambda=math.log(1e-3))
        dev = run_device(Qd, Kd, Vd, block_q=Bq, mode=mode, **kw)
        check_parity(dev, Qh, Kh, Vh, block_q=Bq, mode=mode, **kw)


@pytest.mark.parametrize("name,prefix", [("llama_like_ragged", 256), ("llama_like_ragged", 640),
                                         ("d64_bq64_g2", 192), ("g8", 128)])
def test_chunks_equal_rows_of_the_whole_call_bitwise(name, prefix, mid_tables):
    # a chunk on the query-block grid computes every query block exactly as the whole call does
    B, N, Hq, Hkv, d, Bq = SHAPES[name]
    tab = mid_tables(name)
    Q, K, V = _mid_inputs(name, 18)
    (Qd, Kd, Vd), _ = bf16_pair(Q, K, V)
    Qc = Qd[:, prefix:].contiguous()
    i0 = prefix // Bq
    none = torch.empty(0, dtype=torch.uint8, device="cuda")
    for mode, kw in (("dense", {}), ("relative", dict(log_lambda=math.log(1e-3))),
                     ("absolute", dict(table=tab, budget_slice=1)),
                     ("absolute", dict(table=tab, budget_slice=0, workspace=none))):
        full = run_device(Qd, Kd, Vd, block_q=Bq, mode=mode, **kw)
        part = run_device(Qc, Kd, Vd, block_q=Bq, mode=mode, **kw)
        assert torch.equal(part["O"], full["O"][:, prefix:]), mode
        np.testing.assert_array_equal(part["counts"], full["counts"][:, :, i0:])
        np.testing.assert_array_equal(part["stat"], full["stat"][:, :, i0:])


def test_gate_masks_with_prefix_match_the_whole_call(mid_tables):
    B, N, Hq, Hkv, d, Bq = SHAPES["llama_like_ragged"]
    tab = mid_tables("llama_like_ragged").to_device("cuda")
    Q, K, V = _mid_inputs("llama_like_ragged", 19)
    (Qd, Kd, Vd), _ = bf16_pair(Q, K, V)
    full = _lib.bsfa_gate_masks(Qd, Kd, tab, 1, block_q=Bq)
    part = _lib.bsfa_gate_masks(Qd[:, 384:].contiguous(), Kd, tab, 1, block_q=Bq)
    torch.cuda.synchronize()
    assert torch.equal(part, full[:, :, 3:])


# ---------------------------------------------------------------------------------------------
# Variable-length batches
# ---------------------------------------------------------------------------------------------
def _varlen_batch(seed, Hq, Hkv, d, nq, nk):
    """Packed sequences of the given query / key lengths (key length >= query length)."""
    g = torch.Generator().manual_seed(seed)
    cu_q = np.cumsum([0] + nq).astype(np.int32)
    cu_k = np.cumsum([0] + nk).astype(np.int32)
    Q = torch.randn(int(cu_q[-1]), Hq, d, generator=g) * 1.5
    K = torch.randn(int(cu_k[-1]), Hkv, d, generator=g)
    V = torch.randn(int(cu_k[-1]), Hkv, d, generator=g)
    return Q, K, V, cu_q, cu_k


VARLEN = [   # Hq, Hkv, d, Bq, query lengths, key lengths
    (8, 2, 128, 128, [1000, 0, 300, 64, 517], [1000, 0, 556, 64, 773]),
    (4, 2, 64, 64, [200, 333, 64], [328, 333, 192]),
]


@pytest.mark.parametrize("case", VARLEN)
@pytest.mark.parametrize("mode", ["dense", "absolute", "relative"])
def test_varlen_equals_one_call_per_sequence_bitwise(case, mode):
    Hq, Hkv, d, Bq, nq, nk = case
    Q, K, V, cu_q, cu_k = _varlen_batch(20, Hq, Hkv, d, nq, nk)
    (Qd, Kd, Vd), _ = bf16_pair(Q, K, V)
    B, nqb_max, nkb_max = len(nq), -(-max(nq) // Bq), -(-max(nk) // 64)
    kw = {}
    if mode == "absolute":
        T = np.random.default_rng(3).uniform(-1.0, 3.0, (2, Hq, nqb_max + 8)).astype(np.float32)
        kw = dict(table=make_table(T, Bq, d).to_device("cuda", record_budgets=False),
                  budget_slice=1)   # two launches: the sweep and the walk
    elif mode == "relative":
        kw = dict(log_lambda=math.log(1e-2))
    counts = torch.full((B, Hq, nqb_max), -7, dtype=torch.int32, device="cuda")
    stat = torch.full((B, Hq, nqb_max, nkb_max), float("nan"), device="cuda")
    O = _lib.bsfa_prefill_varlen(Qd, Kd, Vd, torch.tensor(cu_q, device="cuda"),
                                 torch.tensor(cu_k, device="cuda"), max(nq), max(nk),
                                 block_q=Bq, gate_mode=mode, kept_counts=counts,
                                 debug_block_stat=stat, out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    for b in range(B):
        if nq[b] == 0:
            assert (counts[b] == -7).all()
            continue
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        c1 = torch.zeros((1, Hq, -(-nq[b] // Bq)), dtype=torch.int32, device="cuda")
        s1 = torch.full((1, Hq, -(-nq[b] // Bq), -(-nk[b] // 64)), float("nan"), device="cuda")
        O1 = _lib.bsfa_prefill(Qd[None, q0:q1], Kd[None, k0:k1], Vd[None, k0:k1], block_q=Bq,
                               gate_mode=mode, kept_counts=c1, debug_block_stat=s1,
                               out_dtype=torch.float32, **kw)
        torch.cuda.synchronize()
        one = dict(O=O1, counts=c1.cpu().numpy(), stat=s1.cpu().numpy())
        assert torch.equal(O[q0:q1], one["O"][0]), b
        qb, kb = one["counts"].shape[2], one["stat"].shape[3]
        np.testing.assert_array_equal(counts[b, :, :qb].cpu().numpy(), one["counts"][0])
        assert (counts[b, :, qb:] == -7).all()
        np.testing.assert_array_equal(stat[b, :, :qb, :kb].cpu().numpy(), one["stat"][0])


@pytest.mark.parametrize("case", VARLEN)
def test_varlen_parity_with_oracle(case):
    # the packed addressing and the per-sequence prefixes against the oracle (dense: no gate
    # decisions, whose near-ties the per-sequence tests cover)
    Hq, Hkv, d, Bq, nq, nk = case
    Q, K, V, cu_q, cu_k = _varlen_batch(21, Hq, Hkv, d, nq, nk)
    (Qd, Kd, Vd), (Qh, Kh, Vh) = bf16_pair(Q, K, V)
    O = _lib.bsfa_prefill_varlen(Qd, Kd, Vd, torch.tensor(cu_q, device="cuda"),
                                 torch.tensor(cu_k, device="cuda"), max(nq), max(nk),
                                 block_q=Bq, gate_mode="dense", out_dtype=torch.float32)
    torch.cuda.synchronize()
    r = oracle.oracle_prefill_varlen(Qh, Kh, Vh, cu_q, cu_k, block_q=Bq, block_k=64,
                                     mode="dense")
    err = np.abs(O.cpu().numpy() - r.out)
    assert np.isfinite(O.cpu().numpy()).all()
    assert err.max() <= 1e-2 and err.mean() <= 1e-3, (err.max(), err.mean())


def test_back_to_back_launches_bitwise(mid_tables):
    B, N, Hq, Hkv, d, Bq = SHAPES["llama_like_ragged"]
    # two launches per call (the ticket counters are cleared and reused every time)
    tab = mid_tables("llama_like_ragged").to_device("cuda", record_budgets=False)
    Q, K, V = _mid_inputs("llama_like_ragged", 12)
    (Qd, Kd, Vd), _ = bf16_pair(Q, K, V)
    outs = [torch.empty_like(Qd) for _ in range(100)]
    counts = torch.empty((100, B, Hq, -(-N // Bq)), dtype=torch.int32, device="cuda")
    for t in range(100):
        _lib.bsfa_prefill(Qd, Kd, Vd, outs[t], block_q=Bq, gate_mode="absolute", table=tab,
                          budget_slice=t % 2, kept_counts=counts[t])
    torch.cuda.synchronize()
    for t in range(2, 100):
        assert torch.equal(outs[t], outs[t % 2])
        assert torch.equal(counts[t], counts[t % 2])


# ---------------------------------------------------------------------------------------------
# Layouts, output dtype, empty inputs
# ---------------------------------------------------------------------------------------------
def test_head_major_strided_layout_and_fp32_output(mid_tables):
    B, N, Hq, Hkv, d, Bq = SHAPES["d64_bq64_g2"]
    Q, K, V = _mid_inputs("d64_bq64_g2", 13)
    (Qd, Kd, Vd), (Qh, Kh, Vh) = bf16_pair(Q, K, V)
    # a [B, H, N, d] caller: pass permuted views (token and head strides swap)
    Qt = Qd.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    Kt = Kd.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    Vt = Vd.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    assert Qt.stride(1) == d and not Qt.is_contiguous()
    tab = mid_tables("d64_bq64_g2")
    dev = run_device(Qt, Kt, Vt, block_q=Bq, mode="absolute", table=tab, out_dtype=torch.float32)
    assert dev["O"].dtype == torch.float32
    check_parity(dev, Qh, Kh, Vh, block_q=Bq, mode="absolute", table=tab)
    base = run_device(Qd, Kd, Vd, block_q=Bq, mode="absolute", table=tab,
                      out_dtype=torch.bfloat16)
    assert torch.equal(base["O"], dev["O"].to(torch.bfloat16))


@pytest.mark.parametrize("B,N", [(0, 128), (1, 0)])
def test_empty_inputs(B, N):
    Q = torch.zeros((B, N, 2, 64), dtype=torch.bfloat16, device="cuda")
    K = torch.zeros((B, N, 1, 64), dtype=torch.bfloat16, device="cuda")
    total = torch.full((1,), 99, dtype=torch.int64, device="cuda")
    O = _lib.bsfa_prefill(Q, K, K, block_q=64, gate_mode="dense", kept_total=total)
    torch.cuda.synchronize()
    assert O.shape == Q.shape and int(total.item()) == 0


def test_single_token():
    Q, K, V = synth.uniform_mix(5, 1, 1, 4, 1, 128)
    (Qd, Kd, Vd), (Qh, Kh, Vh) = bf16_pair(Q, K, V)
    dev = run_device(Qd, Kd, Vd, block_q=128, mode="relative", log_lambda=math.log(1e-2))
    check_parity(dev, Qh, Kh, Vh, block_q=128, mode="relative", log_lambda=math.log(1e-2))
    np.testing.assert_allclose(dev["O"].float().cpu().numpy()[0, 0, 0], Vh[0, 0, 0], atol=1e-2)


# ---------------------------------------------------------------------------------------------
# Calibration kernel
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["llama_like_ragged", "d64_bq64_g2", "g8"])
def test_calibration_kernel_matches_oracle(name):
    B, N, Hq, Hkv, d, Bq = SHAPES[name]
    Q, K, _ = _mid_inputs(name, 14)
    (Qd, Kd), (Qh, Kh) = bf16_pair(Q, K)
    budgets = [1, 2, 3, 5, 8]
    kth = _lib.bsfa_calibrate_blockmax(Qd, Kd, budgets, block_q=Bq)
    torch.cuda.synchronize()
    kth = kth.cpu().numpy()
    sm = oracle.off_diagonal_block_maxima(Qh, Kh, block_q=Bq, block_k=64)
    for kk, k in enumerate(budgets):
        for b in range(B):
            for h in range(Hq):
                for i in range(sm.shape[2]):
                    n_off = oracle.key_block_range(i, N, Bq, 64)[0]
                    ref = oracle.kth_highest(sm[b, h, i], n_off, k)
                    got = kth[kk, b, h, i]
                    if math.isinf(ref):
                        assert got == ref
                    else:
                        assert abs(got - ref) <= 1e-3, (k, b, h, i, got, ref)


# ---------------------------------------------------------------------------------------------
# Paged K / V
# ---------------------------------------------------------------------------------------------
def _to_pages(X, cu, page, seed):
    """Scatter packed sequences [tokens, H, d] into a shuffled page pool with spare pages."""
    rng = np.random.default_rng(seed)
    lens = np.diff(cu)
    n_pages = [-(-int(n) // page) for n in lens]
    free = list(rng.permutation(sum(n_pages) + 5))
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


@pytest.mark.parametrize("page", [64, 128, 192])
@pytest.mark.parametrize("mode", ["dense", "absolute", "relative"])
def test_paged_equals_packed_bitwise(page, mode):
    Hq, Hkv, d, Bq, nq, nk = VARLEN[0]
    Q, K, V, cu_q, cu_k = _varlen_batch(25, Hq, Hkv, d, nq, nk)
    (Qd, Kd, Vd), _ = bf16_pair(Q, K, V)
    Kp, table = _to_pages(Kd, cu_k, page, 7)
    Vp, table_v = _to_pages(Vd, cu_k, page, 7)
    assert torch.equal(table, table_v)
    kw = {}
    if mode == "absolute":
        T = np.random.default_rng(3).uniform(-1.0, 3.0, (2, Hq, 16)).astype(np.float32)
        kw = dict(table=make_table(T, Bq, d).to_device("cuda", record_budgets=False),
                  budget_slice=1)   # two launches: the sweep and the walk
    elif mode == "relative":
        kw = dict(log_lambda=math.log(1e-2))
    B, nqb = len(nq), -(-max(nq) // Bq)
    cq = torch.tensor(cu_q, device="cuda")
    c1 = torch.full((B, Hq, nqb), -7, dtype=torch.int32, device="cuda")
    c2 = torch.full_like(c1, -7)
    O1 = _lib.bsfa_prefill_varlen(Qd, Kd, Vd, cq, torch.tensor(cu_k, device="cuda"), max(nq),
                                  max(nk), block_q=Bq, gate_mode=mode, kept_counts=c1,
                                  out_dtype=torch.float32, **kw)
    O2 = _lib.bsfa_prefill_paged(Qd, Kp, Vp, cq, torch.tensor(np.diff(cu_k), dtype=torch.int32,
                                                                 device="cuda"),
                                 table, max(nq), max(nk), block_q=Bq, gate_mode=mode,
                                 kept_counts=c2, out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2)
    assert torch.equal(c1, c2)


def test_paged_parity_with_oracle():
    Hq, Hkv, d, Bq, nq, nk = VARLEN[1]
    Q, K, V, cu_q, cu_k = _varlen_batch(26, Hq, Hkv, d, nq, nk)
    (Qd, Kd, Vd), (Qh, Kh, Vh) = bf16_pair(Q, K, V)
    Kp, table = _to_pages(Kd, cu_k, 128, 8)
    Vp, _ = _to_pages(Vd, cu_k, 128, 8)
    lens = np.diff(cu_k).astype(np.int32)
    O = _lib.bsfa_prefill_paged(Qd, Kp, Vp, torch.tensor(cu_q, device="cuda"),
                                torch.tensor(lens, device="cuda"), table, max(nq), max(nk),
                                block_q=Bq, gate_mode="dense", out_dtype=torch.float32)
    torch.cuda.synchronize()
    Kg, cu = oracle.gather_pages(Kp.float().cpu().numpy(), table.cpu().numpy(), lens)
    Vg, _ = oracle.gather_pages(Vp.float().cpu().numpy(), table.cpu().numpy(), lens)
    r = oracle.oracle_prefill_varlen(Qh, Kg, Vg, cu_q, cu, block_q=Bq, block_k=64, mode="dense")
    err = np.abs(O.cpu().numpy() - r.out)
    assert np.isfinite(O.cpu().numpy()).all()
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (err.max(), err.mean())


# ---------------------------------------------------------------------------------------------
# 128-key gate blocks (128 x 128 tiles): decided by the gate sweep
# ---------------------------------------------------------------------------------------------
BK128 = ["llama_like_ragged", "g8", "d64_bq128_g1"]


def _bk128_table(name, budgets=(1, 2)):
    B, N, Hq, Hkv, d, Bq = SHAPES[name]
    samples = []
    for s_ in (101, 102):
        Q, K, _ = _mid_inputs(name, s_)
        _, (Qh, Kh) = bf16_pair(Q, K)
        samples.append((Qh, Kh))
    T = oracle.calibrate(samples, block_q=Bq, block_k=128, budgets=list(budgets),
                         scale=float(np.float32(1 / math.sqrt(d))))
    return make_table(T, Bq, d, list(budgets), block_k=128)


@pytest.mark.parametrize("name", BK128)
def test_bk128_gate_masks_and_prefill_match_oracle(name):
    B, N, Hq, Hkv, d, Bq = SHAPES[name]
    tab = _bk128_table(name)
    dtab = tab.to_device("cuda")
    Q, K, V = _mid_inputs(name, 22)
    (Qd, Kd, Vd), (Qh, Kh, Vh) = bf16_pair(Q, K, V)
    nqb, nkb, ntile = -(-N // Bq), -(-N // 128), -(-N // 64)
    for sl in (0, 1):
        mask = torch.full((B, Hq, nqb, -(-ntile // 64)), -1, dtype=torch.int64, device="cuda")
        stat = torch.full((B, Hq, nqb, nkb), float("nan"), device="cuda")
        _lib.bsfa_gate_masks(Qd, Kd, dtab, sl, mask, block_q=Bq, block_k=128,
                             debug_block_stat=stat)
        counts = torch.full((B, Hq, nqb), -7, dtype=torch.int32, device="cuda")
        O = _lib.bsfa_prefill(Qd, Kd, Vd, block_q=Bq, block_k=128, gate_mode="absolute",
                              table=dtab, budget_slice=sl, kept_counts=counts,
                              out_dtype=torch.float32)
        torch.cuda.synchronize()
        m = np.ascontiguousarray(mask.cpu().numpy()).view(np.uint8)
        bits = np.unpackbits(m, axis=-1, bitorder="little").astype(bool)[..., :ntile]
        st = stat.cpu().numpy()
        # a block's two tiles carry one decision: the device's fp32 comparison of its maximum
        keep_dev = np.zeros((B, Hq, nqb, nkb), bool)
        for i in range(nqb):
            n_off = oracle.key_block_range(i, N, Bq, 128)[0]
            thr = tab.T[sl][:, min(i, tab.t_len - 1)].astype(np.float32)
            kb = st[:, :, i, :n_off] >= thr[None, :, None]
            np.testing.assert_array_equal(bits[:, :, i, 0:2 * n_off:2], kb)
            np.testing.assert_array_equal(bits[:, :, i, 1:2 * n_off:2], kb)
            assert not bits[:, :, i, 2 * n_off:].any()
            keep_dev[:, :, i, :n_off] = kb
        np.testing.assert_array_equal(counts.cpu().numpy(), keep_dev.sum(-1))
        r = oracle.oracle_prefill(Qh, Kh, Vh, block_q=Bq, block_k=128, mode="absolute",
                                  table=tab.T, budget_slice=sl, forced_keep=keep_dev, band=BAND)
        for i in range(nqb):
            n_off = oracle.key_block_range(i, N, Bq, 128)[0]
            mg = r.margin[:, :, i, :n_off]
            out = np.abs(mg) > BAND
            np.testing.assert_array_equal(r.keep[:, :, i, :n_off][out], keep_dev[:, :, i, :n_off][out])
            fin = np.isfinite(r.stat[:, :, i, :n_off])
            np.testing.assert_allclose(st[:, :, i, :n_off][fin], r.stat[:, :, i, :n_off][fin],
                                       rtol=1e-5, atol=2e-3)
        err = np.abs(O.cpu().numpy() - r.out)
        assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (err.max(), err.mean())


@pytest.mark.parametrize("name", ["llama_like_ragged", "d64_bq128_g1"])
def test_bk128_dense_equals_bk64_and_counts_blocks(name):
    B, N, Hq, Hkv, d, Bq = SHAPES[name]
    Q, K, V = _mid_inputs(name, 23)
    (Qd, Kd, Vd), _ = bf16_pair(Q, K, V)
    c64 = torch.zeros((B, Hq, -(-N // Bq)), dtype=torch.int32, device="cuda")
    c128 = torch.zeros_like(c64)
    O64 = _lib.bsfa_prefill(Qd, Kd, Vd, block_q=Bq, gate_mode="dense", kept_counts=c64)
    O128 = _lib.bsfa_prefill(Qd, Kd, Vd, block_q=Bq, block_k=128, gate_mode="dense",
                             kept_counts=c128)
    torch.cuda.synchronize()
    assert torch.equal(O64, O128)
    for i in range(c64.shape[2]):
        assert (c128[:, :, i] == oracle.key_block_range(i, N, Bq, 128)[0]).all()
        assert (c64[:, :, i] == oracle.key_block_range(i, N, Bq, 64)[0]).all()


@pytest.mark.parametrize("name", ["llama_like_ragged", "g8"])
def test_bk128_calibration_kernel_matches_oracle(name):
    B, N, Hq, Hkv, d, Bq = SHAPES[name]
    Q, K, _ = _mid_inputs(name, 24)
    (Qd, Kd), (Qh, Kh) = bf16_pair(Q, K)
    budgets = [1, 2, 3]
    kth = _lib.bsfa_calibrate_blockmax(Qd, Kd, budgets, block_q=Bq, block_k=128)
    torch.cuda.synchronize()
    kth = kth.cpu().numpy()
    sm = oracle.off_diagonal_block_maxima(Qh, Kh, block_q=Bq, block_k=128)
    for kk, k in enumerate(budgets):
        for i in range(sm.shape[2]):
            n_off = oracle.key_block_range(i, N, Bq, 128)[0]
            for h in range(Hq):
                ref = oracle.kth_highest(sm[0, h, i], n_off, k)
                got = kth[kk, 0, h, i]
                assert got == ref if math.isinf(ref) else abs(got - ref) <= 1e-3, (k, h, i)


# ---------------------------------------------------------------------------------------------
# Full-size workloads: the whole call on the device, the oracle on sampled query blocks
# ---------------------------------------------------------------------------------------------
def _sampled_blocks(nqb, k, extra=()):
    s = {0, 1, max(0, k // 2 - 1), k // 2, nqb // 4, nqb // 2 - 1, nqb // 2, 3 * nqb // 4, nqb - 1}
    s.update(extra)
    return sorted(x for x in s if 0 <= x < nqb)


def _full(config, n=None):
    Q, K, V = synth.make_inputs(config, 0, n=n)
    (Qd, Kd, Vd), (Qh, Kh, Vh) = bf16_pair(Q, K, V)
    return Qd, Kd, Vd, Qh, Kh, Vh


def _full_check(config, mode, slices=(0,), log_lambdas=(-math.inf,), blocks=None):
    c = synth.CONFIGS[config]
    Qd, Kd, Vd, Qh, Kh, Vh = _full(config)
    nqb = -(-c["n"] // c["block_q"])
    tab = golden_table(config) if mode == "absolute" else None
    for sl in slices:
        for ll in log_lambdas:
            k = tab.budgets[sl] if tab is not None else 0
            qbs = blocks if blocks is not None else _sampled_blocks(nqb, k)
            dev = run_device(Qd, Kd, Vd, block_q=c["block_q"], mode=mode, table=tab,
                             budget_slice=sl, log_lambda=ll)
            check_parity(dev, Qh, Kh, Vh, block_q=c["block_q"], mode=mode, table=tab,
                         budget_slice=sl, log_lambda=ll, query_blocks=qbs)
            n_off = sum(oracle.key_block_range(i, c["n"], c["block_q"], 64)[0]
                        for i in range(nqb))
            print(f"{config} {mode} slice={sl} loglam={ll:.3f}: kept fraction "
                  f"{dev['total'] / (c['heads_q'] * n_off):.4f}", flush=True)


def test_full_llama_16k_k32():
    _full_check("llama_16k", "absolute")


def test_full_llama_32k_budget_sweep():
    _full_check("llama_32k_sweep", "absolute", slices=(0, 1, 2))


def test_full_llama_128k_k64_reuses_last_threshold():
    # 511 is the last calibrated query block (64K), 512 the first that reuses its threshold
    _full_check("llama_128k", "absolute", blocks=[0, 31, 32, 511, 512, 1023])


def test_full_llama_256k_largest_tensors():
    # the 128K workload's shape at 256K tokens: Q holds 2^30 elements (2 GiB), so every global
    # offset must be formed in 64 bits, and the last query block walks 4094 key tiles (64 mask
    # words). The 128K table (calibrated at 64K) serves unchanged: rows past its last column
    # reuse it, as at 128K.
    c = synth.CONFIGS["llama_128k"]
    n = 2 * c["n"]
    print(f"case llama_128k shape at n={n}", flush=True)
    Qd, Kd, Vd, Qh, Kh, Vh = _full("llama_128k", n=n)
    assert Qd.numel() == 1 << 30
    tab = golden_table("llama_128k")
    nqb = n // c["block_q"]
    dev = run_device(Qd, Kd, Vd, block_q=c["block_q"], mode="absolute", table=tab,
                     budget_slice=0)
    check_parity(dev, Qh, Kh, Vh, block_q=c["block_q"], mode="absolute", table=tab,
                 budget_slice=0, query_blocks=[0, nqb // 2, nqb - 1])


def test_full_llama_64k_relative():
    _full_check("llama_64k_relative", "relative",
                log_lambdas=(math.log(1e-4), math.log(1e-3), math.log(1e-2)),
                blocks=[0, 1, 128, 255, 511])
