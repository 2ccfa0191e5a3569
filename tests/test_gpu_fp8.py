"""GPU parity of the FP8 (E4M3) gate: the HIP path through the C ABI against the CPU oracle
with gate_dtype "fp8", on the same seeded inputs.

Bar: the FP8 copies of Q and K (codes and scales) bit-exact against the oracle's quantisation
(both round in fp32); the sweep's block statistics within 1e-5 relative of the oracle's; keep
decisions bit-exact outside the 1e-2 near-tie band; output max-abs <= 1e-2, mean-abs <= 1e-3.
Identities: on inputs whose FP8 copies are exact, the FP8 gate keeps bitwise what the bf16
gate keeps and the outputs are bitwise equal; packed and paged variable-length batches are
bitwise one call per sequence.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_long_amd import _lib, synth
from gpu_util import (MAX_ABS, MEAN_ABS, absolute_parity, bf16_pair, make_table, pages_of,
                      quantile_table, varlen_batch)

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


def _r256(x):
    return -(-x // 256) * 256


@pytest.mark.parametrize("B,N,Hq,Hkv,d", [(1, 1000, 8, 2, 128), (2, 333, 4, 2, 64)])
def test_fp8_copies_match_the_oracle_bitwise(B, N, Hq, Hkv, d):
    # the workspace of an FP8 gate: masks, then q8 [B][N][Hq][d], its scales [B][Hq][N],
    # k8 [B][N][Hkv][d], its scales [B][Hkv][ceil(N / 64)] and a ticket counter, each on a
    # 256-byte boundary
    Bq = 128 if d == 128 else 64
    Q, K, _ = _inputs(50, N, Hq, Hkv, d, B)
    (Qd, Kd), (Qh, Kh) = bf16_pair(Q, K)
    T = np.zeros((1, Hq, 1), np.float32)
    dtab = make_table(T, Bq, d, [1]).to_device("cuda")
    nbytes = _lib.bsfa_prefill_workspace_bytes(Qd, Kd, block_q=Bq, gate_dtype="fp8")
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    _lib.bsfa_gate_masks(Qd, Kd, dtab, 0, buf, block_q=Bq, gate_dtype="fp8")
    torch.cuda.synchronize()
    w = buf.cpu().numpy()
    nqb, nt = -(-N // Bq), -(-N // 64)
    off = _r256(B * Hq * nqb * (-(-nt // 64)) * 8)
    parts = []
    for size in (B * N * Hq * d, B * Hq * N * 4, B * N * Hkv * d, B * Hkv * nt * 4):
        parts.append(w[off:off + size])
        off += _r256(size)
    assert off + 256 == nbytes     # then the walk's 256-byte ticket counter
    dec = lambda u8: torch.from_numpy(u8.copy()).view(torch.float8_e4m3fn).float().numpy()
    q8, qs = oracle.quantize_q_rows(Qh)
    k8, ks = oracle.quantize_k_tiles(Kh)
    np.testing.assert_array_equal(dec(parts[0]).reshape(B, N, Hq, d), q8)
    np.testing.assert_array_equal(parts[1].view(np.float32).reshape(B, Hq, N),
                                  qs.transpose(0, 2, 1))
    np.testing.assert_array_equal(dec(parts[2]).reshape(B, N, Hkv, d), k8)
    np.testing.assert_array_equal(parts[3].view(np.float32).reshape(B, Hkv, nt),
                                  ks.transpose(0, 2, 1))


CASES = {   # name: (B, N, P, Hq, Hkv, d, Bq, Bk, query blocks checked or None for all)
    "llama_like_ragged": (1, 1000, 0, 8, 2, 128, 128, 64, None),
    "d64_bq64_g2_batch2": (2, 333, 0, 4, 2, 64, 64, 64, None),
    "d128_bq64_g4": (1, 700, 0, 8, 2, 128, 64, 64, None),
    "g8": (1, 384, 0, 16, 2, 128, 128, 64, None),
    "d64_bq128_g1": (1, 515, 0, 2, 2, 64, 128, 64, None),
    "prefix_256": (1, 744, 256, 8, 2, 128, 128, 64, None),
    "bk128_ragged": (1, 1000, 0, 8, 2, 128, 128, 128, None),
    "long_4k": (1, 4600, 0, 2, 1, 128, 128, 64, [0, 20, 34, 35]),
    # two tiles per barrier (four heads per KV group, Bq = 128) after a prefix, up to 200
    # tiles: past the third 64-tile slot of K scales
    "g4_prefix128_12k": (1, 12800, 128, 4, 1, 128, 128, 64, [0, 1, 50, 99]),
    "d64_g4_prefix256": (1, 900, 256, 8, 2, 64, 128, 64, None),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fp8_gate_parity(name):
    B, N, P, Hq, Hkv, d, Bq, Bk, qb = CASES[name]
    print(f"case {name}", flush=True)
    Q, K, V = _inputs(51, N + P, Hq, Hkv, d, B)
    Q = Q[:, P:]
    (Qd, Kd, Vd), (Qh, Kh, Vh) = bf16_pair(Q, K, V)
    tab = quantile_table(Qh, Kh, Bq, Bk)
    for sl in (0, 1):
        absolute_parity(Qd, Kd, Vd, Qh, Kh, Vh, Bq=Bq, Bk=Bk, tab=tab, sl=sl, query_blocks=qb,
                        gate_dtype="fp8")


@pytest.mark.parametrize("name", ["llama_like_ragged", "bk128_ragged"])
def test_fp8_gate_with_mean_correction_parity(name):
    B, N, P, Hq, Hkv, d, Bq, Bk, qb = CASES[name]
    Q, K, V = _inputs(52, N + P, Hq, Hkv, d, B)
    (Qd, Kd, Vd), (Qh, Kh, Vh) = bf16_pair(Q, K, V)
    tab = quantile_table(Qh, Kh, Bq, Bk)
    absolute_parity(Qd, Kd, Vd, Qh, Kh, Vh, Bq=Bq, Bk=Bk, tab=tab, query_blocks=qb,
                    gate_dtype="fp8", mean_correction=True)


def _representable(seed, N, Hq, Hkv, d):
    """Q rows and K tiles whose E4M3 copies are exact (E4M3 values times a power of two, one
    element per row / tile at +-448 times that power): bf16-exact too."""
    rng = np.random.default_rng(seed)
    grid = np.array(sorted({2.0 ** e * (1 + m / 8) for e in range(-6, 9) for m in range(8)
                            if not (e == 8 and m == 7)}))
    def draw(shape):
        return (rng.choice(grid[40:], size=shape) * rng.choice([-1.0, 1.0], size=shape))
    Q = draw((1, N, Hq, d))
    Q[..., 0] = 448.0
    Q *= 2.0 ** rng.integers(-9, -5, size=(1, N, Hq, 1))
    K = draw((1, N, Hkv, d))
    for t in range(-(-N // 64)):
        K[:, t * 64, :, 0] = -448.0
        K[:, t * 64:(t + 1) * 64] *= 2.0 ** rng.integers(-9, -5, size=(1, 1, Hkv, 1))
    V = rng.standard_normal((1, N, Hkv, d))
    return (torch.from_numpy(x.astype(np.float32)) for x in (Q, K, V))


def test_fp8_gate_is_the_bf16_gate_on_representable_inputs():
    N, Hq, Hkv, d, Bq = 1000, 8, 2, 128, 128
    Q, K, V = _representable(53, N, Hq, Hkv, d)
    (Qd, Kd, Vd), (Qh, Kh, _) = bf16_pair(Q, K, V)
    assert torch.equal(Qd.float().cpu(), Q) and torch.equal(Kd.float().cpu(), K)
    tab = quantile_table(Qh, Kh, Bq, 64)
    dtab = tab.to_device("cuda")
    m8 = _lib.bsfa_gate_masks(Qd, Kd, dtab, 0, block_q=Bq, gate_dtype="fp8")
    m16 = _lib.bsfa_gate_masks(Qd, Kd, dtab, 0, block_q=Bq)
    kw = dict(block_q=Bq, gate_mode="absolute", table=dtab, out_dtype=torch.float32)
    O8 = _lib.bsfa_prefill(Qd, Kd, Vd, gate_dtype="fp8", **kw)
    O16 = _lib.bsfa_prefill(Qd, Kd, Vd, **kw)
    torch.cuda.synchronize()
    assert torch.equal(m8, m16)
    assert torch.equal(O8, O16)


@pytest.mark.parametrize("Bk", [64, 128])
def test_fp8_varlen_and_paged_equal_one_call_per_sequence_bitwise(Bk):
    Hq, Hkv, d, Bq = 8, 2, 128, 128
    nq, nk = [1000, 0, 300, 128, 517], [1000, 0, 556, 256, 773]
    Q, K, V, cu_q, cu_k = varlen_batch(54, Hq, Hkv, d, nq, nk)
    (Qd, Kd, Vd), _ = bf16_pair(Q, K, V)
    T = np.random.default_rng(6).uniform(5.0, 6.5, (1, Hq, 16)).astype(np.float32)
    dtab = make_table(T, Bq, d, [1], block_k=Bk).to_device("cuda")
    kw = dict(block_q=Bq, block_k=Bk, gate_mode="absolute", table=dtab, out_dtype=torch.float32,
              gate_dtype="fp8")
    cq, ck = torch.tensor(cu_q, device="cuda"), torch.tensor(cu_k, device="cuda")
    nb = len(nq)
    c1 = torch.full((nb, Hq, -(-max(nq) // Bq)), -7, dtype=torch.int32, device="cuda")
    Ov = _lib.bsfa_prefill_varlen(Qd, Kd, Vd, cq, ck, max(nq), max(nk), kept_counts=c1, **kw)
    Kp, tbl = pages_of(Kd, cu_k, 128, 10)
    Vp, _ = pages_of(Vd, cu_k, 128, 10)
    lens = torch.tensor(np.diff(cu_k), dtype=torch.int32, device="cuda")
    c2 = torch.full_like(c1, -7)
    Op = _lib.bsfa_prefill_paged(Qd, Kp, Vp, cq, lens, tbl, max(nq), max(nk), kept_counts=c2, **kw)
    torch.cuda.synchronize()
    assert torch.equal(Ov, Op) and torch.equal(c1, c2)
    assert (c1 >= 0).any()
    for b in range(nb):
        if nq[b] == 0:
            continue
        q = Qd[cu_q[b]:cu_q[b + 1]][None]
        k = Kd[cu_k[b]:cu_k[b + 1]][None]
        v = Vd[cu_k[b]:cu_k[b + 1]][None]
        O1 = _lib.bsfa_prefill(q, k, v, **kw)
        torch.cuda.synchronize()
        assert torch.equal(O1[0], Ov[cu_q[b]:cu_q[b + 1]]), b


def test_fp8_varlen_matches_oracle():
    Hq, Hkv, d, Bq = 4, 2, 64, 64
    nq, nk = [200, 333, 64], [328, 333, 192]
    Q, K, V, cu_q, cu_k = varlen_batch(55, Hq, Hkv, d, nq, nk)
    (Qd, Kd, Vd), (Qh, Kh, Vh) = bf16_pair(Q, K, V)
    T = np.full((1, Hq, 8), 5.3, np.float32)
    tab = make_table(T, Bq, d, [1])
    dtab = tab.to_device("cuda")
    O = _lib.bsfa_prefill_varlen(Qd, Kd, Vd, torch.tensor(cu_q, device="cuda"),
                                 torch.tensor(cu_k, device="cuda"), max(nq), max(nk), block_q=Bq,
                                 gate_mode="absolute", table=dtab, out_dtype=torch.float32,
                                 gate_dtype="fp8")
    torch.cuda.synchronize()
    # per-sequence device decisions (one-sequence gate-mask calls) for the near-tie rule
    nqb, nkb = -(-max(nq) // Bq), -(-max(nk) // 64)
    keep = np.zeros((len(nq), Hq, nqb, nkb), bool)
    pruned = 0
    for b in range(len(nq)):
        q, k = Qd[cu_q[b]:cu_q[b + 1]][None], Kd[cu_k[b]:cu_k[b + 1]][None]
        mask = _lib.bsfa_gate_masks(q, k, dtab, 0, block_q=Bq, gate_dtype="fp8")
        torch.cuda.synchronize()
        bits = np.unpackbits(np.ascontiguousarray(mask.cpu().numpy()).view(np.uint8), axis=-1,
                             bitorder="little").astype(bool)
        for i in range(-(-nq[b] // Bq)):
            n_off = oracle.key_block_range(i, nq[b], Bq, 64, nk[b] - nq[b])[0]
            keep[b, :, i, :n_off] = bits[0, :, i, :n_off]
            pruned += int((~bits[0, :, i, :n_off]).sum())
    assert pruned > 0
    r = oracle.oracle_prefill_varlen(Qh, Kh, Vh, cu_q, cu_k, block_q=Bq, block_k=64,
                                     mode="absolute", table=T, gate_dtype="fp8",
                                     forced_keep=keep, band=1e-2)
    err = np.abs(O.cpu().numpy() - r.out)
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (err.max(), err.mean())


@pytest.mark.parametrize("Bk", [64, 128])
def test_fp8_calibration_matches_oracle(Bk):
    # thresholds for an FP8 gate are calibrated on its own scores: the k-th highest FP8 block
    # maximum per (b, h, i)
    B, N, Hq, Hkv, d, Bq = 1, 1000, 8, 2, 128, 128
    Q, K, _ = _inputs(56, N, Hq, Hkv, d)
    (Qd, Kd), (Qh, Kh) = bf16_pair(Q, K)
    budgets = [1, 2, 3, 5]
    kth = _lib.bsfa_calibrate_blockmax(Qd, Kd, budgets, block_q=Bq, block_k=Bk, gate_dtype="fp8")
    torch.cuda.synchronize()
    kth = kth.cpu().numpy()
    sm = oracle.off_diagonal_block_maxima(Qh, Kh, block_q=Bq, block_k=Bk, gate_dtype="fp8")
    for kk, k in enumerate(budgets):
        for h in range(Hq):
            for i in range(-(-N // Bq)):
                n_off = oracle.key_block_range(i, N, Bq, Bk)[0]
                ref = oracle.kth_highest(sm[0, h, i], n_off, k)
                got = kth[kk, 0, h, i]
                if math.isinf(ref):
                    assert got == ref
                else:
                    assert abs(got - ref) <= 1e-3, (k, h, i, got, ref)


def test_fp8_zero_rows_and_tiles():
    # an all-zero Q row or K tile has codes 0 and scale 0: its FP8 scores are exactly 0
    B, N, Hq, Hkv, d, Bq = 1, 700, 4, 2, 128, 128
    Q, K, V = _inputs(57, N, Hq, Hkv, d)
    Q[0, 100:180, 1] = 0.0          # rows of head 1 (a whole query block and more)
    K[0, 128:192, 0] = 0.0          # key tile 2 of KV head 0
    K[0, 320:384, 1] = 0.0          # key tile 5 of KV head 1
    (Qd, Kd, Vd), (Qh, Kh, Vh) = bf16_pair(Q, K, V)
    q8, qs = oracle.quantize_q_rows(Qh)
    assert (qs[0, 100:180, 1] == 0).all()
    tab = quantile_table(Qh, Kh, Bq, 64)
    absolute_parity(Qd, Kd, Vd, Qh, Kh, Vh, Bq=Bq, Bk=64, tab=tab, gate_dtype="fp8")


def test_fp8_minus_inf_threshold_is_bitwise_the_bf16_call():
    # nothing to decide: the FP8 copies are made but no block is dropped
    N, Hq, Hkv, d, Bq = 1000, 8, 2, 128, 128
    Q, K, V = _inputs(58, N, Hq, Hkv, d)
    (Qd, Kd, Vd), _ = bf16_pair(Q, K, V)
    dtab = make_table(np.full((1, Hq, 8), -np.inf, np.float32), Bq, d, [1]).to_device("cuda")
    kw = dict(block_q=Bq, gate_mode="absolute", table=dtab, out_dtype=torch.float32)
    a = _lib.bsfa_prefill(Qd, Kd, Vd, gate_dtype="fp8", **kw)
    b = _lib.bsfa_prefill(Qd, Kd, Vd, **kw)
    c = _lib.bsfa_prefill(Qd, Kd, Vd, block_q=Bq, gate_mode="dense", out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


@pytest.mark.parametrize("gate_dtype", ["bf16", "fp8"])
def test_calibrate_table_matches_the_oracle_calibration(gate_dtype):
    # the GPU tool (k-th highest per sample on the device, mean over samples on the host) against
    # oracle.calibrate on the same two samples
    from block_sparse_long_amd.table import calibrate_table
    N, Hq, Hkv, d, Bq = 700, 4, 2, 128, 128
    host, dev = [], []
    for seed in (60, 61):
        Q, K, _ = _inputs(seed, N, Hq, Hkv, d)
        (Qd, Kd), (Qh, Kh) = bf16_pair(Q, K)
        host.append((Qh, Kh))
        dev.append((Qd, Kd))
    budgets = [1, 3]
    tab = calibrate_table(dev, budgets=budgets, block_q=Bq, gate_dtype=gate_dtype)
    ref = oracle.calibrate(host, block_q=Bq, block_k=64, budgets=budgets,
                           scale=float(np.float32(1 / math.sqrt(d))), gate_dtype=gate_dtype)
    assert tab.T.shape == ref.shape
    inf = np.isinf(ref)
    np.testing.assert_array_equal(tab.T[inf], ref[inf])
    np.testing.assert_allclose(tab.T[~inf], ref[~inf], rtol=0, atol=1e-3)


def test_calibration_cli_reproduces_the_oracle_table(tmp_path):
    # the GPU calibration command on the tiny workload's calibration seeds against the stored
    # oracle-calibrated table of the same workload
    import os
    from block_sparse_long_amd import calibrate
    from block_sparse_long_amd.table import ThresholdTable
    out = str(tmp_path / "t.bin")
    calibrate.main(["--config", "tiny_1k", "--seeds", "1-4", "--budgets", "4", "--out", out])
    got = ThresholdTable.load(out)
    ref = ThresholdTable.load(os.path.join(os.path.dirname(__file__), "golden",
                                           "thresholds_tiny_1k.bin"))
    assert got.T.shape == ref.T.shape and got.budgets == ref.budgets
    inf = np.isinf(ref.T)
    np.testing.assert_array_equal(got.T[inf], ref.T[inf])
    np.testing.assert_allclose(got.T[~inf], ref.T[~inf], rtol=0, atol=1e-3)


def test_calibrate_table_at_workload_size_reproduces_the_stored_16k_table():
    # the GPU calibration tool on the 16K workload's 8 calibration seeds (32 query heads, 128
    # query blocks, k = 32) against the table the oracle calibrated from the same seeds
    import os
    from block_sparse_long_amd.table import ThresholdTable, calibrate_table
    c = synth.CONFIGS["llama_16k"]
    ref = ThresholdTable.load(os.path.join(os.path.dirname(__file__), "golden",
                                           "thresholds_llama_16k.bin"))
    samples = []
    for seed in c["calib_seeds"]:
        print(f"case llama_16k calibration seed {seed}", flush=True)
        Q, K, _ = synth.make_inputs("llama_16k", seed)
        samples.append(tuple(x.to(torch.bfloat16).cuda() for x in (Q, K)))
        del Q, K
    got = calibrate_table(samples, budgets=c["budgets"], block_q=c["block_q"],
                          block_k=c["block_k"])
    assert got.T.shape == ref.T.shape == (1, 32, 128) and got.budgets == ref.budgets
    inf = np.isinf(ref.T)
    np.testing.assert_array_equal(got.T[inf], ref.T[inf])
    np.testing.assert_allclose(got.T[~inf], ref.T[~inf], rtol=0, atol=1e-3)
