"""Full-size parity of the two 128K calls the benchmark times besides the headline: the
absolute gate with FP8 gate scores ("FlashPrefill V2: Block-Sparse Prefill Attention for
Long-Context LLM Serving", FP8 path; thresholds calibrated on FP8 scores) and with mean
correction (the same page, mean correction), each through the call's own two launches (the
gate sweep, then the walk over the kept tiles), on the query blocks
[0, 31, 32, 511, 512, 1023] (the first blocks, the -inf boundary of k = 64, the last calibrated
and the first reused threshold column, the last block).

The oracle computes each sampled query block as a chunk: its 128 query rows after the keys
before them (rows P .. P + 127 of a chunk after a prefix of P = 128 i keys are rows of the
whole prefill, a reading the oracle's own pins fix), so that it quantises and walks only what
that block sees.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from block_sparse_long_amd import _lib, synth
from block_sparse_long_amd.table import ThresholdTable
from gpu_util import BAND, MAX_ABS, MEAN_ABS

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
BLOCKS = [0, 31, 32, 511, 512, 1023]


@pytest.fixture(scope="module")
def inputs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load_library()
    print("case llama_128k inputs", flush=True)
    Q, K, V = synth.make_inputs("llama_128k", 0)
    Qd, Kd, Vd = (x.to(torch.bfloat16).cuda() for x in (Q, K, V))
    del Q, K, V
    return Qd, Kd, Vd


def _gated_call_vs_oracle(Qd, Kd, Vd, table, gate_dtype, mean_correction):
    B, N, Hq, d = Qd.shape
    Bq = 128
    nqb, nkb = N // Bq, N // 64
    dtab = table.to_device("cuda")
    stat = torch.full((B, Hq, nqb, nkb), float("nan"), device="cuda")
    mask = _lib.bsfa_gate_masks(Qd, Kd, dtab, 0, block_q=Bq, debug_block_stat=stat,
                                gate_dtype=gate_dtype)
    counts = torch.full((B, Hq, nqb), -7, dtype=torch.int32, device="cuda")
    O = _lib.bsfa_prefill(Qd, Kd, Vd, block_q=Bq, gate_mode="absolute", table=dtab,
                          kept_counts=counts, out_dtype=torch.float32,
                          mean_correction=mean_correction, gate_dtype=gate_dtype)
    torch.cuda.synchronize()
    counts = counts.cpu().numpy()
    bits = np.unpackbits(np.ascontiguousarray(mask.cpu().numpy()).view(np.uint8), axis=-1,
                         bitorder="little").astype(bool)
    st = stat.cpu().numpy()
    n_pruned = 0
    for i in BLOCKS:
        print(f"  query block {i}", flush=True)
        n_off = oracle.key_block_range(i, N, Bq, 64)[0]
        keep = np.zeros((B, Hq, 1, nkb), bool)
        keep[:, :, 0, :n_off] = bits[:, :, i, :n_off]
        np.testing.assert_array_equal(counts[:, :, i], keep[:, :, 0].sum(-1))
        n_pruned += int((counts[:, :, i] < n_off).sum())
        r0, r1 = i * Bq, (i + 1) * Bq
        Qh = Qd[:, r0:r1].float().cpu().numpy()
        Kh = Kd[:, :r1].float().cpu().numpy()
        Vh = Vd[:, :r1].float().cpu().numpy()
        r = oracle.oracle_prefill(Qh, Kh, Vh, block_q=Bq, block_k=64, mode="absolute",
                                  table=table.T, budget_slice=0, forced_keep=keep, band=BAND,
                                  mean_correction=mean_correction, gate_dtype=gate_dtype)
        mg = r.margin[:, :, 0, :n_off]
        out = np.abs(mg) > BAND
        np.testing.assert_array_equal(r.keep[:, :, 0, :n_off][out], keep[:, :, 0, :n_off][out])
        np.testing.assert_array_equal(r.kept_counts[:, :, 0], counts[:, :, i])
        fin = np.isfinite(r.stat[:, :, 0, :n_off])
        np.testing.assert_allclose(st[:, :, i, :n_off][fin], r.stat[:, :, 0, :n_off][fin],
                                   rtol=1e-5, atol=2e-3)
        got = O[:, r0:r1].cpu().numpy()
        assert np.isfinite(got).all()
        err = np.abs(got - r.out)
        assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (i, err.max(), err.mean())
    assert n_pruned > 0


def test_full_llama_128k_fp8_gate(inputs):
    tab = ThresholdTable.load(os.path.join(GOLDEN, "thresholds_llama_128k_fp8.bin"))
    _gated_call_vs_oracle(*inputs, tab, "fp8", False)


def test_full_llama_128k_mean_correction(inputs):
    tab = ThresholdTable.load(os.path.join(GOLDEN, "thresholds_llama_128k.bin"))
    _gated_call_vs_oracle(*inputs, tab, "bf16", True)
