"""The C ABI without a GPU: libbsfa.so loads, exports every symbol include/bsfa.h declares, and
rejects invalid calls on the host with the documented status before anything is enqueued.

No call here reaches a kernel launch: every call fails validation first (pointers are never
dereferenced on the host).
"""
import ctypes
import math
import os
import re

import numpy as np
import pytest

from block_sparse_long_amd import _lib
from block_sparse_long_amd.table import ThresholdTable

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsfa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libbsfa.so not built (python -m block_sparse_long_amd.build_lib)")

FAKE = 0x10000          # 16-byte aligned stand-in address, never dereferenced on these paths


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(bsfa_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = _lib.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    for s in range(8):
        assert _lib.bsfa_status_string(s)
    assert _lib.bsfa_status_string(99) == "unknown status"
    assert _lib.bsfa_version() >> 16 == _lib.ABI_MAJOR == 3


def problem(B=1, N=256, Hq=4, Hkv=2, d=128, bq=128, bk=64, out=_lib.BSFA_BF16):
    p = _lib.BsfaProblem()
    p.batch, p.seqlen, p.heads_q, p.heads_kv, p.head_dim = B, N, Hq, Hkv, d
    p.block_q, p.block_k = bq, bk
    p.softmax_scale = 0.0
    p.in_dtype, p.out_dtype = _lib.BSFA_BF16, out
    p.q_stride[:] = (N * Hq * d, Hq * d, d)
    p.k_stride[:] = (N * Hkv * d, Hkv * d, d)
    p.v_stride[:] = (N * Hkv * d, Hkv * d, d)
    p.o_stride[:] = (N * Hq * d, Hq * d, d)
    return p


def table(Hq=4, bq=128, bk=64, d=128, scale=None, n_budgets=2, t_len=2, ptr=FAKE):
    t = _lib.BsfaTable()
    t.T = ptr
    t.n_budgets, t.t_len, t.heads_q, t.block_q, t.block_k, t.head_dim = n_budgets, t_len, Hq, bq, bk, d
    t.softmax_scale = 1 / math.sqrt(d) if scale is None else scale
    return t


def call_prefill(p, tbl=None, slice_=0, mode=_lib.BSFA_GATE_DENSE, log_lambda=-math.inf,
                 q=FAKE, k=FAKE, v=FAKE, o=FAKE, counts=None, total=None, dbg=None, ws=None,
                 ws_bytes=0):
    lib = _lib.load_library()
    return lib.bsfa_prefill(ctypes.byref(p), q, k, v, ctypes.byref(tbl) if tbl else None, slice_,
                            mode, log_lambda, o, counts, total, dbg, ws, ws_bytes, None)


@pytest.mark.parametrize("mutate,status", [
    (lambda p: setattr(p, "heads_kv", 3), _lib.BSFA_ERR_SHAPE),
    (lambda p: setattr(p, "head_dim", 96), _lib.BSFA_ERR_SHAPE),
    (lambda p: setattr(p, "block_k", 32), _lib.BSFA_ERR_SHAPE),
    (lambda p: setattr(p, "block_q", 256), _lib.BSFA_ERR_SHAPE),
    (lambda p: setattr(p, "in_dtype", _lib.BSFA_FP32), _lib.BSFA_ERR_DTYPE),
    (lambda p: setattr(p, "out_dtype", 7), _lib.BSFA_ERR_DTYPE),
    (lambda p: setattr(p, "seqlen", -1), _lib.BSFA_ERR_ARG),
    (lambda p: setattr(p, "heads_q", 0), _lib.BSFA_ERR_ARG),
    (lambda p: setattr(p, "softmax_scale", -1.0), _lib.BSFA_ERR_ARG),
    (lambda p: setattr(p, "softmax_scale", float("nan")), _lib.BSFA_ERR_ARG),
    (lambda p: p.q_stride.__setitem__(1, 100), _lib.BSFA_ERR_ALIGN),
    (lambda p: p.o_stride.__setitem__(2, -128), _lib.BSFA_ERR_ARG),
])
def test_problem_validation(mutate, status):
    p = problem()
    mutate(p)
    assert call_prefill(p) == status
    assert _lib.bsfa_last_error() != ""


def test_fp32_output_needs_only_4_element_alignment():
    p = problem(out=_lib.BSFA_FP32)
    p.o_stride[:] = (256 * 4 * 132, 4 * 132, 132)      # 132 floats: 16-byte rows, not 32-byte
    assert call_prefill(p, o=FAKE + 1) == _lib.BSFA_ERR_ALIGN   # misaligned O base


@pytest.mark.parametrize("which", ["q", "k", "v", "o"])
def test_misaligned_or_null_pointers(which):
    p = problem()
    assert call_prefill(p, **{which: FAKE + 8}) == _lib.BSFA_ERR_ALIGN
    assert call_prefill(p, **{which: None}) == _lib.BSFA_ERR_ARG


def test_gate_mode_and_lambda_validation():
    p = problem()
    assert call_prefill(p, mode=3) == _lib.BSFA_ERR_ARG
    assert call_prefill(p, mode=_lib.BSFA_GATE_RELATIVE, log_lambda=float("nan"), q=None) == _lib.BSFA_ERR_ARG
    assert call_prefill(p, mode=_lib.BSFA_GATE_RELATIVE, log_lambda=math.inf, q=None) == _lib.BSFA_ERR_ARG


@pytest.mark.parametrize("tbl,slice_", [
    (None, 0),
    (table(ptr=None), 0),
    (table(ptr=FAKE + 2), 0),
    (table(), 2),
    (table(), -1),
    (table(n_budgets=0), 0),
    (table(t_len=0), 0),
    (table(Hq=8), 0),
    (table(bq=64), 0),
    (table(d=64), 0),
    (table(scale=0.1), 0),
])
def test_table_validation(tbl, slice_):
    status = call_prefill(problem(), tbl=tbl, slice_=slice_, mode=_lib.BSFA_GATE_ABSOLUTE, q=None)
    expect = _lib.BSFA_ERR_ALIGN if (tbl is not None and tbl.T == FAKE + 2) else _lib.BSFA_ERR_TABLE
    assert status == expect


def test_table_checked_before_pointers():
    # the table header is validated against the problem (a threshold is bound to its tile shape)
    assert call_prefill(problem(), tbl=table(bq=64), mode=_lib.BSFA_GATE_ABSOLUTE,
                        q=None) == _lib.BSFA_ERR_TABLE


def test_misaligned_outputs():
    p = problem()
    assert call_prefill(p, counts=FAKE + 2) == _lib.BSFA_ERR_ALIGN
    assert call_prefill(p, total=FAKE + 4) == _lib.BSFA_ERR_ALIGN
    assert call_prefill(p, dbg=FAKE + 1) == _lib.BSFA_ERR_ALIGN


def test_workspace_size_and_validation():
    lib = _lib.load_library()
    p = problem()
    N, bq, bk = p.seqlen, p.block_q, p.block_k
    words = -(-(-(-N // bk)) // 64)
    masks = p.batch * p.heads_q * (-(-N // bq)) * words * 8
    # the masks, then (on a 256-byte boundary) the walk's 256-byte ticket counter
    need = -(-masks // 256) * 256 + 256
    assert lib.bsfa_prefill_workspace_bytes(ctypes.byref(p), _lib.BSFA_GATE_ABSOLUTE) == need
    # dense and the relative gate: a 256-byte ticket counter only
    for mode in (_lib.BSFA_GATE_DENSE, _lib.BSFA_GATE_RELATIVE):
        assert lib.bsfa_prefill_workspace_bytes(ctypes.byref(p), mode) == 256
        assert call_prefill(p, mode=mode, ws=FAKE, ws_bytes=255) == _lib.BSFA_ERR_ARG
        assert "workspace" in _lib.bsfa_last_error()
    assert lib.bsfa_prefill_workspace_bytes(ctypes.byref(p), 7) == 0
    assert lib.bsfa_prefill_workspace_bytes(None, _lib.BSFA_GATE_ABSOLUTE) == 0
    assert lib.bsfa_prefill_workspace_bytes(None, _lib.BSFA_GATE_DENSE) == 0
    # 65 key tiles need two mask words per query block
    p2 = problem(N=65 * 64)
    assert lib.bsfa_prefill_workspace_bytes(ctypes.byref(p2), _lib.BSFA_GATE_ABSOLUTE) == \
        -(-(p2.batch * p2.heads_q * (-(-p2.seqlen // p2.block_q)) * 2 * 8) // 256) * 256 + 256
    abs_call = dict(tbl=table(t_len=-(-N // bq)), mode=_lib.BSFA_GATE_ABSOLUTE)
    assert call_prefill(p, ws=FAKE + 4, ws_bytes=need, **abs_call) == _lib.BSFA_ERR_ALIGN
    assert call_prefill(p, ws=FAKE, ws_bytes=need - 8, **abs_call) == _lib.BSFA_ERR_ARG
    assert "workspace" in _lib.bsfa_last_error()


def call_masks(p, tbl, slice_=0, q=FAKE, k=FAKE, mask=FAKE, mask_bytes=1 << 20, dbg=None):
    lib = _lib.load_library()
    return lib.bsfa_gate_masks(ctypes.byref(p), q, k, ctypes.byref(tbl) if tbl else None, slice_,
                               mask, mask_bytes, dbg, None)


def test_gate_masks_validation():
    p = problem()
    # the masks alone: B * Hq * nqb * words * 8 bytes
    need = p.batch * p.heads_q * (-(-p.seqlen // p.block_q)) * (-(-(-(-p.seqlen // 64)) // 64)) * 8
    assert call_masks(p, None) == _lib.BSFA_ERR_TABLE
    assert call_masks(p, table(bq=64)) == _lib.BSFA_ERR_TABLE
    assert call_masks(p, table(), slice_=2) == _lib.BSFA_ERR_TABLE
    assert call_masks(p, table(), mask=None) == _lib.BSFA_ERR_ARG
    assert call_masks(p, table(), q=None) == _lib.BSFA_ERR_ARG
    assert call_masks(p, table(), mask=FAKE + 4) == _lib.BSFA_ERR_ALIGN
    assert call_masks(p, table(), k=FAKE + 8) == _lib.BSFA_ERR_ALIGN
    assert call_masks(p, table(), dbg=FAKE + 2) == _lib.BSFA_ERR_ALIGN
    assert call_masks(p, table(), mask_bytes=need - 8) == _lib.BSFA_ERR_ARG
    assert call_masks(problem(N=2097152 + 64), table(t_len=1)) == _lib.BSFA_ERR_UNSUPPORTED
    q = problem()
    q.head_dim = 96
    assert call_masks(q, table()) == _lib.BSFA_ERR_SHAPE


def test_kv_seqlen_validation():
    lib = _lib.load_library()
    p = problem()
    p.kv_seqlen = p.seqlen - 1
    assert call_prefill(p) == _lib.BSFA_ERR_ARG
    p.kv_seqlen = -5
    assert call_prefill(p) == _lib.BSFA_ERR_ARG
    # the absolute gate reads thresholds by absolute query block: the prefix sits on the grid
    p.kv_seqlen = p.seqlen + 64
    abs_call = dict(tbl=table(t_len=4), mode=_lib.BSFA_GATE_ABSOLUTE)
    assert call_prefill(p, **abs_call) == _lib.BSFA_ERR_SHAPE
    assert call_masks(p, table(t_len=4)) == _lib.BSFA_ERR_SHAPE
    # calibration takes whole sequences
    arr = (ctypes.c_int32 * 1)(4)
    assert lib.bsfa_calibrate_blockmax(ctypes.byref(p), FAKE, FAKE, arr, 1, FAKE, None, 0,
                                       None) == \
        _lib.BSFA_ERR_UNSUPPORTED
    # the masks cover the keys: 65 key tiles after a prefix need two words per query block
    p.kv_seqlen = 65 * 64
    p.seqlen = 128
    assert lib.bsfa_prefill_workspace_bytes(ctypes.byref(p), _lib.BSFA_GATE_ABSOLUTE) == \
        -(-(p.batch * p.heads_q * 1 * 2 * 8) // 256) * 256 + 256


def test_varlen_validation():
    lib = _lib.load_library()
    p = problem()

    def call(cu_q=FAKE, cu_k=FAKE, **kw):
        return lib.bsfa_prefill_varlen(ctypes.byref(p), FAKE, FAKE, FAKE, cu_q, cu_k, None, 0,
                                       _lib.BSFA_GATE_DENSE, -math.inf, FAKE, None, None, None,
                                       None, 0, None)
    assert call(cu_q=None) == _lib.BSFA_ERR_ARG
    assert call(cu_k=None) == _lib.BSFA_ERR_ARG
    assert call(cu_q=FAKE + 2) == _lib.BSFA_ERR_ALIGN
    assert lib.bsfa_prefill_varlen(None, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 0, -math.inf,
                                   FAKE, None, None, None, None, 0, None) == _lib.BSFA_ERR_ARG


def test_paged_validation():
    lib = _lib.load_library()
    p = problem()

    def call(page=64, stride=4, cu=FAKE, lens=FAKE, bt=FAKE):
        return lib.bsfa_prefill_paged(ctypes.byref(p), FAKE, FAKE, FAKE, cu, lens, bt, stride,
                                      page, None, 0, _lib.BSFA_GATE_DENSE, -math.inf, FAKE, None,
                                      None, None, None, 0, None)
    assert call(page=96) == _lib.BSFA_ERR_SHAPE         # pages hold whole 64-key tiles
    assert call(page=0) == _lib.BSFA_ERR_SHAPE
    assert call(stride=3) == _lib.BSFA_ERR_ARG          # 256 keys need 4 pages of 64
    assert call(lens=None) == _lib.BSFA_ERR_ARG
    assert call(bt=None) == _lib.BSFA_ERR_ARG
    assert call(bt=FAKE + 2) == _lib.BSFA_ERR_ALIGN


def test_wide_key_blocks():
    # 128 x 128 tiles: dense and the absolute gate's two launches; the votes inside the loop
    # and the per-tile statistic dump are not built for them
    p = problem(bk=128)
    assert call_prefill(p, mode=_lib.BSFA_GATE_RELATIVE, q=None) == _lib.BSFA_ERR_UNSUPPORTED
    abs_call = dict(tbl=table(bk=128), mode=_lib.BSFA_GATE_ABSOLUTE)
    assert call_prefill(p, **abs_call) == _lib.BSFA_ERR_UNSUPPORTED          # no workspace
    assert call_prefill(p, dbg=FAKE, ws=FAKE, ws_bytes=1 << 20, **abs_call) == \
        _lib.BSFA_ERR_UNSUPPORTED
    assert call_prefill(problem(bq=64, bk=128)) == _lib.BSFA_ERR_SHAPE
    # the workspace keeps one bit per 64-key tile
    lib = _lib.load_library()
    assert lib.bsfa_prefill_workspace_bytes(ctypes.byref(problem(N=65 * 64, bk=128)),
                                            _lib.BSFA_GATE_ABSOLUTE) == \
        lib.bsfa_prefill_workspace_bytes(ctypes.byref(problem(N=65 * 64)), _lib.BSFA_GATE_ABSOLUTE)


def test_absolute_gate_length_limit():
    p = problem(N=2097152 + 64)
    st = call_prefill(p, tbl=table(t_len=1), mode=_lib.BSFA_GATE_ABSOLUTE)
    assert st == _lib.BSFA_ERR_UNSUPPORTED


def call_calib(p, budgets, q=FAKE, k=FAKE, out=FAKE, ws=None, ws_bytes=0):
    lib = _lib.load_library()
    arr = (ctypes.c_int32 * max(1, len(budgets)))(*budgets)
    return lib.bsfa_calibrate_blockmax(ctypes.byref(p), q, k, arr if budgets is not None else None,
                                       len(budgets), out, ws, ws_bytes, None)


def test_calibrate_validation():
    assert call_calib(problem(), []) == _lib.BSFA_ERR_ARG
    assert call_calib(problem(), [0]) == _lib.BSFA_ERR_ARG
    assert call_calib(problem(), list(range(1, 18))) == _lib.BSFA_ERR_ARG
    assert call_calib(problem(N=262144 + 64), [4]) == _lib.BSFA_ERR_UNSUPPORTED
    assert call_calib(problem(), [4], q=FAKE + 4) == _lib.BSFA_ERR_ALIGN
    assert call_calib(problem(), [4], out=None) == _lib.BSFA_ERR_ARG
    p = problem()
    p.head_dim = 80
    assert call_calib(p, [4]) == _lib.BSFA_ERR_SHAPE


def test_table_file_round_trip(tmp_path):
    T = np.array([[[-np.inf, 1.5, 2.25]], [[0.0, np.inf, -3.0]]], dtype=np.float32)
    t = ThresholdTable(T=T, budgets=[4, 16], block_q=64, block_k=64, head_dim=64,
                       softmax_scale=0.125, calib_seqlen=192, seeds=[1, 2], generator="x")
    path = tmp_path / "t.bin"
    t.save(str(path))
    u = ThresholdTable.load(str(path))
    np.testing.assert_array_equal(u.T, T)
    assert u.budgets == [4, 16] and u.slice_index(16) == 1 and u.t_len == 3 and u.heads_q == 1
    assert (u.block_q, u.block_k, u.head_dim, u.softmax_scale) == (64, 64, 64, 0.125)


def test_stored_tables_load(golden_dir):
    for f in os.listdir(golden_dir):
        if f.startswith("thresholds_") and f.endswith(".bin"):
            t = ThresholdTable.load(os.path.join(golden_dir, f))
            assert t.T.dtype == np.float32 and len(t.budgets) == t.T.shape[0]
            # -inf exactly where a query block has fewer than k off-diagonal candidates
            for kk, k in enumerate(t.budgets):
                for i in range(t.t_len):
                    n_off = (i * t.block_q) // t.block_k
                    assert np.isneginf(t.T[kk, :, i]).all() == (n_off < k)


def test_mean_correction_workspace_and_validation():
    lib = _lib.load_library()
    p = problem(N=1000)
    r256 = lambda x: -(-x // 256) * 256
    masks = p.batch * p.heads_q * (-(-1000 // p.block_q)) * 1 * 8
    assert lib.bsfa_prefill_workspace_bytes(ctypes.byref(p), _lib.BSFA_GATE_ABSOLUTE) == \
        r256(masks) + 256
    p.mean_correction = 1
    need = lib.bsfa_prefill_workspace_bytes(ctypes.byref(p), _lib.BSFA_GATE_ABSOLUTE)
    # masks, then three [B][Hkv][floor(Nk / Bk)][d] bf16 arrays and the ticket counter, each
    # on a 256-byte boundary
    part = p.batch * p.heads_kv * (1000 // 64) * p.head_dim * 2
    assert need == r256(masks) + 3 * r256(part) + 256
    for mode in (_lib.BSFA_GATE_DENSE, _lib.BSFA_GATE_RELATIVE):
        assert lib.bsfa_prefill_workspace_bytes(ctypes.byref(p), mode) == 256
    abs_call = dict(tbl=table(t_len=8), mode=_lib.BSFA_GATE_ABSOLUTE)
    # the block means live in the workspace: none, or an 8-byte-aligned one, is refused
    assert call_prefill(p, **abs_call) == _lib.BSFA_ERR_UNSUPPORTED
    assert "workspace" in _lib.bsfa_last_error()
    assert call_prefill(p, ws=FAKE + 8, ws_bytes=need, **abs_call) == _lib.BSFA_ERR_ALIGN
    assert call_prefill(p, ws=FAKE, ws_bytes=need - 1, **abs_call) == _lib.BSFA_ERR_ARG
    # the relative gate's decisions depend on the running max: no stand-ins there
    assert call_prefill(p, mode=_lib.BSFA_GATE_RELATIVE, log_lambda=-1.0) == \
        _lib.BSFA_ERR_UNSUPPORTED
    assert "absolute" in _lib.bsfa_last_error()
    p.mean_correction = 2
    assert call_prefill(p) == _lib.BSFA_ERR_ARG
    # the gate masks need only the masks
    p.mean_correction = 1
    assert call_masks(p, table(t_len=8), mask_bytes=masks - 8) == _lib.BSFA_ERR_ARG
    assert f"required {masks}" in _lib.bsfa_last_error()


def test_fp8_gate_workspace_and_validation():
    lib = _lib.load_library()
    p = problem(N=1000)
    r256 = lambda x: -(-x // 256) * 256
    B, N, Hq, Hkv, d = p.batch, 1000, p.heads_q, p.heads_kv, p.head_dim
    masks = B * Hq * (-(-N // p.block_q)) * 1 * 8
    p.gate_dtype = _lib.BSFA_FP8_E4M3
    need = lib.bsfa_prefill_workspace_bytes(ctypes.byref(p), _lib.BSFA_GATE_ABSOLUTE)
    parts = [B * N * Hq * d, B * Hq * N * 4, B * N * Hkv * d, B * Hkv * (-(-N // 64)) * 4]
    copies = r256(masks) + sum(r256(x) for x in parts)     # what bsfa_gate_masks writes
    assert need == copies + 256                              # then the ticket counter
    # with mean correction the block means follow the FP8 copies
    p.mean_correction = 1
    both = lib.bsfa_prefill_workspace_bytes(ctypes.byref(p), _lib.BSFA_GATE_ABSOLUTE)
    assert both == need + 3 * r256(B * Hkv * (N // 64) * d * 2)
    p.mean_correction = 0
    for mode in (_lib.BSFA_GATE_DENSE, _lib.BSFA_GATE_RELATIVE):
        assert lib.bsfa_prefill_workspace_bytes(ctypes.byref(p), mode) == 256
    abs_call = dict(tbl=table(t_len=8), mode=_lib.BSFA_GATE_ABSOLUTE)
    assert call_prefill(p, **abs_call) == _lib.BSFA_ERR_UNSUPPORTED
    assert "workspace" in _lib.bsfa_last_error()
    assert call_prefill(p, ws=FAKE + 8, ws_bytes=need, **abs_call) == _lib.BSFA_ERR_ALIGN
    assert call_prefill(p, ws=FAKE, ws_bytes=need - 1, **abs_call) == _lib.BSFA_ERR_ARG
    assert call_prefill(p, mode=_lib.BSFA_GATE_RELATIVE, log_lambda=-1.0) == \
        _lib.BSFA_ERR_UNSUPPORTED
    p.gate_dtype = _lib.BSFA_FP32
    assert call_prefill(p, ws=FAKE, ws_bytes=need, **abs_call) == _lib.BSFA_ERR_DTYPE
    # the gate masks need the masks and the FP8 copies, 16-byte aligned
    p.gate_dtype = _lib.BSFA_FP8_E4M3
    assert call_masks(p, table(t_len=8), mask_bytes=copies - 8) == _lib.BSFA_ERR_ARG
    assert f"required {copies}" in _lib.bsfa_last_error()
    assert call_masks(p, table(t_len=8), mask=FAKE + 8, mask_bytes=need) == _lib.BSFA_ERR_ALIGN
    # FP8 calibration: the FP8 copies and the block maxima live in a workspace
    cw = lib.bsfa_calibrate_workspace_bytes(ctypes.byref(p))
    nqb, nkb = -(-N // p.block_q), -(-N // p.block_k)
    assert cw == copies + B * Hq * nqb * nkb * 4
    assert call_calib(p, [1]) == _lib.BSFA_ERR_ARG
    assert call_calib(p, [1], ws=FAKE, ws_bytes=cw - 4) == _lib.BSFA_ERR_ARG
    assert call_calib(p, [1], ws=FAKE + 8, ws_bytes=cw) == _lib.BSFA_ERR_ALIGN
    p.gate_dtype = _lib.BSFA_BF16
    assert lib.bsfa_calibrate_workspace_bytes(ctypes.byref(p)) == 0


def test_mfma_rate_probe_validation():
    lib = _lib.load_library()
    assert lib.bsfa_mfma_rate_probe(0, 4, FAKE, None) == _lib.BSFA_ERR_ARG
    assert lib.bsfa_mfma_rate_probe(4, 0, FAKE, None) == _lib.BSFA_ERR_ARG
    assert lib.bsfa_mfma_rate_probe(4, 4, None, None) == _lib.BSFA_ERR_ARG
    assert lib.bsfa_mfma_rate_probe(4, 4, FAKE + 2, None) == _lib.BSFA_ERR_ALIGN


def test_binding_refuses_inconsistent_tensors():
    # the kernels size every access from Q's shape: tensors that disagree with it are refused
    # by the binding before the library is called (CPU tensors: nothing reaches a device)
    import torch
    bf = torch.bfloat16
    Q = torch.zeros(1, 256, 4, 128, dtype=bf)
    K = torch.zeros(1, 256, 2, 128, dtype=bf)
    V = torch.zeros(1, 256, 2, 128, dtype=bf)
    bad = [
        dict(K=torch.zeros(2, 256, 2, 128, dtype=bf)),            # batch
        dict(K=torch.zeros(1, 256, 2, 64, dtype=bf)),             # head_dim
        dict(K=torch.zeros(1, 128, 2, 128, dtype=bf), V=torch.zeros(1, 128, 2, 128, dtype=bf)),
        dict(V=torch.zeros(1, 64, 2, 128, dtype=bf)),             # V differs from K
        dict(O=torch.zeros(1, 16, 4, 128, dtype=bf)),             # O differs from Q
    ]
    for kw in bad:
        args = dict(Q=Q, K=K, V=V, O=None)
        args.update(kw)
        with pytest.raises(ValueError):
            _lib.bsfa_prefill(args["Q"], args["K"], args["V"], args["O"], block_q=128)
    # per-block outputs must have the problem's size: [B][Hq][nqb], [B][Hq][nqb][nkb]
    with pytest.raises(ValueError, match="kept_counts"):
        _lib.bsfa_prefill(Q, K, V, block_q=128, kept_counts=torch.zeros(3, dtype=torch.int32))
    with pytest.raises(ValueError, match="debug_block_stat"):
        _lib.bsfa_prefill(Q, K, V, block_q=128, debug_block_stat=torch.zeros(4 * 2 * 3))
    with pytest.raises(ValueError, match="kept_total"):
        _lib.bsfa_prefill(Q, K, V, block_q=128, kept_total=torch.zeros(2, dtype=torch.int64))
    with pytest.raises(ValueError, match="kth_out"):
        _lib.bsfa_calibrate_blockmax(Q, K, [4], torch.zeros(4 * 2 - 1), block_q=128)
    with pytest.raises(ValueError, match="debug_block_stat"):
        _lib.bsfa_gate_masks(Q, K, None, 0, torch.zeros(1, 4, 2, 1, dtype=torch.int64),
                             block_q=128, debug_block_stat=torch.zeros(5))
    # varlen: packed [tokens, heads, dim]; paged: K / V pages of one shape
    cu = torch.tensor([0, 256], dtype=torch.int32)
    with pytest.raises(ValueError):
        _lib.bsfa_prefill_varlen(Q[0], K[0], V[0, :100], cu, cu, 256, 256, block_q=128)
    pages = torch.zeros(4, 64, 2, 128, dtype=bf)
    with pytest.raises(ValueError):
        _lib.bsfa_prefill_paged(Q[0], pages, pages[:3], cu, torch.tensor([256], dtype=torch.int32),
                                torch.zeros(1, 4, dtype=torch.int32), 256, 256, block_q=128)


def test_noalloc_validates_and_refuses_calls_beyond_its_scratch():
    # the static-scratch entry point checks the problem like bsfa_prefill, and refuses a call
    # whose workspace exceeds its 64 MiB array before anything is enqueued
    lib = _lib.load_library()

    def call(p, tbl=None, mode=_lib.BSFA_GATE_DENSE, q=FAKE):
        return lib.bsfa_prefill_noalloc(ctypes.byref(p), q, FAKE, FAKE,
                                        ctypes.byref(tbl) if tbl else None, 0, mode, -math.inf,
                                        FAKE, None, None, None, None)
    p = problem()
    p.head_dim = 96
    assert call(p) == _lib.BSFA_ERR_SHAPE
    assert call(problem(), q=None) == _lib.BSFA_ERR_ARG
    assert call(problem(), mode=_lib.BSFA_GATE_ABSOLUTE, q=None) == _lib.BSFA_ERR_TABLE
    # 512K tokens x 32 heads: 4096 query blocks x 128 mask words x 8 B = 128 MiB of masks
    big = problem(N=1 << 19, Hq=32, Hkv=8)
    need = lib.bsfa_prefill_workspace_bytes(ctypes.byref(big), _lib.BSFA_GATE_ABSOLUTE)
    assert need == 32 * 4096 * 128 * 8 + 256
    assert call(big, tbl=table(Hq=32, t_len=4096), mode=_lib.BSFA_GATE_ABSOLUTE) == \
        _lib.BSFA_ERR_UNSUPPORTED
    assert "static scratch" in _lib.bsfa_last_error()
    # the binding needs a caller-provided O (it allocates nothing)
    import torch
    Q = torch.zeros(1, 256, 4, 128, dtype=torch.bfloat16)
    K = torch.zeros(1, 256, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        _lib.bsfa_prefill_noalloc(Q, K, K, None, block_q=128)
