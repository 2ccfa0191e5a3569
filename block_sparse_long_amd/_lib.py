"""ctypes binding of libbsfa.so (include/bsfa.h). Argument marshalling only.

Torch tensors supply device memory and the current HIP stream; every computation happens in the
library's kernels. The functions keep the C names. The library is loaded on first use and a
missing library raises: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import math
import os

BSFA_OK = 0
BSFA_ERR_ARG = 1
BSFA_ERR_SHAPE = 2
BSFA_ERR_DTYPE = 3
BSFA_ERR_ALIGN = 4
BSFA_ERR_TABLE = 5
BSFA_ERR_UNSUPPORTED = 6
BSFA_ERR_HIP = 7

BSFA_GATE_DENSE = 0
BSFA_GATE_ABSOLUTE = 1
BSFA_GATE_RELATIVE = 2

BSFA_BF16 = 0
BSFA_FP32 = 1
BSFA_FP8_E4M3 = 2
GATE_DTYPES = {"bf16": BSFA_BF16, "fp8": BSFA_FP8_E4M3}

GATE_MODES = {"dense": BSFA_GATE_DENSE, "absolute": BSFA_GATE_ABSOLUTE,
              "relative": BSFA_GATE_RELATIVE}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbsfa.so")
ABI_MAJOR = 3    # the layout of bsfa_problem and the entry points' signatures below

EXPORTED = ("bsfa_prefill", "bsfa_prefill_noalloc", "bsfa_prefill_varlen", "bsfa_prefill_paged",
            "bsfa_prefill_workspace_bytes",
            "bsfa_gate_masks", "bsfa_calibrate_blockmax", "bsfa_calibrate_workspace_bytes",
            "bsfa_mfma_rate_probe", "bsfa_status_string", "bsfa_last_error", "bsfa_version")


class BsfaProblem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32), ("heads_q", ctypes.c_int32),
        ("heads_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("block_q", ctypes.c_int32),
        ("block_k", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
        ("kv_seqlen", ctypes.c_int32), ("mean_correction", ctypes.c_int32),
        ("gate_dtype", ctypes.c_int32),
    ]


class BsfaTable(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_void_p), ("n_budgets", ctypes.c_int32), ("t_len", ctypes.c_int32),
        ("heads_q", ctypes.c_int32), ("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("budgets", ctypes.POINTER(ctypes.c_int32)),
    ]


class BsfaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"bsfa status {status}: {detail}")


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libbsfa.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with python -m "
                           "block_sparse_long_amd.build_lib (there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    lib.bsfa_version.restype = ctypes.c_int32
    if lib.bsfa_version() >> 16 != ABI_MAJOR:
        raise RuntimeError(f"{path} has ABI {lib.bsfa_version() >> 16}, this binding "
                           f"expects {ABI_MAJOR}: rebuild it")
    vp = ctypes.c_void_p
    lib.bsfa_prefill.restype = ctypes.c_int32
    lib.bsfa_prefill.argtypes = [ctypes.POINTER(BsfaProblem), vp, vp, vp, ctypes.POINTER(BsfaTable),
                                 ctypes.c_int32, ctypes.c_int32, ctypes.c_float, vp, vp, vp, vp,
                                 vp, ctypes.c_uint64, vp]
    lib.bsfa_prefill_noalloc.restype = ctypes.c_int32
    lib.bsfa_prefill_noalloc.argtypes = [ctypes.POINTER(BsfaProblem), vp, vp, vp,
                                         ctypes.POINTER(BsfaTable), ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_float, vp, vp, vp, vp, vp]
    lib.bsfa_prefill_varlen.restype = ctypes.c_int32
    lib.bsfa_prefill_varlen.argtypes = [ctypes.POINTER(BsfaProblem), vp, vp, vp, vp, vp,
                                        ctypes.POINTER(BsfaTable), ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_float, vp, vp, vp, vp, vp, ctypes.c_uint64, vp]
    lib.bsfa_prefill_paged.restype = ctypes.c_int32
    lib.bsfa_prefill_paged.argtypes = [ctypes.POINTER(BsfaProblem), vp, vp, vp, vp, vp, vp,
                                       ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(BsfaTable),
                                       ctypes.c_int32, ctypes.c_int32, ctypes.c_float, vp, vp, vp,
                                       vp, vp, ctypes.c_uint64, vp]
    lib.bsfa_prefill_workspace_bytes.restype = ctypes.c_uint64
    lib.bsfa_prefill_workspace_bytes.argtypes = [ctypes.POINTER(BsfaProblem), ctypes.c_int32]
    lib.bsfa_gate_masks.restype = ctypes.c_int32
    lib.bsfa_gate_masks.argtypes = [ctypes.POINTER(BsfaProblem), vp, vp, ctypes.POINTER(BsfaTable),
                                    ctypes.c_int32, vp, ctypes.c_uint64, vp, vp]
    lib.bsfa_calibrate_blockmax.restype = ctypes.c_int32
    lib.bsfa_calibrate_blockmax.argtypes = [ctypes.POINTER(BsfaProblem), vp, vp,
                                            ctypes.POINTER(ctypes.c_int32), ctypes.c_int32, vp,
                                            vp, ctypes.c_uint64, vp]
    lib.bsfa_mfma_rate_probe.restype = ctypes.c_int32
    lib.bsfa_mfma_rate_probe.argtypes = [ctypes.c_int32, ctypes.c_int32, vp, vp]
    lib.bsfa_calibrate_workspace_bytes.restype = ctypes.c_uint64
    lib.bsfa_calibrate_workspace_bytes.argtypes = [ctypes.POINTER(BsfaProblem)]
    lib.bsfa_status_string.restype = ctypes.c_char_p
    lib.bsfa_status_string.argtypes = [ctypes.c_int32]
    lib.bsfa_last_error.restype = ctypes.c_char_p
    lib.bsfa_last_error.argtypes = []
    lib.bsfa_version.restype = ctypes.c_int32
    lib.bsfa_version.argtypes = []
    _lib = lib
    return lib


def bsfa_status_string(status: int) -> str:
    return load_library().bsfa_status_string(status).decode()


def bsfa_last_error() -> str:
    return load_library().bsfa_last_error().decode()


def bsfa_version() -> int:
    return load_library().bsfa_version()


def _check(status: int) -> None:
    if status != BSFA_OK:
        raise BsfaError(status, f"{bsfa_status_string(status)}: {bsfa_last_error()}")


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _strides(t, name: str):
    if t.dim() != 4:
        raise ValueError(f"{name} must be [batch, seq, heads, dim]")
    if t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError(f"{name}: the head_dim axis must be contiguous")
    return (t.stride(0), t.stride(1), t.stride(2))


def _stream_handle(stream, device) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream)


def _check_shapes(Q, K, V, O, positions: bool = True) -> None:
    """The kernels size every access from Q's shape and the problem: refuse tensors that
    disagree with it (a mismatch would make them read or write past a buffer)."""
    if K.device != Q.device or (V is not None and V.device != Q.device) or \
            (O is not None and O.device != Q.device):
        raise ValueError("Q, K, V and O must be on one device")
    if K.dim() != Q.dim():
        raise ValueError("Q and K must have the same number of dimensions")
    if K.shape[0] != Q.shape[0]:
        raise ValueError(f"K batch {K.shape[0]} differs from Q batch {Q.shape[0]}")
    if K.shape[-1] != Q.shape[-1]:
        raise ValueError(f"K head_dim {K.shape[-1]} differs from Q head_dim {Q.shape[-1]}")
    if positions and K.shape[1] < Q.shape[1]:
        raise ValueError(f"K holds {K.shape[1]} positions, fewer than Q's {Q.shape[1]}")
    if V is not None and tuple(V.shape) != tuple(K.shape):
        raise ValueError(f"V shape {tuple(V.shape)} differs from K shape {tuple(K.shape)}")
    if O is not None and tuple(O.shape) != tuple(Q.shape):
        raise ValueError(f"O shape {tuple(O.shape)} differs from Q shape {tuple(Q.shape)}")


def _check_outputs(batch: int, heads_q: int, seqlen: int, kv_seqlen: int, block_q: int,
                   block_k: int, kept_counts=None, kept_total=None, debug_block_stat=None,
                   device=None) -> None:
    """dtype, layout, device and size of the optional per-block outputs."""
    import torch
    nqb = -(-seqlen // block_q)
    nkb = -(-kv_seqlen // block_k)
    for name, t, dt, n in (("kept_counts", kept_counts, torch.int32, batch * heads_q * nqb),
                           ("kept_total", kept_total, torch.int64, 1),
                           ("debug_block_stat", debug_block_stat, torch.float32,
                            batch * heads_q * nqb * nkb)):
        if t is None:
            continue
        if t.dtype != dt or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} tensor")
        if device is not None and t.device != device:
            raise ValueError(f"{name} must be on {device}")
        if t.numel() != n:
            raise ValueError(f"{name} holds {t.numel()} elements, the problem needs {n}")


def make_problem(Q, K, V=None, O=None, *, block_q: int, block_k: int = 64,
                 softmax_scale: float = 0.0, mean_correction: bool = False,
                 gate_dtype="bf16", paged: bool = False) -> BsfaProblem:
    import torch
    _check_shapes(Q, K, V, O, positions=not paged)
    p = BsfaProblem()
    p.batch, p.seqlen, p.heads_q, p.head_dim = (int(x) for x in Q.shape)
    p.heads_kv = int(K.shape[2])
    # K and V may hold more positions than Q: the query rows are their last seqlen positions
    p.kv_seqlen = int(K.shape[1]) if K.shape[1] != Q.shape[1] else 0
    p.block_q, p.block_k = int(block_q), int(block_k)
    p.softmax_scale = float(softmax_scale)
    p.mean_correction = int(bool(mean_correction))
    p.gate_dtype = GATE_DTYPES[gate_dtype] if isinstance(gate_dtype, str) else int(gate_dtype)
    dt = {torch.bfloat16: BSFA_BF16, torch.float32: BSFA_FP32}
    p.in_dtype = dt.get(Q.dtype, -1)
    p.out_dtype = dt.get(O.dtype, -1) if O is not None else BSFA_BF16
    p.q_stride[:] = _strides(Q, "Q")
    p.k_stride[:] = _strides(K, "K")
    if V is not None:
        p.v_stride[:] = _strides(V, "V")
    if O is not None:
        p.o_stride[:] = _strides(O, "O")
    return p


def bsfa_prefill(Q, K, V, O=None, *, block_q: int, block_k: int = 64, gate_mode="dense",
                 table=None, budget_slice: int = 0, log_lambda: float = -math.inf,
                 kept_counts=None, kept_total=None, debug_block_stat=None,
                 softmax_scale: float = 0.0, stream=None, out_dtype=None, workspace=None,
                 mean_correction: bool = False, gate_dtype="bf16"):
    """Run the gated prefill kernel. Q: [B, N, Hq, d] bf16; K, V: [B, Nk, Hkv, d] bf16 (device),
    Nk >= N (Nk > N: a chunk of N query rows after Nk - N cached keys).

    O (allocated if None, dtype ``out_dtype`` or bf16), kept_counts (int32 [B, Hq, nqb]),
    kept_total (int64 [1], read as uint64) and debug_block_stat (fp32 [B, Hq, nqb, nkb]) are
    written by the kernel on ``stream`` (default: torch's current stream). ``table`` is a
    block_sparse_long_amd.table.DeviceTable (needed for gate_mode "absolute"). ``workspace`` is a
    device uint8 tensor of at least bsfa_prefill_workspace_bytes bytes: the ticket counter of
    dense and relative launches, the absolute gate's keep masks (and, with
    ``mean_correction``, the block means); None allocates one, and an empty tensor asks for
    the path without it. ``mean_correction``: pruned blocks add their
    mean-key / mean-value stand-ins (absolute gate with a workspace). ``gate_dtype`` "fp8":
    the absolute gate scores E4M3 copies of Q and K (the table must be calibrated on the same
    scores). Returns O.
    """
    import torch
    lib = load_library()
    if O is None:
        O = torch.empty(Q.shape, dtype=out_dtype or torch.bfloat16, device=Q.device)
    mode = GATE_MODES[gate_mode] if isinstance(gate_mode, str) else int(gate_mode)
    p = make_problem(Q, K, V, O, block_q=block_q, block_k=block_k, softmax_scale=softmax_scale,
                     mean_correction=mean_correction,
                     gate_dtype=gate_dtype)
    tbl = None
    if table is not None:
        tbl = table.c_struct()
    _check_outputs(p.batch, p.heads_q, p.seqlen, int(K.shape[1]), block_q, block_k, kept_counts,
                   kept_total, debug_block_stat, Q.device)
    if workspace is None:
        nbytes = int(lib.bsfa_prefill_workspace_bytes(ctypes.byref(p), mode))
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=Q.device)
    if workspace is not None and workspace.numel() == 0:
        workspace = None
    if workspace is not None and (not workspace.is_contiguous() or workspace.device != Q.device):
        raise ValueError("workspace must be a contiguous tensor on Q's device")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.bsfa_prefill(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V),
                          ctypes.byref(tbl) if tbl is not None else None, int(budget_slice),
                          mode, float(log_lambda), _ptr(O), _ptr(kept_counts), _ptr(kept_total),
                          _ptr(debug_block_stat), _ptr(workspace), ctypes.c_uint64(ws_bytes),
                          _stream_handle(stream, Q.device))
    _check(st)
    return O


def bsfa_prefill_noalloc(Q, K, V, O, *, block_q: int, block_k: int = 64, gate_mode="dense",
                         table=None, budget_slice: int = 0, log_lambda: float = -math.inf,
                         kept_counts=None, kept_total=None, debug_block_stat=None,
                         softmax_scale: float = 0.0, stream=None, mean_correction: bool = False,
                         gate_dtype="bf16"):
    """bsfa_prefill with its workspace in the library's static device scratch:
    neither this function nor the library allocates (O and every output are the caller's).
    Same arguments and results as bsfa_prefill with a workspace. Returns O."""
    lib = load_library()
    if O is None:
        raise ValueError("bsfa_prefill_noalloc writes into a caller-provided O")
    mode = GATE_MODES[gate_mode] if isinstance(gate_mode, str) else int(gate_mode)
    p = make_problem(Q, K, V, O, block_q=block_q, block_k=block_k, softmax_scale=softmax_scale,
                     mean_correction=mean_correction, gate_dtype=gate_dtype)
    tbl = table.c_struct() if table is not None else None
    _check_outputs(p.batch, p.heads_q, p.seqlen, int(K.shape[1]), block_q, block_k, kept_counts,
                   kept_total, debug_block_stat, Q.device)
    st = lib.bsfa_prefill_noalloc(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V),
                                  ctypes.byref(tbl) if tbl is not None else None,
                                  int(budget_slice), mode, float(log_lambda), _ptr(O),
                                  _ptr(kept_counts), _ptr(kept_total), _ptr(debug_block_stat),
                                  _stream_handle(stream, Q.device))
    _check(st)
    return O


def bsfa_prefill_varlen(Q, K, V, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
                        max_seqlen_k: int, O=None, *, block_q: int, block_k: int = 64,
                        gate_mode="dense", table=None, budget_slice: int = 0,
                        log_lambda: float = -math.inf, kept_counts=None, kept_total=None,
                        debug_block_stat=None, softmax_scale: float = 0.0, stream=None,
                        out_dtype=None, workspace=None, mean_correction: bool = False,
                        gate_dtype="bf16"):
    """bsfa_prefill over sequences packed along the token axis. Q: [total_q, Hq, d] bf16;
    K, V: [total_k, Hkv, d] bf16; cu_seqlens_q / cu_seqlens_k: device int32 [B + 1] token
    offsets. Per-sequence outputs are padded to the longest sequence. Returns O."""
    import torch
    lib = load_library()
    if Q.dim() != 3 or K.dim() != 3 or V.dim() != 3:
        raise ValueError("Q, K and V must be [tokens, heads, dim]")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if t.dtype != torch.int32 or not t.is_contiguous() or t.dim() != 1:
            raise ValueError(f"{name} must be a contiguous int32 vector")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    if O is None:
        O = torch.empty(Q.shape, dtype=out_dtype or torch.bfloat16, device=Q.device)
    mode = GATE_MODES[gate_mode] if isinstance(gate_mode, str) else int(gate_mode)
    # the per-token views as [1, tokens, heads, dim] give the token and head strides
    p = make_problem(Q[None], K[None], V[None], O[None], block_q=block_q, block_k=block_k,
                     softmax_scale=softmax_scale, mean_correction=mean_correction,
                     gate_dtype=gate_dtype)
    p.batch = cu_seqlens_q.numel() - 1
    p.seqlen = int(max_seqlen_q)
    p.kv_seqlen = int(max_seqlen_k) if int(max_seqlen_k) != int(max_seqlen_q) else 0
    for st in (p.q_stride, p.k_stride, p.v_stride, p.o_stride):
        st[0] = 0
    tbl = table.c_struct() if table is not None else None
    _check_outputs(p.batch, p.heads_q, p.seqlen, p.kv_seqlen or p.seqlen, block_q, block_k,
                   kept_counts, kept_total, debug_block_stat, Q.device)
    if workspace is None:
        nbytes = int(lib.bsfa_prefill_workspace_bytes(ctypes.byref(p), mode))
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=Q.device)
    if workspace is not None and workspace.numel() == 0:
        workspace = None
    if workspace is not None and (not workspace.is_contiguous() or workspace.device != Q.device):
        raise ValueError("workspace must be a contiguous tensor on Q's device")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.bsfa_prefill_varlen(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(cu_seqlens_q),
                                 _ptr(cu_seqlens_k),
                                 ctypes.byref(tbl) if tbl is not None else None,
                                 int(budget_slice), mode, float(log_lambda), _ptr(O),
                                 _ptr(kept_counts), _ptr(kept_total), _ptr(debug_block_stat),
                                 _ptr(workspace), ctypes.c_uint64(ws_bytes),
                                 _stream_handle(stream, Q.device))
    _check(st)
    return O


def bsfa_prefill_paged(Q, K_pages, V_pages, cu_seqlens_q, kv_lens, block_table,
                       max_seqlen_q: int, max_seqlen_k: int, O=None, *, block_q: int,
                       block_k: int = 64, gate_mode="dense", table=None, budget_slice: int = 0,
                       log_lambda: float = -math.inf, kept_counts=None, kept_total=None,
                       debug_block_stat=None, softmax_scale: float = 0.0, stream=None,
                       out_dtype=None, workspace=None, mean_correction: bool = False,
                       gate_dtype="bf16"):
    """bsfa_prefill_varlen with K / V in a paged cache. Q: [total_q, Hq, d] bf16;
    K_pages, V_pages: [num_pages, page_size, Hkv, d] bf16; cu_seqlens_q: int32 [B + 1];
    kv_lens: int32 [B]; block_table: int32 [B, pages per sequence]. Returns O."""
    import torch
    lib = load_library()
    if Q.dim() != 3 or K_pages.dim() != 4 or V_pages.dim() != 4:
        raise ValueError("Q must be [tokens, heads, dim], K_pages / V_pages [pages, page, heads, dim]")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("kv_lens", kv_lens),
                    ("block_table", block_table)):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 tensor")
    if block_table.dim() != 2 or kv_lens.numel() != cu_seqlens_q.numel() - 1 or \
            block_table.shape[0] != kv_lens.numel():
        raise ValueError("block_table must be [B, pages]; kv_lens [B]; cu_seqlens_q [B + 1]")
    if O is None:
        O = torch.empty(Q.shape, dtype=out_dtype or torch.bfloat16, device=Q.device)
    mode = GATE_MODES[gate_mode] if isinstance(gate_mode, str) else int(gate_mode)
    if tuple(V_pages.shape) != tuple(K_pages.shape):
        raise ValueError("K_pages and V_pages must have the same shape")
    p = make_problem(Q[None], K_pages[:, 0][None], V_pages[:, 0][None], O[None],
                     block_q=block_q, block_k=block_k, softmax_scale=softmax_scale,
                     mean_correction=mean_correction,
                     gate_dtype=gate_dtype, paged=True)
    p.batch = kv_lens.numel()
    p.seqlen = int(max_seqlen_q)
    p.kv_seqlen = int(max_seqlen_k) if int(max_seqlen_k) != int(max_seqlen_q) else 0
    p.q_stride[0] = p.o_stride[0] = 0
    p.k_stride[:] = (K_pages.stride(0), K_pages.stride(1), K_pages.stride(2))
    p.v_stride[:] = (V_pages.stride(0), V_pages.stride(1), V_pages.stride(2))
    tbl = table.c_struct() if table is not None else None
    _check_outputs(p.batch, p.heads_q, p.seqlen, p.kv_seqlen or p.seqlen, block_q, block_k,
                   kept_counts, kept_total, debug_block_stat, Q.device)
    if workspace is None:
        nbytes = int(lib.bsfa_prefill_workspace_bytes(ctypes.byref(p), mode))
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=Q.device)
    if workspace is not None and workspace.numel() == 0:
        workspace = None
    if workspace is not None and (not workspace.is_contiguous() or workspace.device != Q.device):
        raise ValueError("workspace must be a contiguous tensor on Q's device")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.bsfa_prefill_paged(ctypes.byref(p), _ptr(Q), _ptr(K_pages), _ptr(V_pages),
                                _ptr(cu_seqlens_q), _ptr(kv_lens), _ptr(block_table),
                                int(block_table.shape[1]), int(K_pages.shape[1]),
                                ctypes.byref(tbl) if tbl is not None else None,
                                int(budget_slice), mode, float(log_lambda), _ptr(O),
                                _ptr(kept_counts), _ptr(kept_total), _ptr(debug_block_stat),
                                _ptr(workspace), ctypes.c_uint64(ws_bytes),
                                _stream_handle(stream, Q.device))
    _check(st)
    return O


def bsfa_gate_masks(Q, K, table, budget_slice: int = 0, keep_mask=None, *, block_q: int,
                    block_k: int = 64, debug_block_stat=None, softmax_scale: float = 0.0,
                    stream=None, gate_dtype="bf16"):
    """Keep bitmasks of the absolute gate: int64 [B, Hq, nqb, W] (bit j % 64 of word j // 64 set
    iff off-diagonal 64-key tile j is kept; a kept 128-key block sets both of its tiles);
    allocated if None. Returns keep_mask. With ``gate_dtype`` "fp8" the call also needs room
    for the FP8 copies: keep_mask is then None or a contiguous 1-D buffer of at least
    bsfa_prefill_workspace_bytes(..., gate_dtype="fp8") bytes, and the masks come back as a view
    of its start. A contiguous 1-D uint8 buffer with bf16 scores is taken the same way (masks
    at its start); one of bsfa_prefill_workspace_bytes(...) bytes makes the sweep run as inside
    bsfa_prefill (units from the workspace's counter)."""
    import torch
    lib = load_library()
    B, N, Hq, _ = Q.shape
    nqb, ntile = -(-N // block_q), -(-int(K.shape[1]) // 64)   # one bit per 64-key tile
    shape = (B, Hq, nqb, -(-ntile // 64))
    fp8 = (GATE_DTYPES[gate_dtype] if isinstance(gate_dtype, str) else int(gate_dtype)) \
        == BSFA_FP8_E4M3
    buf = None
    flat = keep_mask is not None and keep_mask.dim() == 1 and keep_mask.dtype == torch.uint8
    if fp8 or flat:
        nbytes = bsfa_prefill_workspace_bytes(Q, K, block_q=block_q, block_k=block_k,
                                              gate_dtype="fp8") if fp8 else \
            B * Hq * nqb * shape[3] * 8
        buf = keep_mask if keep_mask is not None else torch.empty(nbytes, dtype=torch.uint8,
                                                                  device=Q.device)
        if not buf.is_contiguous() or buf.numel() * buf.element_size() < nbytes:
            raise ValueError(f"keep_mask needs a contiguous buffer of {nbytes} bytes")
        nbuf = buf.numel() * buf.element_size()
        keep_mask = buf.view(torch.uint8)[:B * Hq * nqb * shape[3] * 8].view(torch.int64)
        keep_mask = keep_mask.view(shape)
    elif keep_mask is None:
        keep_mask = torch.empty(shape, dtype=torch.int64, device=Q.device)
    if not keep_mask.is_contiguous() or keep_mask.element_size() != 8:
        raise ValueError("keep_mask must be a contiguous 8-byte-element tensor")
    if keep_mask.device != Q.device:
        raise ValueError("keep_mask must be on Q's device")
    _check_outputs(B, Hq, N, int(K.shape[1]), block_q, block_k,
                   debug_block_stat=debug_block_stat, device=Q.device)
    p = make_problem(Q, K, block_q=block_q, block_k=block_k, softmax_scale=softmax_scale,
                     gate_dtype=gate_dtype)
    tbl = table.c_struct()
    st = lib.bsfa_gate_masks(ctypes.byref(p), _ptr(Q), _ptr(K), ctypes.byref(tbl),
                             int(budget_slice), _ptr(keep_mask),
                             ctypes.c_uint64(nbuf if buf is not None else keep_mask.numel() * 8),
                             _ptr(debug_block_stat), _stream_handle(stream, Q.device))
    _check(st)
    return keep_mask


def bsfa_calibrate_blockmax(Q, K, budgets, kth_out=None, *, block_q: int, block_k: int = 64,
                            softmax_scale: float = 0.0, stream=None, gate_dtype="bf16",
                            workspace=None):
    """k-th highest off-diagonal block max per (budget, b, h, i): fp32 [n_budgets, B, Hq, nqb].
    ``gate_dtype`` "fp8": on the FP8 gate's scores (a workspace is allocated if None)."""
    import torch
    lib = load_library()
    B, N, Hq, _ = Q.shape
    nqb = -(-N // block_q)
    if kth_out is None:
        kth_out = torch.empty((len(budgets), B, Hq, nqb), dtype=torch.float32, device=Q.device)
    if kth_out.dtype != torch.float32 or not kth_out.is_contiguous() or \
            kth_out.device != Q.device or kth_out.numel() != len(budgets) * B * Hq * nqb:
        raise ValueError(f"kth_out must be a contiguous float32 tensor of {len(budgets)} x {B} x "
                         f"{Hq} x {nqb} elements on Q's device")
    p = make_problem(Q, K, block_q=block_q, block_k=block_k, softmax_scale=softmax_scale,
                     gate_dtype=gate_dtype)
    if workspace is None:
        n = int(lib.bsfa_calibrate_workspace_bytes(ctypes.byref(p)))
        if n:
            workspace = torch.empty(n, dtype=torch.uint8, device=Q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    arr = (ctypes.c_int32 * max(1, len(budgets)))(*[int(k) for k in budgets])
    st = lib.bsfa_calibrate_blockmax(ctypes.byref(p), _ptr(Q), _ptr(K), arr, len(budgets),
                                     _ptr(kth_out), _ptr(workspace), ctypes.c_uint64(ws_bytes),
                                     _stream_handle(stream, Q.device))
    _check(st)
    return kth_out


def bsfa_prefill_workspace_bytes(Q, K, *, block_q: int, block_k: int = 64,
                                 gate_mode="absolute", mean_correction: bool = False,
                                 gate_dtype="bf16") -> int:
    """Bytes of workspace bsfa_prefill can use for this problem and gate mode (0: none)."""
    mode = GATE_MODES[gate_mode] if isinstance(gate_mode, str) else int(gate_mode)
    p = make_problem(Q, K, block_q=block_q, block_k=block_k, mean_correction=mean_correction,
                     gate_dtype=gate_dtype)
    return int(load_library().bsfa_prefill_workspace_bytes(ctypes.byref(p), mode))


def bsfa_mfma_rate_probe(workgroups: int = 1024, iters: int = 256, sink=None, stream=None,
                         device="cuda"):
    """Enqueue the MFMA rate probe; returns (sink, executed FLOPs). Time it on `stream`."""
    import torch
    lib = load_library()
    if sink is None:
        sink = torch.empty(workgroups * 256, dtype=torch.float32, device=device)
    _check(lib.bsfa_mfma_rate_probe(int(workgroups), int(iters), _ptr(sink),
                                    _stream_handle(stream, sink.device)))
    return sink, float(workgroups) * 4 * 4 * iters * 32768
