"""Threshold tables: the offline calibration artifact and its file format.

A table holds T[n_budgets][heads_q][t_len] (fp32, +-inf allowed) for one layer, one slice per
budget k, plus the tile semantics it was calibrated for. Budgets are selected at call time by
slice index without recalibration; a table is only valid for the model, head count, tile shape
and softmax scale it was calibrated with ("Block Sparse Flash Attention", Method > Key Designs
1). Positions past t_len reuse the last column.

File format: one JSON header line (UTF-8, ending in a newline), then the float32 array in
little-endian order, C-contiguous [n_budgets][heads_q][t_len].
"""
from __future__ import annotations

import ctypes
import json
from dataclasses import dataclass, field

import numpy as np

from . import _lib

MAGIC = "bsfa-threshold-table-v1"


@dataclass
class ThresholdTable:
    T: np.ndarray                 # float32 [n_budgets, heads_q, t_len]
    budgets: list
    block_q: int
    block_k: int
    head_dim: int
    softmax_scale: float
    calib_seqlen: int = 0
    seeds: list = field(default_factory=list)
    generator: str = ""

    def __post_init__(self):
        self.T = np.ascontiguousarray(self.T, dtype=np.float32)
        if self.T.ndim != 3 or self.T.shape[0] != len(self.budgets):
            raise ValueError("T must be [n_budgets, heads_q, t_len] with one slice per budget")

    @property
    def heads_q(self) -> int:
        return int(self.T.shape[1])

    @property
    def t_len(self) -> int:
        return int(self.T.shape[2])

    def slice_index(self, k: int) -> int:
        return self.budgets.index(int(k))

    def header(self) -> dict:
        return {"magic": MAGIC, "n_budgets": len(self.budgets), "heads_q": self.heads_q,
                "t_len": self.t_len, "budgets": [int(k) for k in self.budgets],
                "block_q": self.block_q, "block_k": self.block_k, "head_dim": self.head_dim,
                "softmax_scale": float(self.softmax_scale), "calib_seqlen": self.calib_seqlen,
                "seeds": list(self.seeds), "generator": self.generator}

    def save(self, path: str) -> None:
        with open(path, "wb") as f:
            f.write((json.dumps(self.header()) + "\n").encode())
            f.write(self.T.astype("<f4").tobytes())

    @classmethod
    def load(cls, path: str) -> "ThresholdTable":
        with open(path, "rb") as f:
            hdr = json.loads(f.readline().decode())
            if hdr.get("magic") != MAGIC:
                raise ValueError(f"{path}: not a threshold table")
            shape = (hdr["n_budgets"], hdr["heads_q"], hdr["t_len"])
            data = np.frombuffer(f.read(), dtype="<f4")
        if data.size != shape[0] * shape[1] * shape[2]:
            raise ValueError(f"{path}: payload holds {data.size} floats, header says {shape}")
        return cls(T=data.reshape(shape).astype(np.float32), budgets=hdr["budgets"],
                   block_q=hdr["block_q"], block_k=hdr["block_k"], head_dim=hdr["head_dim"],
                   softmax_scale=hdr["softmax_scale"], calib_seqlen=hdr.get("calib_seqlen", 0),
                   seeds=hdr.get("seeds", []), generator=hdr.get("generator", ""))

    def to_device(self, device, record_budgets: bool = True) -> "DeviceTable":
        """The table in device memory. record_budgets=False hands the library no budgets (it
        then cannot predict a call's density and runs the absolute gate in two launches
        whenever it has a workspace)."""
        import torch
        return DeviceTable(torch.from_numpy(self.T.copy()).to(device), self, record_budgets)


class DeviceTable:
    """A table resident in device memory, passed to bsfa_prefill."""

    def __init__(self, T_dev, host: ThresholdTable, record_budgets: bool = True):
        self.T = T_dev
        self.host = host
        self.record_budgets = record_budgets

    def c_struct(self) -> _lib.BsfaTable:
        t = _lib.BsfaTable()
        t.T = self.T.data_ptr()
        t.n_budgets = self.host.T.shape[0]
        t.t_len = self.host.t_len
        t.heads_q = self.host.heads_q
        t.block_q = self.host.block_q
        t.block_k = self.host.block_k
        t.head_dim = self.host.head_dim
        t.softmax_scale = float(self.host.softmax_scale)
        # the k of each slice (host memory, read during the call): kept alive with the table
        if self.record_budgets:
            self._budgets = (ctypes.c_int32 * len(self.host.budgets))(
                *[int(k) for k in self.host.budgets])
            t.budgets = self._budgets
        return t


def calibrate_table(samples, *, budgets, block_q: int, block_k: int = 64,
                    softmax_scale: float = 0.0, gate_dtype="bf16") -> ThresholdTable:
    """Offline calibration on the GPU ("Block Sparse Flash Attention", Method > Key Designs 1):
    for each sample (Q [B, N, Hq, d], K [B, N, Hkv, d], bf16 device tensors; every batch entry
    counts as one sample) the k-th highest off-diagonal block maximum per head and query block
    (bsfa_calibrate_blockmax, on the FP8 gate's scores for gate_dtype "fp8"), then the
    arithmetic mean over samples in float64 (-inf where a query block has fewer than k
    candidates). All samples share one shape; T_len = their number of query blocks."""
    import math
    import torch
    acc, count, shape = None, 0, None
    for Q, K in samples:
        if shape is None:
            shape = tuple(Q.shape[1:])
        elif tuple(Q.shape[1:]) != shape:
            raise ValueError("calibration samples must share one shape")
        kth = _lib.bsfa_calibrate_blockmax(Q, K, list(budgets), block_q=block_q, block_k=block_k,
                                           softmax_scale=softmax_scale, gate_dtype=gate_dtype)
        torch.cuda.synchronize(Q.device)
        kth = kth.cpu().numpy().astype(np.float64)          # [n_budgets, B, Hq, nqb]
        acc = kth.sum(axis=1) if acc is None else acc + kth.sum(axis=1)
        count += kth.shape[1]
    if not count:
        raise ValueError("no calibration samples")
    N, d = shape[0], shape[2]
    scale = softmax_scale if softmax_scale > 0 else float(np.float32(1 / math.sqrt(d)))
    return ThresholdTable(T=(acc / count).astype(np.float32), budgets=[int(k) for k in budgets],
                          block_q=block_q, block_k=block_k, head_dim=d, softmax_scale=scale,
                          calib_seqlen=N)
