"""Write the stored threshold tables used by the parity tests and the benchmark.

    python tests/golden/make_tables.py [config ...]

Each table is calibrated by the CPU oracle (oracle.calibrate: k-th highest off-diagonal block
maximum per sample, head and query block, averaged over samples; "Block Sparse Flash
Attention", Method > Key Designs 1) on the calibration seeds of a named synthetic workload,
on the bf16-rounded inputs the device consumes (a workload with gate_dtype "fp8" against the
FP8 gate's block maxima). Nothing here calls the HIP library.

File format: one JSON header line, then little-endian float32 [n_budgets][heads_q][t_len].
"""
import json
import math
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from block_sparse_long_amd import synth  # noqa: E402  (input generator only)

MAGIC = "bsfa-threshold-table-v1"


def table_path(config: str) -> str:
    return os.path.join(HERE, f"thresholds_{config}.bin")


def samples(config: str, seeds, n):
    for s in seeds:
        t0 = time.time()
        Q, K, _ = synth.make_inputs(config, s, n=n)
        Qb, Kb = synth.to_bf16(Q, K)
        print(f"  seed {s}: generated in {time.time() - t0:.1f}s", flush=True)
        yield Qb.float().numpy(), Kb.float().numpy()


def make(config: str) -> None:
    c = synth.CONFIGS[config]
    if not c["budgets"]:
        return
    t0 = time.time()
    scale = float(np.float32(1.0 / math.sqrt(c["d"])))
    gate_dtype = c.get("gate_dtype", "bf16")
    T = oracle.calibrate(samples(config, c["calib_seeds"], c["calib_n"]), block_q=c["block_q"],
                         block_k=c["block_k"], budgets=c["budgets"], scale=scale,
                         gate_dtype=gate_dtype)
    hdr = {"magic": MAGIC, "n_budgets": len(c["budgets"]), "heads_q": int(T.shape[1]),
           "t_len": int(T.shape[2]), "budgets": c["budgets"], "block_q": c["block_q"],
           "block_k": c["block_k"], "head_dim": c["d"], "softmax_scale": scale,
           "calib_seqlen": c["calib_n"], "seeds": c["calib_seeds"],
           "generator": f"block_sparse_long_amd.synth.make_inputs('{config}')",
           "calibrated_by": "oracle.calibrate (CPU, float32)", "gate_dtype": gate_dtype}
    with open(table_path(config), "wb") as f:
        f.write((json.dumps(hdr) + "\n").encode())
        f.write(T.astype("<f4").tobytes())
    print(f"{config}: T{list(T.shape)} in {time.time() - t0:.1f}s", flush=True)


if __name__ == "__main__":
    names = sys.argv[1:] or [k for k, v in synth.CONFIGS.items() if v["budgets"]]
    for name in names:
        make(name)
