"""Offline threshold calibration on the GPU, as a command:

    python -m block_sparse_long_amd.calibrate --config llama_32k_sweep --seeds 1-8 \\
        --budgets 16,64,256 [--seqlen 32768] [--gate-dtype fp8] --out table.bin

For each calibration seed of a named synthetic workload (block_sparse_long_amd.synth), the
k-th highest off-diagonal block maximum per head and query block is taken on the device
(bsfa_calibrate_blockmax; on FP8 gate scores with --gate-dtype fp8), and the thresholds are
the float64 mean over seeds ("Block Sparse Flash Attention", Method > Key Designs 1). The table
is written in the file format of block_sparse_long_amd.table.
"""
from __future__ import annotations

import argparse
import time


def _seeds(text: str) -> list:
    out = []
    for part in text.split(","):
        if "-" in part:
            a, b = part.split("-")
            out += list(range(int(a), int(b) + 1))
        else:
            out.append(int(part))
    return out


def main(argv=None) -> None:
    import torch

    from . import _lib, synth
    from .table import calibrate_table

    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--config", required=True, choices=sorted(synth.CONFIGS))
    ap.add_argument("--seeds", default="1-8", help="calibration seeds, e.g. 1-8 or 1,3,5")
    ap.add_argument("--budgets", required=True, help="comma-separated k values")
    ap.add_argument("--seqlen", type=int, default=None, help="calibration length (default: "
                    "the workload's calibration length)")
    ap.add_argument("--gate-dtype", choices=("bf16", "fp8"), default="bf16")
    ap.add_argument("--out", required=True)
    args = ap.parse_args(argv)

    c = synth.CONFIGS[args.config]
    n = args.seqlen or c["calib_n"] or c["n"]
    budgets = [int(k) for k in args.budgets.split(",")]
    _lib.load_library()
    dev = torch.device("cuda:0")

    def samples():
        for s in _seeds(args.seeds):
            Q, K, _ = synth.make_inputs(args.config, s, n=n)
            Qb, Kb = synth.to_bf16(Q, K)
            yield Qb.to(dev), Kb.to(dev)

    t0 = time.time()
    tab = calibrate_table(samples(), budgets=budgets, block_q=c["block_q"],
                          block_k=c["block_k"], gate_dtype=args.gate_dtype)
    tab.seeds = _seeds(args.seeds)
    tab.generator = f"block_sparse_long_amd.synth.make_inputs('{args.config}')"
    tab.save(args.out)
    print(f"{args.config}: T{list(tab.T.shape)} ({args.gate_dtype} scores) in "
          f"{time.time() - t0:.1f}s -> {args.out}")


if __name__ == "__main__":
    main()
