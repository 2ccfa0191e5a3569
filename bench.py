"""Benchmark: gated prefill attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--quick]
    python bench.py --profile-once     # one 1 GiB copy + one gated call, for counter runs
    python bench.py --counters FETCH_DIR WRITE_DIR   # counter runs -> profiles/traffic_*.json

A step is one bsfa_prefill call over one batch of synthetic input already resident in HBM:
exact QK^T on every causally visible tile, the gate, online softmax and PV on kept tiles.
Prints one JSON line. `value` is executed TFLOP/s of the gated call: tile-level FLOPs of QK on
every visible tile plus PV on every kept or diagonal tile, counted from the kernel's own kept
counts (2*Bq*Bk*d per tile product), divided by the time of the step. The same line carries
the dense path of the same kernel (gate compiled out), the zero-skip taxes, the kept fraction,
the roofline of the call's dominant kernel and the CPU oracle timed on a bounded sample of the
same workload. Under the absolute gate the call is two launches: the gate sweep (QK on every
off-diagonal tile, timed on its own through bsfa_gate_masks with HIP events on the launch
stream) and the softmax walk over the kept tiles (the rest of the call). roofline.traffic is
the HBM bytes per launch that rocprofv3 counters measured for that kernel on the current kernel
source (profiles/traffic_<workload>.json, FETCH_SIZE + WRITE_SIZE scaled by a 1 GiB copy); it
is null when the kernel source changed.
"""
import hashlib
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "gated prefill attn ms + executed TFLOP/s (% MFMA peak) at 32K/128K vs dense"
PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 MFMA, published
PEAK_FP8_TFLOPS = 5000.0           # MI355X dense fp8 MFMA, published
PEAK_HBM_GBS = 8000.0
GOLDEN = os.path.join(ROOT, "tests", "golden")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama_128k")
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-once", action="store_true",
                    help="run a 1 GiB device copy and one gated call, then exit (counter runs)")
    ap.add_argument("--gate-dtype", choices=("bf16", "fp8"), default="bf16",
                    help="--profile-once / --counters: the gated call with bf16 or FP8 gate "
                         "scores (FP8: its own FP8-calibrated table)")
    ap.add_argument("--counters", nargs="+", metavar="DIR",
                    help="summarise rocprofv3 --pmc runs of --profile-once: FETCH_SIZE, "
                         "WRITE_SIZE and optionally MfmaUtil MfmaFlopsBF16 "
                         "SQ_INSTS_VALU_MFMA_MOPS_F8, into profiles/traffic_<workload>.json")
    return ap.parse_args()


KERNEL_DIR = os.path.join(ROOT, "block_sparse_long_amd", "csrc")
COPY_BYTES = 1 << 30


def kernel_source_sha256():
    """Digest of the device code: the kernel header, the argument structs and every HIP unit."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(KERNEL_DIR)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(KERNEL_DIR, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_counters(workload, kernel):
    """The committed counter summary of `kernel` (its profiler name), if it was taken on the
    current kernel source; else {}."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_sha256():
        return {}
    return rec.get("kernels", {}).get(kernel, {})


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None."""
    return measured_counters(workload, kernel).get("hbm_bytes_per_launch")


def summarise_counters(args):
    """FETCH_SIZE / WRITE_SIZE per dispatch of the prefill-path kernels, each scaled by what the
    same counter reads for the 1 GiB device copy of --profile-once (a plain copy reads and
    writes exactly COPY_BYTES), written to profiles/traffic_<workload>.json."""
    import csv
    import glob
    import re

    def per_dispatch(d, counter):
        rows = {}
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            sys.exit(f"no counter_collection.csv under {d}")
        with open(max(files, key=os.path.getmtime)) as fh:   # the newest run only
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
                rows[key] = rows.get(key, 0.0) + float(r["Counter_Value"])
        return rows

    if len(args.counters) not in (2, 3):
        sys.exit("--counters takes FETCH_DIR WRITE_DIR [MFMA_DIR]")
    fetch, write = per_dispatch(args.counters[0], "FETCH_SIZE"), per_dispatch(args.counters[1],
                                                                              "WRITE_SIZE")
    def copy_kib(rows):
        v = [x for (_, n), x in rows.items() if "copyBuffer" in n]
        return max(v) if v else None
    fk, wk = copy_kib(fetch), copy_kib(write)
    if not fk or not wk:
        sys.exit("no 1 GiB copy dispatch found in the counter runs")
    f_scale, w_scale = COPY_BYTES / (fk * 1024.0), COPY_BYTES / (wk * 1024.0)
    kernels = {}
    for rows, tag, sc in ((fetch, "fetch", f_scale), (write, "write", w_scale)):
        for (_, name), kib in rows.items():
            m = re.search(r"bsfa::\(anonymous namespace\)::(\w+<[^>]*>)", name)
            if not m:
                continue
            k = kernels.setdefault(m.group(1), {})
            k[f"{tag}_size_kib"] = kib
            k[f"{tag}_bytes"] = kib * 1024.0 * sc
    for k in kernels.values():
        k["hbm_bytes_per_launch"] = k.get("fetch_bytes", 0.0) + k.get("write_bytes", 0.0)
    # MFMA counters (third run): rocprofv3's derived MfmaUtil (MFMA-busy cycles per SIMD over
    # GPU-active cycles, %) and MfmaFlopsBF16 (bf16 MFMA ops x 512), and the FP8 op count
    if len(args.counters) == 3:
        for counter, key, sc in (("MfmaUtil", "mfma_util_pct", 1.0),
                                 ("MfmaFlopsBF16", "mfma_flops_bf16", 1.0),
                                 ("SQ_INSTS_VALU_MFMA_MOPS_F8", "mfma_flops_f8", 512.0)):
            for (_, name), v in per_dispatch(args.counters[2], counter).items():
                m = re.search(r"bsfa::\(anonymous namespace\)::(\w+<[^>]*>)", name)
                if m and m.group(1) in kernels:
                    kernels[m.group(1)][key] = v * sc
    tag = "" if args.gate_dtype == "bf16" else f" --gate-dtype {args.gate_dtype}"
    rec = {"workload": args.workload, "gate_dtype": args.gate_dtype,
           "kernel_source_sha256": kernel_source_sha256(),
           "copy_bytes": COPY_BYTES, "fetch_scale": f_scale, "write_scale": w_scale,
           "copy_fetch_kib": fk, "copy_write_kib": wk, "kernels": kernels,
           "commands": ["cd /tmp && export TMPDIR=/tmp",
                        "rocprofv3 --pmc FETCH_SIZE -d <fetch_dir> -- python3 "
                        "<repo>/bench.py --profile-once --workload " + args.workload + tag,
                        "rocprofv3 --pmc WRITE_SIZE -d <write_dir> -- python3 "
                        "<repo>/bench.py --profile-once --workload " + args.workload + tag,
                        "rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 SQ_INSTS_VALU_MFMA_MOPS_F8 "
                        "-d <mfma_dir> -- python3 <repo>/bench.py --profile-once --workload "
                        + args.workload + tag,
                        "python3 bench.py --counters <fetch_dir> <write_dir> <mfma_dir> "
                        "--workload " + args.workload + tag]}
    suffix = "" if args.gate_dtype == "bf16" else f"_{args.gate_dtype}"
    path = os.path.join(ROOT, "profiles", f"traffic_{args.workload}{suffix}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def profile_once(args):
    """The command the counter summaries are taken from: a plain 1 GiB device copy (the
    scale reference for FETCH_SIZE / WRITE_SIZE), then one gated call of the workload (and,
    with bf16 gate scores, one dense call: the softmax loop without a gate)."""
    import torch
    from block_sparse_long_amd import _lib
    _lib.load_library()
    dev = torch.device("cuda:0")
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    w = Workload(args.workload, dev)
    mode = "absolute" if w.table is not None else "relative"
    kw = dict(budget_slice=0) if mode == "absolute" else dict(log_lambda=math.log(1e-3))
    if args.gate_dtype == "fp8":
        from block_sparse_long_amd.table import ThresholdTable
        path = os.path.join(GOLDEN, f"thresholds_{args.workload}_fp8.bin")
        kw.update(gate_dtype="fp8", table=ThresholdTable.load(path).to_device(dev))
    w.call(mode, **kw)
    if args.gate_dtype == "bf16":
        w.call("dense")
    torch.cuda.synchronize()
    print(json.dumps({"profile_once": args.workload, "gate_dtype": args.gate_dtype,
                      "copy_bytes": COPY_BYTES,
                      "kernel_source_sha256": kernel_source_sha256()}), flush=True)


def block_ranges(N, Bq, Bk=64):
    """(n_off, n_end) per query block: the same block structure the kernel walks."""
    out = []
    for i in range(-(-N // Bq)):
        n_off = (i * Bq) // Bk
        n_end = (min((i + 1) * Bq, N) - 1) // Bk + 1
        out.append((n_off, n_end))
    return out


def executed_flops(kept_counts, N, Bq, d, Bk=64, query_blocks=None):
    """2*Bq*64*d per product of a query block with a 64-key tile: QK on every visible tile, PV
    on every diagonal-region tile and on the tiles of kept blocks (kept_counts counts blocks of
    Bk keys, Bk / 64 tiles each)."""
    import numpy as np
    kc = np.asarray(kept_counts, dtype=np.int64)        # [B, Hq, nqb]
    rng = block_ranges(N, Bq, 64)
    qbs = range(len(rng)) if query_blocks is None else query_blocks
    B, Hq = kc.shape[0], kc.shape[1]
    tiles = 0
    for i in qbs:
        n_off, n_end = rng[i]
        tiles += B * Hq * (n_end + (n_end - n_off)) + (Bk // 64) * int(kc[:, :, i].sum())
    return 2.0 * Bq * 64 * d * tiles


def dense_flops(B, Hq, N, Bq, d, Bk=64):
    rng = block_ranges(N, Bq, Bk)
    return 2.0 * Bq * Bk * d * B * Hq * sum(2 * n_end for _, n_end in rng)


def predicted_density(N, Bq, k, Bk=64):
    rng = block_ranges(N, Bq, Bk)
    den = sum(n_off for n_off, _ in rng)
    return sum(min(n_off, k) for n_off, _ in rng) / den if den else 1.0


class Workload:
    def __init__(self, name, device, skip=None, host=None):
        import torch
        from block_sparse_long_amd import synth
        from block_sparse_long_amd.table import ThresholdTable
        self.name = name
        self.c = c = synth.CONFIGS[name]
        self.skip = skip
        if host is None:
            Q, K, V = synth.make_inputs(name, 0, skip=skip)
            host = synth.to_bf16(Q, K, V)
            del Q, K, V
        self.host = host
        self.Qd, self.Kd, self.Vd = (x.to(device) for x in self.host)
        self.O = torch.empty_like(self.Qd)
        self.N, self.Hq, self.d, self.Bq = c["n"], c["heads_q"], c["d"], c["block_q"]
        self.Bk = c["block_k"]
        nqb = -(-self.N // self.Bq)
        self.counts = torch.zeros((1, self.Hq, nqb), dtype=torch.int32, device=device)
        self.table = None
        if c["budgets"]:
            self.table = ThresholdTable.load(os.path.join(GOLDEN, f"thresholds_{name}.bin"))
            self.dtable = self.table.to_device(device)
        rng = block_ranges(self.N, self.Bq, self.Bk)
        self.n_off_total = sum(n_off for n_off, _ in rng)     # off-diagonal gate blocks

    def call(self, mode, budget_slice=0, log_lambda=-math.inf, table=None, workspace=None,
             mean_correction=False, gate_dtype="bf16"):
        import torch
        from block_sparse_long_amd import _lib
        if workspace is None:
            attr = f"workspace_{mode}_{int(mean_correction)}_{gate_dtype}"
            if getattr(self, attr, None) is None:
                n = _lib.bsfa_prefill_workspace_bytes(self.Qd, self.Kd, block_q=self.Bq,
                                                      block_k=self.Bk, gate_mode=mode,
                                                      mean_correction=mean_correction,
                                                      gate_dtype=gate_dtype)
                setattr(self, attr, torch.empty(n, dtype=torch.uint8, device=self.Qd.device))
            workspace = getattr(self, attr)
        _lib.bsfa_prefill(self.Qd, self.Kd, self.Vd, self.O, block_q=self.Bq, block_k=self.Bk,
                          gate_mode=mode, table=table if table is not None else
                          (self.dtable if mode == "absolute" else None),
                          budget_slice=budget_slice, log_lambda=log_lambda,
                          kept_counts=self.counts, workspace=workspace,
                          mean_correction=mean_correction, gate_dtype=gate_dtype)


def timed(fn, steps, warmup):
    """(ms per call from HIP events on the launch stream, wall ms per call)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return e0.elapsed_time(e1) / steps, wall


def sweep_flops(w):
    """QK on every off-diagonal tile of every (b, h, i): the gate sweep's work."""
    return 2.0 * w.Bq * w.Bk * w.d * w.Hq * w.n_off_total


def run_sweep(w, steps, warmup):
    """The gate sweep on its own (bsfa_gate_masks), timed like a step. Its buffer is the size
    of bsfa_prefill's workspace, so the sweep runs exactly as inside the gated call."""
    import torch
    from block_sparse_long_amd import _lib
    if getattr(w, "masks", None) is None:
        n = _lib.bsfa_prefill_workspace_bytes(w.Qd, w.Kd, block_q=w.Bq, block_k=w.Bk)
        w.masks = torch.empty(n, dtype=torch.uint8, device=w.Qd.device)
    ev_ms, wall_ms = timed(lambda: _lib.bsfa_gate_masks(w.Qd, w.Kd, w.dtable, 0, w.masks,
                                                        block_q=w.Bq), steps, warmup)
    fl = sweep_flops(w)
    return dict(ms=ev_ms, wall_ms=wall_ms, flops=fl, tflops=fl / ev_ms / 1e9)


def run_chunked(w, chunk, steps, warmup, budget_slice=0):
    """Chunked prefill of the workload under the absolute gate: the query rows in chunks of
    `chunk`, chunk c against the K/V prefix of every earlier position (kv_seqlen), one call per
    chunk. A step is all chunks; executed FLOPs come from each chunk's kept counts."""
    import numpy as np
    import torch
    from block_sparse_long_amd import _lib
    n_chunks = -(-w.N // chunk)
    spans = [(c * chunk, min((c + 1) * chunk, w.N)) for c in range(n_chunks)]
    counts = [torch.zeros((1, w.Hq, -(-(r1 - r0) // w.Bq)), dtype=torch.int32,
                          device=w.Qd.device) for r0, r1 in spans]
    ws = torch.empty(_lib.bsfa_prefill_workspace_bytes(w.Qd, w.Kd, block_q=w.Bq),
                     dtype=torch.uint8, device=w.Qd.device)

    def step():
        for (r0, r1), kc in zip(spans, counts):
            _lib.bsfa_prefill(w.Qd[:, r0:r1], w.Kd[:, :r1], w.Vd[:, :r1], w.O[:, r0:r1],
                              block_q=w.Bq, gate_mode="absolute", table=w.dtable,
                              budget_slice=budget_slice, kept_counts=kc, workspace=ws)
    ev_ms, wall_ms = timed(step, steps, warmup)
    torch.cuda.synchronize()
    tiles = kept = 0
    for (r0, r1), kc in zip(spans, counts):
        kc = kc.cpu().numpy()
        kept += int(kc.sum())
        for i in range(kc.shape[2]):
            n_end = (r0 + min((i + 1) * w.Bq, r1 - r0) - 1) // 64 + 1
            n_off = (r0 + i * w.Bq) // 64
            tiles += w.Hq * (n_end + (n_end - n_off)) + int(kc[:, :, i].sum())
    flops = 2.0 * w.Bq * 64 * w.d * tiles
    return dict(ms=ev_ms, chunks=n_chunks, flops=flops, tflops=flops / ev_ms / 1e9, kept=kept)


def run_gate(w, mode, steps, warmup, **kw):
    import numpy as np
    import torch
    ev_ms, wall_ms = timed(lambda: w.call(mode, **kw), steps, warmup)
    torch.cuda.synchronize()
    counts = w.counts.cpu().numpy()
    flops = executed_flops(counts, w.N, w.Bq, w.d, w.Bk)
    kept = int(counts.sum())
    return dict(ms=ev_ms, wall_ms=wall_ms, flops=flops, tflops=flops / ev_ms / 1e9, kept=kept,
                kept_fraction=kept / (w.Hq * w.n_off_total) if w.n_off_total else 1.0,
                pct_peak=100.0 * flops / ev_ms / 1e9 / PEAK_BF16_TFLOPS)


def paired_tax(w, mode, rounds, steps, warmup, **kw):
    """Zero-skip tax of a gated call that skips nothing, against the dense path: `rounds`
    rounds of `steps` dense calls then `steps` gated calls, alternating, so that both see the
    same clock and thermal state. Returns the ratio of the medians of the rounds' means minus
    one, and the gated call's median."""
    import statistics
    dense, gated = [], []
    for _ in range(rounds):
        dense.append(run_gate(w, "dense", steps, warmup)["ms"])
        gated.append(run_gate(w, mode, steps, warmup, **kw)["ms"])
    g = statistics.median(gated)
    return g / statistics.median(dense) - 1, g


def measured_mfma_rate(steps=5, warmup=2):
    """The device's sustained bf16 MFMA rate (bsfa_mfma_rate_probe), TFLOP/s."""
    from block_sparse_long_amd import _lib
    sink, fl = _lib.bsfa_mfma_rate_probe(workgroups=1024, iters=8192)
    ms, _ = timed(lambda: _lib.bsfa_mfma_rate_probe(workgroups=1024, iters=8192, sink=sink),
                  steps, warmup)
    return fl / ms / 1e9


def flushed_median_ms(w, mode, n=20, warmup=3, **kw):
    """Median over n calls of one call's time (HIP events), a 512 MiB buffer written before
    each call so that no input is left in L2 or the last-level cache."""
    import statistics
    import torch
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=w.Qd.device)
    stream = torch.cuda.current_stream()
    out = []
    for t in range(warmup + n):
        scratch.fill_(t & 255)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        w.call(mode, **kw)
        e1.record(stream)
        torch.cuda.synchronize()
        if t >= warmup:
            out.append(e0.elapsed_time(e1))
    del scratch
    return statistics.median(out)


def run_mean_correction(w, steps, warmup, gated_ms, dense_ms):
    """The gated call with mean correction (block-means pass, sweep, walk with the pruned
    blocks' stand-ins): its time, and the deviation of the outputs with and without the
    correction from the dense output."""
    import torch
    r = run_gate(w, "absolute", steps, warmup, budget_slice=0, mean_correction=True)
    outs = {}
    for key, mode, mc in (("dense", "dense", False), ("plain", "absolute", False),
                          ("mean", "absolute", True)):
        w.call(mode, mean_correction=mc)
        outs[key] = w.O.clone()
    torch.cuda.synchronize()
    dev = {}
    for key in ("plain", "mean"):
        mx, tot = 0.0, 0.0
        for r0 in range(0, w.N, 8192):          # in row chunks: fp32 copies stay small
            e = (outs[key][:, r0:r0 + 8192].float() - outs["dense"][:, r0:r0 + 8192].float()).abs()
            mx, tot = max(mx, e.max().item()), tot + e.sum().item()
        dev[key] = (mx, tot / outs[key].numel())
    del outs
    torch.cuda.empty_cache()
    return {"ms": round(r["ms"], 3), "vs_gated": round(r["ms"] / gated_ms, 4),
            "speedup_vs_dense": round(dense_ms / r["ms"], 4),
            "max_abs_vs_dense": {"uncorrected": round(dev["plain"][0], 5),
                                 "corrected": round(dev["mean"][0], 5)},
            "mean_abs_vs_dense": {"uncorrected": round(dev["plain"][1], 7),
                                  "corrected": round(dev["mean"][1], 7)}}


def run_fp8_gate(w, steps, warmup, gated, dense_ms):
    """The gated call with FP8 gate scores (its own table, calibrated on FP8 scores): the call,
    its FP8 sweep on its own (bsfa_gate_masks), kept density, and the deviation of its output
    from the bf16-gated and the dense outputs. None if the table is not there."""
    import torch
    from block_sparse_long_amd import _lib
    from block_sparse_long_amd.table import ThresholdTable
    path = os.path.join(GOLDEN, f"thresholds_{w.name}_fp8.bin")
    if not os.path.exists(path):
        return None
    tab = ThresholdTable.load(path).to_device(w.Qd.device)
    r = run_gate(w, "absolute", steps, warmup, table=tab, gate_dtype="fp8")
    buf = torch.empty(_lib.bsfa_prefill_workspace_bytes(w.Qd, w.Kd, block_q=w.Bq,
                                                        gate_dtype="fp8"),
                      dtype=torch.uint8, device=w.Qd.device)
    sw_ms, _ = timed(lambda: _lib.bsfa_gate_masks(w.Qd, w.Kd, tab, 0, buf, block_q=w.Bq,
                                                  gate_dtype="fp8"), steps, warmup)
    fl = sweep_flops(w)
    outs = {}
    for key, kw in (("dense", dict(mode="dense")), ("bf16", dict(mode="absolute")),
                    ("fp8", dict(mode="absolute", table=tab, gate_dtype="fp8"))):
        w.call(**kw)
        outs[key] = w.O.clone()
    torch.cuda.synchronize()
    dev = {}
    for a_, b_ in (("fp8", "bf16"), ("fp8", "dense"), ("bf16", "dense")):
        tot = 0.0
        for r0 in range(0, w.N, 8192):
            tot += (outs[a_][:, r0:r0 + 8192].float()
                    - outs[b_][:, r0:r0 + 8192].float()).abs().sum().item()
        dev[f"{a_}_vs_{b_}"] = round(tot / outs[a_].numel(), 7)
    del outs
    torch.cuda.empty_cache()
    return {"ms": round(r["ms"], 3), "tflops": round(r["tflops"], 2),
            "speedup_vs_dense": round(dense_ms / r["ms"], 4),
            "vs_bf16_gate": round(r["ms"] / gated["ms"], 4),
            "kept_fraction": round(r["kept_fraction"], 4),
            "kept_fraction_bf16_gate": round(gated["kept_fraction"], 4),
            "sweep": {"ms": round(sw_ms, 3), "tflops": round(fl / sw_ms / 1e9, 2),
                      "pct_fp8_peak": round(100.0 * fl / sw_ms / 1e9 / PEAK_FP8_TFLOPS, 2)},
            "mean_abs_output_deviation": dev}


# ---- the CPU oracle, timed on the host's cores (before the GPU is touched) ----
# Worker processes are forked from this process while it has not initialised the GPU, so no
# child inherits device state; each runs the unchanged oracle on one query head (one BLAS
# thread: the oracle multiplies one tile at a time, too small for threads to help) and returns
# its kept counts and the output rows of the sampled query blocks.
_POOL = {}


def _oracle_head(h):
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_limits
    d = _POOL
    Qh, Kh, Vh, T, kw, blocks, Bq = d["Q"], d["K"], d["V"], d["T"], d["kw"], d["blocks"], d["Bq"]
    G = Qh.shape[2] // Kh.shape[2]
    g = h // G
    with threadpool_limits(limits=1):
        r = oracle.oracle_prefill(Qh[:, :, h:h + 1], Kh[:, :, g:g + 1], Vh[:, :, g:g + 1],
                                  table=None if T is None else T[:, h:h + 1, :],
                                  query_blocks=blocks, **kw)
    rows = np.concatenate([np.arange(i * Bq, min((i + 1) * Bq, Qh.shape[1])) for i in blocks])
    return h, r.kept_counts[:, 0], r.out[:, rows, 0, :]


def host_cores():
    """Worker count: the host cores this process may run on, at most 16 (the CPU share of one
    GPU on the benchmark machines)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_info():
    import numpy as np
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = ""
    try:
        from threadpoolctl import threadpool_info
        blas = ", ".join(f"{x.get('internal_api')} {x.get('version')}" for x in threadpool_info()
                         if x.get("user_api") == "blas")
    except Exception:
        pass
    return {"cpu": model, "blas": blas or "numpy", "numpy": np.__version__}


def oracle_timed(host, table_T, Bq, Bk, mode, blocks, log_lambda=-math.inf, budget_slice=0):
    """The oracle over every head of the given query blocks, one head per worker process, on
    all host cores. Returns (seconds, kept counts [B, Hq, nqb] (-1 outside the blocks), output
    rows [B, rows, Hq, d], cores)."""
    import multiprocessing as mp
    import numpy as np
    Qh, Kh, Vh = (x.float().numpy() for x in host)
    _POOL.update(Q=Qh, K=Kh, V=Vh, T=table_T, Bq=Bq, blocks=list(blocks),
                 kw=dict(block_q=Bq, block_k=Bk, mode=mode, budget_slice=budget_slice,
                         log_lambda=log_lambda))
    Hq = Qh.shape[2]
    cores = min(host_cores(), Hq)
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(cores) as pool:
        res = pool.map(_oracle_head, range(Hq), chunksize=1)
    sec = time.perf_counter() - t0
    nqb = -(-Qh.shape[1] // Bq)
    counts = np.full((Qh.shape[0], Hq, nqb), -1, np.int64)
    out = None
    for h, kc, o in res:
        counts[:, h] = kc
        if out is None:
            out = np.empty((o.shape[0], o.shape[1], Hq, o.shape[2]), np.float32)
        out[:, :, h] = o
    _POOL.clear()
    return sec, counts, out, cores


def sample_blocks(nqb, k):
    """Bounded sample of query blocks for the headline oracle timing: every 32nd block, the
    first two, the table's -inf boundary (k/2 - 1, k/2), the last calibrated and first reused
    threshold columns at 128K (511, 512) and the last."""
    kk = k or 2
    s = set(range(0, nqb, 32)) | {0, 1, kk // 2 - 1, kk // 2, nqb // 2 - 1, nqb // 2, nqb - 1}
    return sorted(x for x in s if 0 <= x < nqb)


def deviation(dev_O, oracle_out, blocks, Bq):
    """max-abs and mean-abs of the device output against the oracle on the given blocks."""
    import numpy as np
    N = dev_O.shape[1]
    rows = np.concatenate([np.arange(i * Bq, min((i + 1) * Bq, N)) for i in blocks])
    got = dev_O[:, rows].float().cpu().numpy()
    e = np.abs(got - oracle_out)
    return {"max_abs": float(e.max()), "mean_abs": float(e.mean())}


def device_out_fp32(w, mode, **kw):
    """One call of workload w with a float32 output (for the comparison with the oracle)."""
    import torch
    from block_sparse_long_amd import _lib
    O = torch.empty(w.Qd.shape, dtype=torch.float32, device=w.Qd.device)
    _lib.bsfa_prefill(w.Qd, w.Kd, w.Vd, O, block_q=w.Bq, block_k=w.Bk, gate_mode=mode,
                      table=kw.pop("table", w.dtable if mode == "absolute" else None), **kw)
    torch.cuda.synchronize()
    return O


def gate_row(r, dense_ms, N, Bq, k=None, Bk=64):
    row = {"ms": round(r["ms"], 4), "tflops": round(r["tflops"], 2),
           "pct_mfma_peak": round(r["pct_peak"], 2),
           "speedup_vs_dense": round(dense_ms / r["ms"], 4),
           "kept_fraction": round(r["kept_fraction"], 4)}
    if k is not None:
        row["predicted_density"] = round(predicted_density(N, Bq, k, Bk), 4)
    return row


def config_rows(name, dev, steps, warmup, oracle_run=None, slice_for_oracle=0):
    """Configs 1-3 of the workload list: dense and every budget slice (both ways of running the
    absolute gate where they differ), and the oracle's full-size time and output deviation."""
    import numpy as np
    import torch
    from block_sparse_long_amd.table import ThresholdTable
    w = Workload(name, dev, host=None if oracle_run is None else oracle_run["host"])
    d = run_gate(w, "dense", steps, warmup)
    rows = {"dense": {"ms": round(d["ms"], 4), "tflops": round(d["tflops"], 2),
                      "pct_mfma_peak": round(d["pct_peak"], 2)}}
    none = torch.empty(0, dtype=torch.uint8, device=dev)
    for sl, kk in enumerate(w.table.budgets):
        r = run_gate(w, "absolute", steps, warmup, budget_slice=sl)
        row = gate_row(r, d["ms"], w.N, w.Bq, kk, w.Bk)
        # the library's choice against both ways forced: two launches (table without its
        # budgets) and one launch (no workspace)
        two = run_gate(w, "absolute", steps, warmup, budget_slice=sl,
                       table=w.table.to_device(dev, record_budgets=False))
        one = run_gate(w, "absolute", steps, warmup, budget_slice=sl, workspace=none)
        row["two_launches_ms"] = round(two["ms"], 4)
        row["one_launch_ms"] = round(one["ms"], 4)
        rows[f"k={kk}"] = row
    if name == "tiny_1k":
        for label, v in (("T=-inf", -np.inf), ("T=+inf", np.inf)):
            T = np.full_like(w.table.T[:1], v)
            tab = ThresholdTable(T=T, budgets=[0], block_q=w.Bq, block_k=w.Bk, head_dim=w.d,
                                 softmax_scale=w.table.softmax_scale).to_device(dev)
            r = run_gate(w, "absolute", steps, warmup, table=tab)
            rows[label] = gate_row(r, d["ms"], w.N, w.Bq)
    if oracle_run is not None:
        sec, counts, out, cores = (oracle_run[x] for x in ("sec", "counts", "out", "cores"))
        fl = executed_flops(np.maximum(counts, 0), w.N, w.Bq, w.d, w.Bk)
        O = device_out_fp32(w, "absolute", budget_slice=slice_for_oracle)
        rows["oracle"] = {"budget_k": w.table.budgets[slice_for_oracle], "seconds": round(sec, 2),
                          "cores": cores, "tflops": round(fl / sec / 1e12, 6),
                          "kind": "oracle, whole workload",
                          "device_vs_oracle": deviation(O, out, range(-(-w.N // w.Bq)), w.Bq)}
        del O
    del w
    torch.cuda.empty_cache()
    return rows


def dialled_rows(dev, steps, warmup):
    """The relative gate on the 64K workload whose skip rate its generator dials (cold key
    blocks): kept fraction, time and speed-up over dense per skip rate at lambda = 1e-3, and
    the lambda grid at a 50 % skip rate."""
    import torch
    from block_sparse_long_amd import synth
    c = synth.CONFIGS["llama_64k_dial"]
    out = {}
    for skip in [0.0] + list(c["skips"]):
        w = Workload("llama_64k_dial", dev, skip=skip)
        d = run_gate(w, "dense", steps, warmup)
        row = {"dense_ms": round(d["ms"], 3)}
        lams = (0.0, 1e-4, 1e-3, 1e-2) if skip == c["skip"] else (0.0, 1e-3)
        for lam in lams:
            r = run_gate(w, "relative", steps, warmup,
                         log_lambda=math.log(lam) if lam else -math.inf)
            row[f"lambda={lam:g}"] = gate_row(r, d["ms"], w.N, w.Bq)
        out[f"skip={skip:g}"] = row
        del w
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(the attention shards by KV head with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    if args.profile_once:
        profile_once(args)
        return
    if args.counters:
        summarise_counters(args)
        return
    import numpy as np
    from block_sparse_long_amd import synth
    from block_sparse_long_amd.table import ThresholdTable

    c = synth.CONFIGS[args.workload]
    k = c["budgets"][0] if c["budgets"] else None
    mode = "absolute" if c["budgets"] else "relative"
    gate_kw = dict(budget_slice=0) if mode == "absolute" else dict(log_lambda=math.log(1e-3))
    N, Bq, Bk = c["n"], c["block_q"], c["block_k"]

    # ---- CPU phase: the oracle on the host cores, before anything touches the GPU ----
    host_main = synth.to_bf16(*synth.make_inputs(args.workload, 0))
    cpu, oracle_main, oracle_cfg = None, None, {}
    if not args.no_cpu_baseline:
        T = (ThresholdTable.load(os.path.join(GOLDEN, f"thresholds_{args.workload}.bin")).T
             if mode == "absolute" else None)
        blocks = sample_blocks(-(-N // Bq), k)
        sec, counts, out, cores = oracle_timed(host_main, T, Bq, Bk, mode, blocks,
                                               log_lambda=gate_kw.get("log_lambda", -math.inf))
        fl = executed_flops(np.maximum(counts, 0), N, Bq, c["d"], Bk, query_blocks=blocks)
        cpu = {"value": round(fl / sec / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
               "kind": "oracle", "seconds": round(sec, 2),
               "sample": f"{args.workload}: query blocks {blocks} ({len(blocks)} of "
                         f"{-(-N // Bq)}) x all {c['heads_q']} heads, same inputs and table, "
                         f"float32 numpy, one process per head on {cores} host cores, one BLAS "
                         f"thread each; executed TFLOP/s of the sample",
               **cpu_info()}
        oracle_main = dict(blocks=blocks, out=out)
        if not args.quick:
            # configs 1-3 in full (32K at k = 64)
            for name, sl in (("tiny_1k", 0), ("llama_16k", 0), ("llama_32k_sweep", 1)):
                cc = synth.CONFIGS[name]
                host = synth.to_bf16(*synth.make_inputs(name, 0))
                Tn = ThresholdTable.load(os.path.join(GOLDEN, f"thresholds_{name}.bin")).T
                nb = -(-cc["n"] // cc["block_q"])
                sec, counts, out, cores = oracle_timed(host, Tn, cc["block_q"], cc["block_k"],
                                                       "absolute", range(nb), budget_slice=sl)
                oracle_cfg[name] = dict(host=host, sec=sec, counts=counts, out=out, cores=cores,
                                        slice=sl)

    # ---- GPU phase ----
    import torch
    from block_sparse_long_amd import _lib
    _lib.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    w = Workload(args.workload, dev, host=host_main)
    gated = run_gate(w, mode, args.steps, args.warmup, **gate_kw)
    sweep = run_sweep(w, args.steps, args.warmup) if mode == "absolute" else None
    dense = run_gate(w, "dense", args.steps, args.warmup)
    # zero-skip taxes: the gated instantiations with a gate that never skips, each against
    # dense calls made in alternation with it (three rounds)
    tax_steps = max(2, args.steps // 3)
    if w.table is not None:
        T = np.full_like(w.table.T[:1], -np.inf)
        ninf = ThresholdTable(T=T, budgets=[0], block_q=w.table.block_q, block_k=64,
                              head_dim=w.d, softmax_scale=w.table.softmax_scale).to_device(dev)
        tax_abs, _ = paired_tax(w, "absolute", 3, tax_steps, 1, table=ninf)
    tax_rel, _ = paired_tax(w, "relative", 3, tax_steps, 1, log_lambda=-math.inf)
    extras = {
        "gated_ms": round(gated["ms"], 3), "dense_ms": round(dense["ms"], 3),
        "speedup_vs_dense": round(dense["ms"] / gated["ms"], 4),
        "executed_tflops": round(gated["tflops"], 2),
        "pct_mfma_peak": round(gated["pct_peak"], 2),
        "dense_tflops": round(dense["tflops"], 2),
        "dense_pct_mfma_peak": round(dense["pct_peak"], 2),
        "dense_textbook_tflops": round(4.0 * w.N * w.N / 2 * w.Hq * w.d / dense["ms"] / 1e9, 2),
        "kept_fraction": round(gated["kept_fraction"], 4),
        "predicted_density": round(predicted_density(w.N, w.Bq, k), 4) if k else None,
        "zero_skip_tax_relative": round(tax_rel, 4),
    }
    if w.table is not None:
        extras["zero_skip_tax_absolute"] = round(tax_abs, 4)
    if oracle_main is not None:
        O = device_out_fp32(w, mode, **dict(gate_kw))
        extras["device_vs_oracle_sample"] = deviation(O, oracle_main["out"],
                                                      oracle_main["blocks"], w.Bq)
        del O
    # the same gated call with L2 and the last-level cache flushed before each call (median)
    extras["gated_ms_flushed_median"] = round(flushed_median_ms(w, mode, **gate_kw), 3)
    # executed TFLOP/s against the matrix cores' measured sustained rate as well as the spec
    rate = measured_mfma_rate()
    extras["measured_mfma_tflops"] = round(rate, 1)
    extras["pct_measured_mfma_peak"] = round(100.0 * gated["tflops"] / rate, 2)
    # the call's launches: under the absolute gate the sweep, then the walk over kept tiles
    # (QK again and PV on every kept and diagonal tile)
    walk_tiles = gated["kept"] + w.Hq * sum(
        n_end - n_off for n_off, n_end in block_ranges(w.N, w.Bq))
    walk_flops = 2 * 2.0 * w.Bq * 64 * w.d * walk_tiles
    if sweep is not None:
        walk_ms = gated["ms"] - sweep["ms"]
        extras["launches"] = {
            "gate_sweep": {"ms": round(sweep["ms"], 3), "tflops": round(sweep["tflops"], 2),
                           "flops": sweep["flops"]},
            "softmax_walk": {"ms": round(walk_ms, 3), "flops": walk_flops,
                             "tflops": round(walk_flops / walk_ms / 1e9, 2)}}
        # kernel names as the profiler reports them (template arguments: head dim, query tile,
        # heads or waves per workgroup, gate, paged K/V, mean correction)
        if sweep["ms"] >= walk_ms:
            dom = dict(kernel=f"gate_sweep_kernel<{w.d}, {w.Bq}, 2, false>", ms=sweep["ms"],
                       flops=sweep["flops"])
        else:
            dom = dict(kernel=f"prefill_kernel<{w.d}, {w.Bq}, 4, 1, false, false>", ms=walk_ms,
                       flops=walk_flops)
    else:
        dom = dict(kernel=f"prefill_kernel<{w.d}, {w.Bq}, 4, {2 if mode == 'relative' else 0}, "
                          "false, false>", ms=gated["ms"], flops=gated["flops"])
    if w.table is not None:
        extras["mean_correction"] = run_mean_correction(w, args.steps, args.warmup, gated["ms"],
                                                        dense["ms"])
        fp8 = run_fp8_gate(w, args.steps, args.warmup, gated, dense["ms"])
        if fp8 is not None:
            extras["fp8_gate"] = fp8

    if not args.quick and w.table is not None:
        # chunked prefill of the same sequence (chunks of 16K after their KV prefix)
        ch = run_chunked(w, 16384, args.steps, args.warmup)
        extras["chunked_16k"] = {"ms": round(ch["ms"], 3), "chunks": ch["chunks"],
                                 "tflops": round(ch["tflops"], 2),
                                 "kept_blocks": ch["kept"], "kept_blocks_whole_call": gated["kept"],
                                 "vs_whole_call": round(ch["ms"] / gated["ms"], 4)}
    line_cfg = {"workload": args.workload, "batch": 1, "seq_len": w.N,
                "heads_q": c["heads_q"], "heads_kv": c["heads_kv"], "head_dim": w.d,
                "tile": f"{w.Bq}x64", "gate": mode,
                "budget_k": k, "calibrated_len": c["calib_n"] if k else None}
    del w
    torch.cuda.empty_cache()
    if not args.quick:
        # configs 1-3 (tiny 1K, 16K k = 32, the 32K budget sweep), with the oracle's full-size
        # runs from the CPU phase
        cfg = {}
        for name in ("tiny_1k", "llama_16k", "llama_32k_sweep"):
            orc = oracle_cfg.get(name)
            cfg[name] = config_rows(name, dev, args.steps, args.warmup, orc,
                                    orc["slice"] if orc else 0)
        oracle_cfg.clear()
        extras["configs"] = cfg
        sweeps = {}
        wb = Workload("llama_32k_bk128", dev)
        d32 = cfg["llama_32k_sweep"]["dense"]["ms"]
        rows = {}
        for sl, kk in enumerate(wb.table.budgets):
            r = run_gate(wb, "absolute", args.steps, args.warmup, budget_slice=sl)
            rows[f"k={kk}"] = gate_row(r, d32, wb.N, wb.Bq, kk, 128)
        sweeps["llama_32k_bk128"] = rows
        del wb
        torch.cuda.empty_cache()
        w64 = Workload("llama_64k_relative", dev)
        d64 = run_gate(w64, "dense", args.steps, args.warmup)
        rows = {"dense": {"ms": round(d64["ms"], 3), "tflops": round(d64["tflops"], 2)}}
        for lam in (0.0, 1e-4, 1e-3, 1e-2):
            ll = math.log(lam) if lam > 0 else -math.inf
            r = run_gate(w64, "relative", args.steps, args.warmup, log_lambda=ll)
            rows[f"lambda={lam:g}"] = gate_row(r, d64["ms"], w64.N, w64.Bq)
        # the zero-skip tax as at 128K, from alternating rounds of dense and gated calls: at
        # lambda = 0 and at 1e-4, which keeps every block of this workload with the gate
        # deciding each one
        rows["zero_skip_tax_alternating_rounds"] = {
            f"lambda={lam:g}": round(paired_tax(w64, "relative", 3, args.steps, 1,
                                                log_lambda=math.log(lam) if lam > 0
                                                else -math.inf)[0], 4)
            for lam in (0.0, 1e-4)}
        sweeps["llama_64k_relative"] = rows
        del w64
        torch.cuda.empty_cache()
        sweeps["llama_64k_dial"] = dialled_rows(dev, args.steps, args.warmup)
        extras["sweeps"] = sweeps

    line = {
        "metric": METRIC, "value": round(gated["tflops"], 3), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(gated["wall_ms"], 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": line_cfg,
        "roofline": {"bound": "mfma", "achieved": round(dom["flops"] / dom["ms"] / 1e9, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(dom["flops"] / dom["ms"] / 1e9 / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(args.workload, dom["kernel"]),
                     "kernel": dom["kernel"], "ms_per_launch": round(dom["ms"], 3),
                     "flops_per_launch": dom["flops"],
                     # from the committed counter runs of the same kernel source (else null):
                     # MFMA-busy share of SIMD cycles and the MFMA FLOPs the hardware counted
                     "mfma_util_pct": measured_counters(args.workload, dom["kernel"]).get(
                         "mfma_util_pct"),
                     "mfma_flops_counted": measured_counters(args.workload, dom["kernel"]).get(
                         "mfma_flops_bf16"),
                     # the measured HBM traffic over this run's launch time (GB/s), or null
                     "hbm_gbs": (None if measured_traffic(args.workload, dom["kernel"]) is None
                                 else round(measured_traffic(args.workload, dom["kernel"])
                                            / dom["ms"] / 1e6, 1))},
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
