"""Seeded synthetic inputs for gated prefill attention.

This module holds input generation only: it computes none of the attention method's
arithmetic. Both the HIP path and the CPU oracle are fed from it (the oracle never imports it;
callers pass it arrays).

The pages measure on long-document benchmarks and trained models that are not available
here; these generators stand in for them with the attention shapes the pages use (Llama-3.1-8B:
32 query heads, 8 KV heads, head_dim 128) and with the score structures the pages name:
initial attention-sink positions and remote relevant content ("Block Sparse Flash Attention",
Method > Key Designs 1), single-needle retrieval (Key Experimental Results).

Determinism: every tensor is drawn in fixed-size chunks, each from its own torch CPU generator
seeded by a 64-bit mix of (seed, stream, chunk). Results do not depend on the number of threads.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import torch

_CHUNK = 1 << 22
_MASK64 = (1 << 64) - 1


def _mix(*vals: int) -> int:
    """splitmix64 over a sequence of integers -> a 63-bit seed."""
    x = 0x9E3779B97F4A7C15
    for v in vals:
        x = (x + (int(v) & _MASK64) + 0x9E3779B97F4A7C15) & _MASK64
        z = x
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        x = z ^ (z >> 31)
    return x & ((1 << 63) - 1)


def normal(shape, seed: int, stream: int, threads: int = 8) -> torch.Tensor:
    """float32 N(0, 1) tensor of ``shape`` on the CPU, reproducible from (seed, stream)."""
    numel = 1
    for s in shape:
        numel *= int(s)
    out = torch.empty(numel, dtype=torch.float32)
    n_chunks = (numel + _CHUNK - 1) // _CHUNK

    def fill(c: int) -> None:
        g = torch.Generator().manual_seed(_mix(seed, stream, c))
        lo = c * _CHUNK
        hi = min(numel, lo + _CHUNK)
        out[lo:hi].normal_(generator=g)

    if n_chunks <= 1:
        for c in range(n_chunks):
            fill(c)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out.view(*shape)


def _unit(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm()


def tiny_single_head(seed: int, n: int = 1024, d: int = 64, sinks: int = 4,
                     sink_norm: float = 4.0):
    """Q, K, V ~ N(0, 1), shape [1, n, 1, d], float32, plus ``sinks`` sink keys.

    The sink keys at positions 0..sinks-1 point along the mean query direction with norm
    sink_norm * sqrt(d) (sink_norm times the expected key norm).
    """
    Q = normal((1, n, 1, d), seed, 1)
    K = normal((1, n, 1, d), seed, 2)
    V = normal((1, n, 1, d), seed, 3)
    u = _unit(Q[0, :, 0, :].mean(dim=0))
    K[0, :sinks, 0, :] = sink_norm * math.sqrt(d) * u
    return Q, K, V


def structured(seed: int, n: int, heads_q: int = 32, heads_kv: int = 8, d: int = 128,
               rank: int = 4, weight: float = 0.5, sinks: int = 4, sink_norm: float = 4.0,
               needles: int = 32, cosine: float = 0.8):
    """Llama-3.1-8B-shaped single-layer Q, K, V, float32 on the CPU.

    Q: [1, n, heads_q, d]; K, V: [1, n, heads_kv, d].
      * Z ~ N(0, 1) for Q and K; V ~ N(0, 1).
      * a shared rank-``rank`` component per KV group g: W_g ~ N(0,1)^{rank x d}; per token and
        head C ~ N(0,1)^rank; Q_h += weight * C_q W_g, K_g += weight * C_k W_g.
      * ``sinks`` sink keys per KV group at positions 0.., along the unit mean of the group's
        queries, norm sink_norm * sqrt(d).
      * ``needles`` needle keys per KV group: position p in [sinks, n - 1), a query row r in
        (p, n) and a query head h of the group; K[p, g] keeps its norm and is turned to
        cosine * q_hat(r, h) + sqrt(1 - cosine^2) * e, e a random unit vector orthogonal to
        q_hat.
    """
    G = heads_q // heads_kv
    Q = normal((1, n, heads_q, d), seed, 1)
    K = normal((1, n, heads_kv, d), seed, 2)
    V = normal((1, n, heads_kv, d), seed, 3)
    W = normal((heads_kv, rank, d), seed, 4)
    Cq = normal((1, n, heads_q, rank), seed, 5)
    Ck = normal((1, n, heads_kv, rank), seed, 6)
    for g in range(heads_kv):
        hs = slice(g * G, (g + 1) * G)
        Q[:, :, hs, :] += weight * torch.matmul(Cq[:, :, hs, :], W[g])
        K[:, :, g, :] += weight * torch.matmul(Ck[:, :, g, :], W[g])
    for g in range(heads_kv):
        u = _unit(Q[0, :, g * G:(g + 1) * G, :].mean(dim=(0, 1)))
        K[0, :sinks, g, :] = sink_norm * math.sqrt(d) * u
    gen = torch.Generator().manual_seed(_mix(seed, 7))
    ortho = math.sqrt(max(0.0, 1.0 - cosine * cosine))
    if n - 1 > sinks:
        for g in range(heads_kv):
            for _ in range(needles):
                p = int(torch.randint(sinks, n - 1, (1,), generator=gen))
                r = int(torch.randint(p + 1, n, (1,), generator=gen))
                h = g * G + int(torch.randint(0, G, (1,), generator=gen))
                qh = _unit(Q[0, r, h, :].clone())
                e = torch.randn(d, generator=gen)
                e = _unit(e - (e @ qh) * qh)
                K[0, p, g, :] = K[0, p, g, :].norm() * (cosine * qh + ortho * e)
    return Q, K, V


def dialled(seed: int, n: int, skip: float, heads_q: int = 32, heads_kv: int = 8, d: int = 128,
            shift: float = 6.0, depth: float = 4.0, noise: float = 0.25, block: int = 64):
    """The structured generator (without sinks) with a dialled share of negligible key blocks,
    for the relative gate: the skip rate is an input of the workload ("Skipping attention
    blocks was the easy part", BLASST blog, The scoreboard: sparsity dialled synthetically).

      * every query of KV group g gets a shared component ``shift`` * u_g along a unit
        direction u_g of its group (queries of a group share a dominant direction), and a
        query whose component along u_g is still below shift / 2 is moved along u_g up to
        shift / 2 (so that the claim below holds for every row, not just typical ones);
      * each key block j >= 1 of group g (``block`` keys) is cold with probability ``skip``
        (a seeded draw per (g, j)); a cold block's keys are -depth * sqrt(d) * u_g +
        ``noise`` * N(0, 1): every query scores at most about -depth * shift / 2 = -12
        against them (typically -24),
        far below the running max the first (never cold) block already sets, so every row's
        block max sits more than |ln lambda| below its running max for lambda >= 1e-4 and the
        relative gate skips the block; the other blocks keep their maxima near the running max
        and are kept;
      * values are unchanged.

    Returns (Q, K, V, cold) with cold a bool tensor [heads_kv, ceil(n / block)].
    """
    Q, K, V = structured(seed, n, heads_q=heads_q, heads_kv=heads_kv, d=d, sinks=0)
    G = heads_q // heads_kv
    U = normal((heads_kv, d), seed, 8)
    U = U / U.norm(dim=1, keepdim=True)
    nb = -(-n // block)
    gen = torch.Generator().manual_seed(_mix(seed, 9))
    cold = torch.rand((heads_kv, nb), generator=gen) < skip
    cold[:, 0] = False
    Z = normal((1, n, heads_kv, d), seed, 10)
    for g in range(heads_kv):
        Qg = Q[0, :, g * G:(g + 1) * G, :]
        Qg += shift * U[g]
        Qg += torch.clamp(0.5 * shift - Qg @ U[g], min=0.0)[..., None] * U[g]
        for j in torch.nonzero(cold[g]).flatten().tolist():
            r = slice(j * block, min(n, (j + 1) * block))
            K[0, r, g, :] = -depth * math.sqrt(d) * U[g] + noise * Z[0, r, g, :]
    return Q, K, V, cold


def uniform_mix(seed: int, b: int, n: int, heads_q: int, heads_kv: int, d: int):
    """Plain N(0, 1) Q, K, V with batch ``b`` (parity cases with no structure)."""
    return (normal((b, n, heads_q, d), seed, 1), normal((b, n, heads_kv, d), seed, 2),
            normal((b, n, heads_kv, d), seed, 3))


def to_bf16(*xs: torch.Tensor):
    """Round-to-nearest-even to bfloat16 (the values the device path consumes)."""
    r = tuple(x.to(torch.bfloat16) for x in xs)
    return r if len(r) > 1 else r[0]


CONFIGS = {
    # name: (generator kwargs, tile, calibration budgets, calibration length)
    "tiny_1k": dict(kind="tiny", n=1024, heads_q=1, heads_kv=1, d=64, block_q=64, block_k=64,
                    budgets=[4], calib_n=1024, calib_seeds=[1, 2, 3, 4]),
    "llama_16k": dict(kind="structured", n=16384, heads_q=32, heads_kv=8, d=128, block_q=128,
                      block_k=64, budgets=[32], calib_n=16384, calib_seeds=list(range(1, 9))),
    "llama_32k_sweep": dict(kind="structured", n=32768, heads_q=32, heads_kv=8, d=128,
                            block_q=128, block_k=64, budgets=[16, 64, 256], calib_n=32768,
                            calib_seeds=list(range(1, 9))),
    # the 32K sweep with 128-key tiles: the same key budgets (8, 32, 128 blocks of 128 keys)
    "llama_32k_bk128": dict(kind="structured", n=32768, heads_q=32, heads_kv=8, d=128,
                            block_q=128, block_k=128, budgets=[8, 32, 128], calib_n=32768,
                            calib_seeds=list(range(1, 9))),
    "llama_128k": dict(kind="structured", n=131072, heads_q=32, heads_kv=8, d=128, block_q=128,
                       block_k=64, budgets=[64], calib_n=65536, calib_seeds=list(range(1, 9))),
    # the 128K workload under the FP8 gate: its thresholds calibrated on FP8 scores
    "llama_128k_fp8": dict(kind="structured", n=131072, heads_q=32, heads_kv=8, d=128,
                           block_q=128, block_k=64, budgets=[64], calib_n=65536,
                           calib_seeds=list(range(1, 9)), gate_dtype="fp8"),
    "llama_64k_relative": dict(kind="structured", n=65536, heads_q=32, heads_kv=8, d=128,
                               block_q=128, block_k=64, budgets=[], calib_n=0, calib_seeds=[],
                               log_lambdas=[-math.inf, math.log(1e-4), math.log(1e-3),
                                            math.log(1e-2)]),
    # the relative-gate workload with its skip rate dialled by the generator (cold key blocks)
    "llama_64k_dial": dict(kind="dialled", n=65536, heads_q=32, heads_kv=8, d=128, block_q=128,
                           block_k=64, budgets=[], calib_n=0, calib_seeds=[],
                           skips=[0.25, 0.5, 0.75, 0.95], skip=0.5,
                           log_lambdas=[-math.inf, math.log(1e-4), math.log(1e-3),
                                        math.log(1e-2)]),
}


def make_inputs(config: str, seed: int, n: int | None = None, skip: float | None = None):
    """float32 CPU (Q, K, V) for a named workload at its length (or ``n``; a dialled workload
    at its default skip rate or ``skip``)."""
    c = CONFIGS[config]
    n = c["n"] if n is None else n
    if c["kind"] == "tiny":
        return tiny_single_head(seed, n=n, d=c["d"])
    if c["kind"] == "dialled":
        return dialled(seed, n, c["skip"] if skip is None else skip, heads_q=c["heads_q"],
                       heads_kv=c["heads_kv"], d=c["d"])[:3]
    return structured(seed, n, heads_q=c["heads_q"], heads_kv=c["heads_kv"], d=c["d"])
