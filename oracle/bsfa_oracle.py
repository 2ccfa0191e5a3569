"""CPU oracle for exact-score-gated block-sparse causal prefill attention (BSFA).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute this
module: only the test suite, the entry point's smoke check and the benchmark's CPU-baseline
leg use it. It shares no code, constants or helpers with the HIP library.

It is deliberately plain and slow: one (batch, head, query block) at a time, one key block at a
time, in the order the method describes, with numpy doing each matrix product. Floating point
is float32 by default (the precision the oracle is asked to compute in); pass
``dtype=np.float64`` for a float64 run.

Sources (page title, then the part of the page followed):
  * "Block Sparse Flash Attention" (paper notes), Method:
      - Overall Architecture: inputs Q, K, V and the threshold slice of the chosen budget; the
        output is renormalised over the retained blocks; the causal diagonal region always goes
        to aggregation.
      - Key Designs 1 (Offline Threshold Calibration): k-th highest visible off-diagonal block
        maximum per sample, averaged over samples; -inf where fewer than k candidates exist;
        positions past the calibrated length reuse the last calibrated position.
      - Key Designs 2 (Exact-Score Gating), keep-rule equation: s_max over the whole query-key
        score tile of scaled pre-softmax scores; keep iff s_max >= T.
      - Key Designs 3 (Selective Streaming Aggregation): online softmax on kept blocks; a
        rejected block touches neither V, nor the exponentials, nor m, l, O.
      - A Worked Example.
  * "FlashPrefill V2: Block-Sparse Prefill Attention for Long-Context LLM Serving", mean
    correction (a pruned block J stands in as |B_J| copies of its mean key and mean value:
    |B_J| e^{s_J} vbar_J joins the numerator and |B_J| e^{s_J} the denominator, i.e. one more
    online-softmax step on a single logit shifted by log|B_J|).
  * FP8 (e4m3) scores for the gate (FlashPrefill V2's FP8 path quantises on the fly; the
    format is OCP FP8 E4M3: 4 exponent bits with bias 7, 3 mantissa bits, largest finite value
    448, subnormal spacing 2^-9, no infinities).
  * "Skipping attention blocks was the easy part" (BLASST blog), sections "FlashAttention"
    (running max m, running sum l, accumulator O, rescale by exp(m_old - m_new)) and
    "Vote, then skip" (skip iff block max minus running max < ln(lambda); any row that wants
    the block vetoes the skip).

Readings taken where the pages are silent or ambiguous (each is listed in the design notes):
  * keep uses ">=" (the paper notes follow the main text; the simplified algorithm uses ">").
  * Off-diagonal key blocks of query block i are the blocks wholly before the block's first
    row, j < n_off(i) = floor(i*Bq/Bk); the diagonal region is n_off(i) <= j < n_end(i).
  * Key blocks are visited in ascending order, so the diagonal region comes last.
  * Thresholds are per query head; GQA maps query head h to KV head h // G.
  * The relative gate compares max over the tile's rows of (row max of the block - running row
    max before the block) with ln(lambda); lambda = 0 means never skip.
  * Rows past the end of a ragged last block do not exist (blocks are clipped to N).
  * Chunked prefill: a chunk of N_q query rows follows a prefix of P = N_k - N_q keys (its rows
    sit at absolute positions P .. N_k - 1). Query block i then starts at absolute row
    P + i*Bq, the causal mask and n_off / n_end use absolute positions, and the absolute gate
    reads the threshold column of the absolute query block P/Bq + i, which needs P to be a
    multiple of Bq (thresholds are bound to the calibration's tile grid).
  * Mean correction: the stand-in logit of a pruned block is the scaled score of the row's query
    against the block's mean key, s_J = scale * q . kbar_J (the means are plain arithmetic
    means over the block's keys and values); only pruned off-diagonal blocks are corrected (the
    diagonal region always runs exactly); the stand-in step takes the pruned block's place in
    the ascending block order. It is defined for the absolute gate (whose decisions do not
    depend on the softmax state), not for the relative gate.

  * FP8 gate: only the gate statistic of off-diagonal blocks uses FP8 scores; the softmax
    and the output use the exact scores of the kept blocks. Q is quantised per (token, head)
    row and K per (64-key tile, KV head), each with scale amax / 448 (codes = x * (448 / amax)
    rounded to nearest even, all in float32; an all-zero row or tile has codes 0 and scale 0),
    and a score is (q8 . k8) * scale_q(row) * scale_k(tile) * softmax_scale.

Pins (tests that tie each function to something other than itself) are in
tests/test_oracle_pins.py; every public function here is pinned.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

GATE_DENSE = "dense"
GATE_ABSOLUTE = "absolute"
GATE_RELATIVE = "relative"
_MODES = (GATE_DENSE, GATE_ABSOLUTE, GATE_RELATIVE)


def num_blocks(n: int, block: int) -> int:
    """Number of blocks of size ``block`` covering ``n`` positions (the last one may be short)."""
    return (n + block - 1) // block


def key_block_range(i: int, n: int, block_q: int, block_k: int,
                    prefix: int = 0) -> tuple[int, int]:
    """(n_off, n_end) for query block i of a causal prefill of n query rows that follow
    ``prefix`` earlier keys (rows at absolute positions prefix .. prefix + n - 1).

    Key blocks j < n_off lie wholly before the query block's first row, so every pair in them is
    visible: these are the off-diagonal candidates the gate acts on. Blocks n_off <= j < n_end
    hold the causal diagonal region (they need the causal mask and always run); blocks at or
    past n_end are invisible to every row of the block. ("Block Sparse Flash Attention",
    Method > Key Designs 2, on the causal diagonal region and on unequal tile shapes.)
    """
    n_off = (prefix + i * block_q) // block_k
    last_row = prefix + min((i + 1) * block_q, n) - 1
    n_end = last_row // block_k + 1
    return n_off, n_end


def effective_threshold(table: np.ndarray, budget_slice: int, h: int, i: int) -> float:
    """T_eff(h, i) = T[slice][h][min(i, T_len - 1)].

    Query blocks past the calibrated length reuse the final calibrated position's threshold
    ("Block Sparse Flash Attention", Method > Key Designs 1, last paragraph).
    """
    t_len = table.shape[2]
    return float(table[budget_slice, h, min(i, t_len - 1)])


@dataclass
class OracleResult:
    out: np.ndarray          # [B, Nq, Hq, d]; NaN rows for query blocks not computed
    kept_counts: np.ndarray  # [B, Hq, nqb] int64, kept OFF-diagonal blocks; -1 if not computed
    stat: np.ndarray         # [B, Hq, nqb, nkb] (nkb over Nk) gate statistic per visible block
    keep: np.ndarray         # [B, Hq, nqb, nkb] bool; True for kept blocks and the diagonal region
    margin: np.ndarray       # [B, Hq, nqb, nkb] stat - threshold (off-diagonal only); NaN elsewhere


E4M3_MAX = 448.0


def quantize_e4m3(x) -> np.ndarray:
    """Round float32 values to the nearest E4M3 value (ties to even), saturating at +-448.

    E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; normal values 2^e (1 + m/8) for
    e = -6 .. 8 (the largest finite one 448 = 2^8 * 1.75), subnormals m * 2^-9. The grid step
    near |x| is 2^(max(e, -6) - 3) with e = floor(log2 |x|); rounding to that step is exact in
    float64 and numpy rounds halves to even. Returns float32. (Elementwise; done in slices of
    2^20 values so that the float64 temporaries stay small.)
    """
    x = np.asarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.float32)
    src, dst = x.reshape(-1), out.reshape(-1)
    for s0 in range(0, src.size, 1 << 20):
        v = src[s0:s0 + (1 << 20)].astype(np.float64)
        a = np.abs(v)
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
        step = np.exp2(np.maximum(e, -6.0) - 3.0)
        q = np.minimum(np.round(a / step) * step, E4M3_MAX)
        dst[s0:s0 + (1 << 20)] = np.sign(v) * q
    return out


def _e4m3_codes(x, amax):
    """Codes of x (float32) against a float32 amax (broadcast): x * (448 / amax), rounded; and
    the scale amax / 448. amax == 0 gives codes 0 and scale 0."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.asarray(amax, dtype=np.float32)
    safe = np.where(amax > 0, amax, np.float32(1))
    inv = np.where(amax > 0, np.float32(E4M3_MAX) / safe, np.float32(0)).astype(np.float32)
    lim = np.float32(E4M3_MAX)
    y = np.minimum(np.maximum((x * inv).astype(np.float32), -lim), lim)
    scale = np.where(amax > 0, safe / np.float32(E4M3_MAX), np.float32(0)).astype(np.float32)
    return quantize_e4m3(y), scale


def quantize_q_rows(Q):
    """FP8 copy of Q [B, N, Hq, d]: codes [B, N, Hq, d] (float32 values of E4M3) and one scale
    per (b, token, head) row, [B, N, Hq]."""
    Q = np.asarray(Q, dtype=np.float32)
    amax = np.abs(Q).max(axis=-1)
    codes, scale = _e4m3_codes(Q, amax[..., None])
    return codes, scale[..., 0]


def quantize_k_tiles(K, tile: int = 64):
    """FP8 copy of K [B, Nk, Hkv, d]: codes [B, Nk, Hkv, d] and one scale per (b, 64-key tile,
    KV head), [B, ceil(Nk / 64), Hkv] (a last short tile uses its own keys)."""
    K = np.asarray(K, dtype=np.float32)
    B, Nk, Hkv, d = K.shape
    nt = num_blocks(Nk, tile)
    codes = np.zeros_like(K)
    scales = np.zeros((B, nt, Hkv), dtype=np.float32)
    for t in range(nt):
        c0, c1 = t * tile, min((t + 1) * tile, Nk)
        amax = np.abs(K[:, c0:c1]).max(axis=(1, 3))                    # [B, Hkv]
        codes[:, c0:c1], sc = _e4m3_codes(K[:, c0:c1], amax[:, None, :, None])
        scales[:, t] = sc[:, 0, :, 0]
    return codes, scales


def oracle_prefill(Q, K, V, *, block_q: int, block_k: int, mode: str,
                   scale: float | None = None, table: np.ndarray | None = None,
                   budget_slice: int = 0, log_lambda: float = -math.inf,
                   forced_keep: np.ndarray | None = None, band: float = 1e-2,
                   query_blocks=None, mean_correction: bool = False,
                   gate_dtype: str = "bf16", dtype=np.float32) -> OracleResult:
    """Gated causal prefill attention, one (b, h, i) work unit at a time.

    Q: [B, Nq, Hq, d]; K, V: [B, Nk, Hkv, d] with Nk >= Nq and Hq % Hkv == 0. The query rows
    are the last Nq positions of the sequence (a chunk after a prefix of P = Nk - Nq keys; P = 0
    is a whole prefill).
    mode: "dense" (keep everything), "absolute" (keep iff s_max >= T_eff(h, i) from ``table``
    [n_budgets][Hq][T_len] at ``budget_slice``) or "relative" (keep iff
    max_r(rowmax_j[r] - m[r]) >= log_lambda).
    forced_keep: optional [B, Hq, nqb, nkb] decisions adopted where |margin| <= band (the
    near-tie rule used when comparing against a device that rounds differently).
    query_blocks: optional iterable of query-block indices to compute (default: all).
    mean_correction: a pruned block adds its zero-order stand-in (FlashPrefill V2's mean
    correction) instead of nothing.
    gate_dtype: "bf16" (the exact scores) or "fp8" (the absolute gate's off-diagonal block
    maxima from E4M3 copies of Q and K; see quantize_q_rows / quantize_k_tiles).
    """
    if mode not in _MODES:
        raise ValueError(f"unknown gate mode {mode!r}")
    Q = np.asarray(Q, dtype=dtype)
    K = np.asarray(K, dtype=dtype)
    V = np.asarray(V, dtype=dtype)
    B, N, Hq, d = Q.shape
    Hkv, Nk = K.shape[2], K.shape[1]
    if K.shape != (B, Nk, Hkv, d) or V.shape != K.shape or Hq % Hkv != 0 or Nk < N:
        raise ValueError("shape mismatch")
    P = Nk - N                                               # keys before the chunk
    if mode == GATE_ABSOLUTE and table is None:
        raise ValueError("absolute gate needs a threshold table")
    if mode == GATE_ABSOLUTE and P % block_q != 0:
        raise ValueError("the absolute gate needs the prefix to be a multiple of block_q")
    if gate_dtype not in ("bf16", "fp8"):
        raise ValueError(f"unknown gate dtype {gate_dtype!r}")
    if gate_dtype == "fp8" and mode == GATE_RELATIVE:
        raise ValueError("FP8 gate scores are defined for the absolute gate")
    if mean_correction and mode == GATE_RELATIVE:
        # the relative gate decides from the running max, which a stand-in step would move
        raise ValueError("mean correction is defined for the dense and absolute gates only")
    G = Hq // Hkv
    sc = dtype(1.0 / math.sqrt(d) if scale is None else scale)
    nqb, nkb = num_blocks(N, block_q), num_blocks(Nk, block_k)
    blocks = range(nqb) if query_blocks is None else sorted(set(int(x) for x in query_blocks))

    if gate_dtype == "fp8":
        # the dequantised copies, (q8 sq) . (k8 sk) = sq sk (q8 . k8), in the oracle's
        # precision (exact in float64)
        q8, q8s = quantize_q_rows(Q)
        k8, k8s = quantize_k_tiles(K)
        Q8f = (q8.astype(np.float64) * q8s[..., None]).astype(dtype)
        K8f = (k8.astype(np.float64) * np.repeat(k8s, 64, axis=1)[:, :Nk, :, None]).astype(dtype)
    out = np.full((B, N, Hq, d), np.nan, dtype=dtype)
    kept_counts = np.full((B, Hq, nqb), -1, dtype=np.int64)
    stat = np.full((B, Hq, nqb, nkb), np.nan, dtype=np.float64)
    keep_mask = np.zeros((B, Hq, nqb, nkb), dtype=bool)
    margin = np.full((B, Hq, nqb, nkb), np.nan, dtype=np.float64)

    with np.errstate(invalid="ignore", over="ignore"):
        for b in range(B):
            for h in range(Hq):
                g = h // G                                   # GQA: query head -> its KV head
                for i in blocks:
                    r0, r1 = i * block_q, min((i + 1) * block_q, N)
                    q = Q[b, r0:r1, h, :]
                    R = r1 - r0
                    # online-softmax state (BLASST blog, "FlashAttention"): m, l, O on chip
                    m = np.full(R, -np.inf, dtype=dtype)
                    l = np.zeros(R, dtype=dtype)
                    o = np.zeros((R, d), dtype=dtype)
                    n_off, n_end = key_block_range(i, N, block_q, block_k, P)
                    # thresholds belong to the absolute query block
                    te = (effective_threshold(table, budget_slice, h, P // block_q + i)
                          if mode == GATE_ABSOLUTE else None)
                    kept = 0

                    def absorb(s, vals):
                        # one online-softmax step over the logits s [R, n] and values [n, d]
                        nonlocal m, l, o
                        m_new = np.maximum(m, s.max(axis=1))
                        alpha = np.exp(m - m_new)          # exp(-inf) = 0 on the first step
                        p = np.exp(s - m_new[:, None])
                        l = alpha * l + p.sum(axis=1)
                        o = alpha[:, None] * o + p @ vals
                        m = m_new

                    for j in range(n_end):                    # ascending; diagonal region last
                        c0, c1 = j * block_k, min((j + 1) * block_k, Nk)
                        # exact scaled pre-softmax scores of the whole tile (keep-rule equation)
                        s = (q @ K[b, c0:c1, g, :].T) * sc
                        if j >= n_off:
                            # causal diagonal region: mask future keys, always aggregated
                            rows = P + np.arange(r0, r1)[:, None]     # absolute positions
                            cols = np.arange(c0, c1)[None, :]
                            s = np.where(cols > rows, dtype(-np.inf), s)
                            stat[b, h, i, j] = float(s.max())
                            keep = True
                        else:
                            rmax = s.max(axis=1)
                            if mode == GATE_RELATIVE:
                                # each row tests itself against its running max; one row that
                                # wants the block vetoes the skip
                                st = float((rmax - m).max())
                                thr = float(log_lambda)
                            elif gate_dtype == "fp8" and mode == GATE_ABSOLUTE:
                                # the same tile maximum over FP8 scores
                                s8 = Q8f[b, r0:r1, h, :] @ K8f[b, c0:c1, g, :].T
                                st = float(s8.max()) * float(sc)
                                thr = te
                            else:
                                st = float(rmax.max())            # s_max over the whole tile
                                thr = te if mode == GATE_ABSOLUTE else -math.inf
                            stat[b, h, i, j] = st
                            mg = st - thr
                            margin[b, h, i, j] = mg
                            keep = st >= thr
                            if forced_keep is not None and abs(mg) <= band:
                                keep = bool(forced_keep[b, h, i, j])
                            kept += int(keep)
                        keep_mask[b, h, i, j] = keep
                        if keep:
                            absorb(s, V[b, c0:c1, g, :])
                        elif mean_correction:
                            # the block's stand-in: |B| copies of (mean key, mean value), i.e. one
                            # logit scale * q . kbar shifted by log|B|
                            kbar = K[b, c0:c1, g, :].mean(axis=0)
                            vbar = V[b, c0:c1, g, :].mean(axis=0)
                            sbar = (q @ kbar) * sc + dtype(math.log(c1 - c0))
                            absorb(sbar[:, None], vbar[None, :])
                        # else skipped: no V, no exp, m, l and O untouched
                    out[b, r0:r1, h, :] = o / l[:, None]     # renormalise over kept + diagonal
                    kept_counts[b, h, i] = kept
    return OracleResult(out, kept_counts, stat, keep_mask, margin)


def oracle_prefill_varlen(Q, K, V, cu_q, cu_k, *, block_q: int, block_k: int, mode: str,
                          **kw) -> OracleResult:
    """oracle_prefill for sequences packed along the token axis.

    Q: [total_q, Hq, d]; K, V: [total_k, Hkv, d]; sequence b owns query tokens
    cu_q[b] .. cu_q[b+1] and key tokens cu_k[b] .. cu_k[b+1] (its queries are the last of its
    key positions). Each sequence is computed on its own; the per-block results are padded to
    the longest sequence (NaN / -1 / False past a sequence's blocks). ``out`` is
    [total_q, Hq, d].
    """
    cu_q = [int(x) for x in cu_q]
    cu_k = [int(x) for x in cu_k]
    B = len(cu_q) - 1
    Q = np.asarray(Q)
    Hq, d = Q.shape[1], Q.shape[2]
    nq = [cu_q[b + 1] - cu_q[b] for b in range(B)]
    nk = [cu_k[b + 1] - cu_k[b] for b in range(B)]
    nqb = num_blocks(max(nq + [0]), block_q)
    nkb = num_blocks(max(nk + [0]), block_k)
    dtype = kw.get("dtype", np.float32)
    out = np.full((cu_q[-1], Hq, d), np.nan, dtype=dtype)
    kept_counts = np.full((B, Hq, nqb), -1, dtype=np.int64)
    stat = np.full((B, Hq, nqb, nkb), np.nan, dtype=np.float64)
    keep = np.zeros((B, Hq, nqb, nkb), dtype=bool)
    margin = np.full((B, Hq, nqb, nkb), np.nan, dtype=np.float64)
    forced = kw.pop("forced_keep", None)
    for b in range(B):
        if nq[b] == 0:
            continue
        r = oracle_prefill(Q[None, cu_q[b]:cu_q[b + 1]], np.asarray(K)[None, cu_k[b]:cu_k[b + 1]],
                           np.asarray(V)[None, cu_k[b]:cu_k[b + 1]], block_q=block_q,
                           block_k=block_k, mode=mode,
                           forced_keep=None if forced is None else forced[b:b + 1], **kw)
        qb, kb = r.kept_counts.shape[2], r.stat.shape[3]
        out[cu_q[b]:cu_q[b + 1]] = r.out[0]
        kept_counts[b, :, :qb] = r.kept_counts[0]
        stat[b, :, :qb, :kb] = r.stat[0]
        keep[b, :, :qb, :kb] = r.keep[0]
        margin[b, :, :qb, :kb] = r.margin[0]
    return OracleResult(out, kept_counts, stat, keep, margin)


def gather_pages(pages, block_table, kv_lens):
    """Keys (or values) of a paged cache laid out as packed sequences.

    pages: [num_pages, page_size, H, d]; block_table: [B, pages per sequence]; kv_lens: [B].
    Returns ([sum(kv_lens), H, d], cu [B + 1]): sequence b's token t lives at row
    t % page_size of page block_table[b, t // page_size].
    """
    pages = np.asarray(pages)
    page_size = pages.shape[1]
    rows, cu = [], [0]
    for b, n in enumerate(int(x) for x in kv_lens):
        t = np.arange(n)
        rows.append(pages[np.asarray(block_table)[b, t // page_size], t % page_size])
        cu.append(cu[-1] + n)
    if not rows:
        return np.zeros((0,) + pages.shape[2:], pages.dtype), np.asarray(cu)
    return np.concatenate(rows, axis=0), np.asarray(cu)


def off_diagonal_block_maxima(Q, K, *, block_q: int, block_k: int, scale: float | None = None,
                              dtype=np.float32, gate_dtype: str = "bf16") -> np.ndarray:
    """s_max[b, h, i, j] for every off-diagonal block j < n_off(i); NaN elsewhere.

    The maximum of the scaled pre-softmax scores over the whole Bq x Bk tile
    ("Block Sparse Flash Attention", Method > Key Designs 2, keep-rule equation). The scores of
    one (b, h, i) against all its off-diagonal keys come from one matrix product, then each
    Bk-wide column group is reduced. gate_dtype "fp8": the scores of the FP8 gate (E4M3 copies
    of Q and K and their scales, as in oracle_prefill).
    """
    fp8 = gate_dtype == "fp8"
    if fp8:
        # the dequantised copies, (q8 sq) . (k8 sk) = sq sk (q8 . k8), in the oracle's
        # precision (exact in float64)
        q8, q8s = quantize_q_rows(Q)
        k8, k8s = quantize_k_tiles(K)
        Qf = (q8.astype(np.float64) * q8s[..., None]).astype(dtype)
        Kf = (k8.astype(np.float64) * np.repeat(k8s, 64, axis=1)[:, :k8.shape[1], :, None]
              ).astype(dtype)
    Q = np.asarray(Q, dtype=dtype)
    K = np.asarray(K, dtype=dtype)
    B, N, Hq, d = Q.shape
    Hkv = K.shape[2]
    G = Hq // Hkv
    sc = dtype(1.0 / math.sqrt(d) if scale is None else scale)
    nqb, nkb = num_blocks(N, block_q), num_blocks(N, block_k)
    sm = np.full((B, Hq, nqb, nkb), np.nan, dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(nqb):
                n_off, _ = key_block_range(i, N, block_q, block_k)
                if n_off == 0:
                    continue
                r0, r1 = i * block_q, min((i + 1) * block_q, N)
                c1 = n_off * block_k
                if fp8:
                    s = (Qf[b, r0:r1, h, :] @ Kf[b, :c1, g, :].T) * sc
                else:
                    s = (Q[b, r0:r1, h, :] @ K[b, :c1, g, :].T) * sc
                sm[b, h, i, :n_off] = s.reshape(r1 - r0, n_off, block_k).max(axis=(0, 2))
    return sm


def kth_highest(maxima: np.ndarray, n_off: int, k: int) -> float:
    """k-th highest of the first n_off block maxima (1-indexed), or -inf if n_off < k.

    ("Block Sparse Flash Attention", Method > Key Designs 1: sort the maxima and take the k-th
    highest; a -inf threshold where the position has too few off-diagonal candidates.)
    """
    if n_off < k:
        return -math.inf
    return float(np.sort(maxima[:n_off])[::-1][k - 1])


def calibrate(samples, *, block_q: int, block_k: int, budgets, scale: float | None = None,
              dtype=np.float32, gate_dtype: str = "bf16") -> np.ndarray:
    """Offline threshold calibration: T[n_budgets][Hq][T_len] (float32).

    samples: iterable of (Q, K) pairs of equal shape [B, N, Hq, d] / [B, N, Hkv, d]; every
    batch entry counts as one calibration sample. For each sample, head and query block the
    k-th highest off-diagonal block maximum is taken; thresholds are the arithmetic mean over
    samples ("Block Sparse Flash Attention", Method > Key Designs 1). T_len = number of query
    blocks of the calibration length. gate_dtype "fp8" calibrates against the FP8 gate's
    block maxima (thresholds are bound to the scores they were measured on).
    """
    budgets = [int(k) for k in budgets]
    acc = None
    count = 0
    shape0 = None
    for Q, K in samples:
        Q = np.asarray(Q)
        if shape0 is None:
            shape0 = Q.shape
        elif Q.shape[1:] != shape0[1:]:
            raise ValueError("calibration samples must share one shape")
        sm = off_diagonal_block_maxima(Q, K, block_q=block_q, block_k=block_k, scale=scale,
                                       dtype=dtype, gate_dtype=gate_dtype)
        B, Hq, nqb, _ = sm.shape
        N = Q.shape[1]
        if acc is None:
            acc = np.zeros((len(budgets), Hq, nqb), dtype=np.float64)
        for b in range(B):
            for h in range(Hq):
                for i in range(nqb):
                    n_off, _ = key_block_range(i, N, block_q, block_k)
                    for kk, k in enumerate(budgets):
                        acc[kk, h, i] += kth_highest(sm[b, h, i], n_off, k)
            count += 1
    if count == 0:
        raise ValueError("no calibration samples")
    return (acc / count).astype(np.float32)
