"""Independent references used to pin the oracle (library routines and brute force, float64).

None of these re-types the oracle's streaming algorithm: attention comes from torch's
scaled_dot_product_attention on the CPU with an explicit boolean mask, block maxima from one
full float64 score matrix.
"""
import math

import numpy as np
import torch


def sdpa_masked(Q, K, V, mask, scale=None):
    """Softmax attention in float64 with an explicit mask.

    Q: [B, N, Hq, d]; K, V: [B, N, Hkv, d]; mask: bool [B, Hq, N, N] (True = attend).
    """
    Q = torch.as_tensor(np.asarray(Q, dtype=np.float64))
    K = torch.as_tensor(np.asarray(K, dtype=np.float64))
    V = torch.as_tensor(np.asarray(V, dtype=np.float64))
    G = Q.shape[2] // K.shape[2]
    K = K.repeat_interleave(G, dim=2)
    V = V.repeat_interleave(G, dim=2)
    d = Q.shape[-1]
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    o = torch.nn.functional.scaled_dot_product_attention(
        Q.transpose(1, 2), K.transpose(1, 2), V.transpose(1, 2),
        attn_mask=torch.as_tensor(mask), scale=sc)
    return o.transpose(1, 2).numpy()


def causal_mask(B, Hq, N):
    m = np.tril(np.ones((N, N), dtype=bool))
    return np.broadcast_to(m, (B, Hq, N, N)).copy()


def full_scores(Q, K, scale=None):
    """float64 S[b, h, r, c] = (Q K^T) * scale for every pair (no mask)."""
    Q = torch.as_tensor(np.asarray(Q, dtype=np.float64))
    K = torch.as_tensor(np.asarray(K, dtype=np.float64))
    G = Q.shape[2] // K.shape[2]
    K = K.repeat_interleave(G, dim=2)
    d = Q.shape[-1]
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    return (torch.einsum("bnhd,bmhd->bhnm", Q, K) * sc).numpy()


def first_offdiag_blocks(N, Bq, Bk):
    """n_off(i) by brute force: key blocks whose last key precedes the query block's first row."""
    nqb = -(-N // Bq)
    nkb = -(-N // Bk)
    out = []
    for i in range(nqb):
        first_row = i * Bq
        out.append(sum(1 for j in range(nkb) if min((j + 1) * Bk, N) - 1 < first_row))
    return out


def brute_block_max(Q, K, Bq, Bk, scale=None):
    """s_max[b, h, i, j] over every pair of the tile for off-diagonal blocks; NaN elsewhere."""
    S = full_scores(Q, K, scale)
    B, Hq, N, _ = S.shape
    nqb, nkb = -(-N // Bq), -(-N // Bk)
    noff = first_offdiag_blocks(N, Bq, Bk)
    out = np.full((B, Hq, nqb, nkb), np.nan)
    for i in range(nqb):
        for j in range(noff[i]):
            out[:, :, i, j] = S[:, :, i * Bq:min((i + 1) * Bq, N), j * Bk:(j + 1) * Bk].max(axis=(2, 3))
    return out


def block_mask_to_token_mask(keep, N, Bq, Bk):
    """Expand a per-(b, h, i, j) keep decision to a causal token mask [B, Hq, N, N]."""
    B, Hq, nqb, nkb = keep.shape
    m = np.zeros((B, Hq, N, N), dtype=bool)
    for i in range(nqb):
        for j in range(nkb):
            sel = keep[:, :, i, j]
            m[:, :, i * Bq:min((i + 1) * Bq, N), j * Bk:min((j + 1) * Bk, N)] = sel[:, :, None, None]
    return m & np.tril(np.ones((N, N), dtype=bool))


def diagonal_region_mask(B, Hq, N, Bq, Bk):
    """Token mask of the causal diagonal region only: keys not wholly before the query block."""
    noff = first_offdiag_blocks(N, Bq, Bk)
    m = np.zeros((B, Hq, N, N), dtype=bool)
    for i, no in enumerate(noff):
        m[:, :, i * Bq:min((i + 1) * Bq, N), no * Bk:] = True
    return m & np.tril(np.ones((N, N), dtype=bool))


def quantized_normal(rng, shape, step=1 / 64, lim=2.0):
    """Gaussian values rounded to a coarse grid, so products and short sums are exact."""
    x = np.clip(rng.standard_normal(shape), -lim, lim)
    return (np.round(x / step) * step).astype(np.float32)
