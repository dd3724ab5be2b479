"""Indexer scoring, top-K selection, hierarchical pool and index reuse (oracle).

Sources:
  [P1] section "CSA2": every CSA2 layer runs in one of three static modes.
       Full computes its own main KV and indexer K and selects its own top-K
       indices; Reindex reuses an earlier layer's main KV and indexer K but
       re-scores them with its own query to select new indices; Reuse takes
       an earlier layer's indices and runs no indexer at all.
  [P1] section "Hierarchical Sparse Indexer": in the decoder the first Full
       layer scores every causally visible position, picks its own top-K and,
       in the same pass, gives each block of positions the maximum index score
       inside it; the best blocks (at most 2048 blocks of 8 positions, so at
       most 16,384 positions) form a candidate pool, and the later Reindex
       layers score and select only inside that pool.

Readings taken where the pages are silent (listed in the design notes):
  * Score (64-dim fp32 / bf16 keys): a single-query dot product
    score[t] = q_idx . k_idx[t], evaluated in float64 from the stored key
    values and an fp32 query.
  * Score at the pages' indexer shape ([P1] section "CSA2": 32 indexer query
    heads of dimension 128; FP4 storage as in section "FP4 KV cache"): keys
    stored in the same FP4 format as the latent (E2M1 + one E4M3 scale per 16
    dims, 72 B per 128-dim key), queries given per head in fp16 with one fp32
    weight per head, and heads combined as
        score[t] = sum_h w[h] * max(0, q[h] . k[t]),
    the weighted-ReLU rule of DeepSeek's earlier lightning indexer; the pages
    give the head count and dimension but no combining rule.  Evaluated in
    float64 from the exact dequantized keys and the fp16 query values.
  * Top-K: the K largest scores; equal scores go to the lower position; when
    fewer than K positions are visible the result is padded with -1.  The
    selection is a set (order is not part of the result).
  * Blocks: aligned runs of 8 positions [8j, 8j+8), the last one possibly
    partial; block score = max over its visible positions; the top
    P = min(pool_blocks, number of blocks) blocks by (score desc, block asc).
  * The Full layer's own top-K is taken over all visible positions.
"""

import numpy as np

from .ced import bf16_bits_to_f64


def keys_to_f64(keys, dtype):
    """Stored indexer keys -> float64.  dtype 'f32' (float32 array) or 'bf16' (uint16 bits)."""
    if dtype == "f32":
        return np.asarray(keys, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(keys)
    raise ValueError(dtype)


def fp4_keys_to_f64(codes, scales):
    """FP4 indexer keys (codes [n][D/2], scales [n][D/16], the latent's format) -> float64 [n][D]."""
    from .fp4 import fp4_unpack

    return fp4_unpack(codes, scales)


def index_scores(q_idx, keys_f64, w=None):
    """Index scores in float64; keys: [n][D].

    w is None: score[t] = sum_d q_idx[d] * k[t, d], q_idx fp32 [D].
    w given:   score[t] = sum_h w[h] * max(0, sum_d q_idx[h, d] * k[t, d]),
               q_idx fp16 [H][D] (the query heads), w fp32 [H].
    """
    if w is None:
        q = np.asarray(q_idx, dtype=np.float32).astype(np.float64)
        return keys_f64 @ q
    q = np.asarray(q_idx, dtype=np.float16).astype(np.float64)
    ww = np.asarray(w, dtype=np.float32).astype(np.float64)
    return np.maximum(keys_f64 @ q.T, 0.0) @ ww


def topk(scores, k, positions=None):
    """Indices of the k best scores: sort by (-score, position) and take the head.

    scores: float64 [n]; positions: the position of each score (default 0..n-1).
    returns int64 [k], padded with -1 when n < k.
    """
    scores = np.asarray(scores, dtype=np.float64)
    n = scores.shape[0]
    pos = np.arange(n, dtype=np.int64) if positions is None else np.asarray(positions, dtype=np.int64)
    order = np.lexsort((pos, -scores))  # primary key -score, secondary key position
    take = pos[order[: min(k, n)]]
    out = np.full(k, -1, dtype=np.int64)
    out[: take.shape[0]] = take
    return out


def block_scores(scores, block_tokens=8):
    """bscore[j] = max of scores over positions [8j, min(8j+8, n))."""
    scores = np.asarray(scores, dtype=np.float64)
    n = scores.shape[0]
    nb = -(-n // block_tokens)
    out = np.empty(nb, dtype=np.float64)
    for j in range(nb):
        out[j] = scores[j * block_tokens : min((j + 1) * block_tokens, n)].max()
    return out


def block_scores_fast(scores, block_tokens=8):
    """Same result as block_scores, vectorised (padding with -inf)."""
    scores = np.asarray(scores, dtype=np.float64)
    n = scores.shape[0]
    nb = -(-n // block_tokens)
    pad = np.full(nb * block_tokens, -np.inf)
    pad[:n] = scores
    return pad.reshape(nb, block_tokens).max(axis=1)


def pool_blocks(scores, pool_blocks_max=2048, block_tokens=8):
    """Block ids of the candidate pool: top min(P, #blocks) blocks by (-bscore, j).

    returns int64 [pool_blocks_max], padded with -1.
    """
    b = block_scores_fast(scores, block_tokens)
    return topk(b, pool_blocks_max)


def pool_positions(block_ids, n, block_tokens=8):
    """Sorted positions covered by the pool blocks (valid ids only), clipped to n."""
    ids = np.asarray(block_ids, dtype=np.int64)
    ids = ids[ids >= 0]
    pos = (ids[:, None] * block_tokens + np.arange(block_tokens)[None, :]).reshape(-1)
    return np.sort(pos[pos < n])


def full_select(q_idx, keys_f64, k, pool_blocks_max=None, block_tokens=8, w=None):
    """Full mode: scores over all visible positions -> (indices, pool block ids or None)."""
    s = index_scores(q_idx, keys_f64, w)
    idx = topk(s, k)
    pool = pool_blocks(s, pool_blocks_max, block_tokens) if pool_blocks_max else None
    return idx, pool


def reindex_select(q_idx, keys_f64, k, pool_block_ids, block_tokens=8, w=None):
    """Reindex mode: this layer's own query scores only the pool positions."""
    n = keys_f64.shape[0]
    pos = pool_positions(pool_block_ids, n, block_tokens)
    s = index_scores(q_idx, keys_f64[pos], w)
    return topk(s, k, positions=pos)


def reuse_select(indices):
    """Reuse mode: the earlier layer's indices, unchanged (no indexer work)."""
    return np.array(indices, copy=True)
