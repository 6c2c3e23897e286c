"""The pages' tiled forward with an online softmax, in fp64 (test infrastructure).

Follows [P2 "Tiling: Breaking the Problem into Pieces"], [P2 "The Trick: Online Softmax"] and the
conceptual FlashAttention loop of [P2 "A Worked Example in Pseudocode"]: for each block of query
rows, walk the key/value blocks keeping, per row, the largest score seen so far and the sum of
exponentials relative to it; when the maximum grows, the partial output and the partial sum are
multiplied by exp(old max - new max); the output block is divided by the sum once at the end.

Additions the pages leave open (readings, see the package docs):
  * the scale factor multiplies Q K^T;
  * causal and 128x128 block visibility set invisible scores to -inf;
  * a row that has seen no visible key keeps max = -inf; its rescale factor is taken as 1 and its
    exponentials as 0, and a row that never sees one ends with O = 0, LSE = -inf;
  * the natural-log row statistic LSE = max + ln(sum) is returned too.

It exists so that the tests can check that this re-association reaches the materialised
definition in attention.py, which is the exactness the pages claim.
"""
from __future__ import annotations

import numpy as np

MASK_BLOCK = 128


def _tile_visibility(rows, cols, causal, block_mask):
    ok = np.ones((rows.size, cols.size), dtype=bool)
    if causal:
        ok &= rows[:, None] >= cols[None, :]
    if block_mask is not None:
        ok &= np.asarray(block_mask)[rows // MASK_BLOCK][:, cols // MASK_BLOCK] != 0
    return ok


def tiled_forward_head(q, k, v, scale, causal=False, block_mask=None, block_q=128, block_k=128):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, d = q.shape
    Nk = k.shape[0]
    O = np.zeros((N, v.shape[1]))
    lse = np.zeros(N)
    n_qblocks = -(-N // block_q)
    n_kblocks = -(-Nk // block_k)
    for i in range(n_qblocks):
        rows = np.arange(i * block_q, min(N, (i + 1) * block_q))
        acc = np.zeros((rows.size, v.shape[1]))
        run_max = np.full(rows.size, -np.inf)
        run_sum = np.zeros(rows.size)
        for j in range(n_kblocks):
            cols = np.arange(j * block_k, min(Nk, (j + 1) * block_k))
            s = scale * (q[rows] @ k[cols].T)
            s = np.where(_tile_visibility(rows, cols, causal, block_mask), s, -np.inf)
            new_max = np.maximum(run_max, s.max(axis=1))
            seen = np.isfinite(new_max)
            had = np.isfinite(run_max)
            # factor that moves the old partial results onto the new maximum; a row that had seen
            # nothing holds zeros, and a row that still sees nothing keeps them
            factor = np.ones(rows.size)
            factor[seen & had] = np.exp(run_max[seen & had] - new_max[seen & had])
            factor[seen & ~had] = 0.0
            acc *= factor[:, None]
            run_sum *= factor
            p = np.exp(s - np.where(seen, new_max, 0.0)[:, None])
            p = np.where(seen[:, None], p, 0.0)
            run_sum += p.sum(axis=1)
            acc += p @ v[cols]
            run_max = new_max
        alive = run_sum > 0
        O[rows] = acc / np.where(alive, run_sum, 1.0)[:, None]
        with np.errstate(divide="ignore"):
            lse[rows] = np.where(alive, run_max + np.log(np.where(alive, run_sum, 1.0)), -np.inf)
    return O, lse
