"""Exact attention by its plain definition, in fp64 (test infrastructure; see package header).

Per (batch, head), with Q, K, V as N x d matrices:
  S = scale * Q K^T                       [P2 "The Quadratic Memory Bottleneck"; the scale is the
                                            usual 1/sqrt(d)-style factor, passed as an argument]
  S_ij = -inf where key j is not visible  (causal: j <= i; block mask at 128x128 granularity,
                                            [P3 "Innovation #5: Extension to block-sparse attention patterns"])
  P = row softmax of S                    [P2 "The Trick: Online Softmax", the softmax formula]
  O = P V                                 [P2 "A Worked Example in Pseudocode", Standard Attention]
  LSE_i = ln sum_j exp(S_ij)              (the row statistic kept for the backward pass,
                                            [P3 "Innovation #3: Strategic recomputation in the backward pass"])

Backward, for an upstream gradient dO of L = sum(O * dO), by differentiating the above
(the pages give no formulas; this is calculus of the definition):
  dV = P^T dO;  dP = dO V^T;  D_i = sum_j P_ij dP_ij;  dS = P * (dP - D);  dQ = scale dS K;
  dK = scale dS^T Q.
D is computed from P and dP here, not from O, so it is independent of any rowsum(dO*O) shortcut.

A row with no visible key has no defined softmax; its reading here is O_i = 0, LSE_i = -inf and
zero gradient contribution.

S and P are materialised in row chunks (every row in full width) so that long sequences fit in
host memory; nothing else is blocked, fused or reordered.
"""
from __future__ import annotations

import numpy as np

MASK_BLOCK = 128


def visible(rows: np.ndarray, cols: np.ndarray, causal: bool, block_mask: np.ndarray | None) -> np.ndarray:
    """bool [len(rows), len(cols)]: may query `rows[a]` attend key `cols[b]`?"""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    vis = np.ones((rows.size, cols.size), dtype=bool)
    if causal:
        vis &= cols[None, :] <= rows[:, None]
    if block_mask is not None:
        bm = np.asarray(block_mask) != 0
        vis &= bm[np.ix_(rows // MASK_BLOCK, cols // MASK_BLOCK)]
    return vis


def _scores(q, k, rows, scale, causal, block_mask):
    S = scale * (q[rows] @ k.T)
    vis = visible(rows, np.arange(k.shape[0]), causal, block_mask)
    return np.where(vis, S, -np.inf)


def _softmax_rows(S):
    """Row softmax of S (entries -inf are invisible).  Returns (P, lse, dead) where dead marks
    rows with no visible entry (P row = 0, lse = -inf)."""
    m = S.max(axis=1)
    dead = ~np.isfinite(m)
    m_safe = np.where(dead, 0.0, m)
    E = np.exp(S - m_safe[:, None])
    den = E.sum(axis=1)
    P = E / np.where(dead, 1.0, den)[:, None]
    with np.errstate(divide="ignore"):
        lse = np.where(dead, -np.inf, m_safe + np.log(np.where(dead, 1.0, den)))
    return P, lse, dead


def probabilities(q, k, scale, causal=False, block_mask=None, rows=None):
    """P (rows x N) for one head; exposed for the invariant tests."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    P, _, _ = _softmax_rows(_scores(q, k, rows, scale, causal, block_mask))
    return P


def forward_head(q, k, v, scale, causal=False, block_mask=None, rows=None, chunk=1024):
    """O [len(rows), d] and LSE [len(rows)] for one head (all rows if `rows` is None)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    O = np.zeros((rows.size, v.shape[1]))
    lse = np.zeros(rows.size)
    for a in range(0, rows.size, chunk):
        r = rows[a:a + chunk]
        P, l, _ = _softmax_rows(_scores(q, k, r, scale, causal, block_mask))
        O[a:a + r.size] = P @ v
        lse[a:a + r.size] = l
    return O, lse


def p_rounding_bound(q, k, v, scale, causal=False, block_mask=None, rows=None, rel=2.0 ** -4, floor=2.0 ** -10,
                     chunk=1024):
    """Elementwise bound [len(rows), d] on |sum_j p'_j v_j / sum_j p_j - O| when every visible
    weight p_j = exp(S_ij - max_j S_ij) (so max_j p_j = 1) is replaced in the numerator only by
    some p'_j with |p'_j - p_j| <= max(rel p_j, floor):  sum_j max(rel p_j, floor) |v_j| / sum_j p_j
    over the visible keys (triangle inequality, attained by the worst-signed perturbation).

    With rel = 2^-4 and floor = 2^-10 it bounds the rounding of P to E4M3 before the P V product
    in the MX-FP8 forward: E4M3 keeps 3 fraction bits (half an ulp is at most 2^-4 of a normal
    value) and its subnormal step is 2^-9 (rounding error at most 2^-10), for weights held as
    c p_j with c >= 1 (the kernel's running-max offset never exceeds the row max), which only
    shrinks the floor in units of p.  Dead rows get 0."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    out = np.zeros((rows.size, v.shape[1]))
    absv = np.abs(v)
    for a in range(0, rows.size, chunk):
        r = rows[a:a + chunk]
        S = _scores(q, k, r, scale, causal, block_mask)
        vis = np.isfinite(S)
        m = np.where(vis.any(axis=1), S.max(axis=1), 0.0)
        p = np.where(vis, np.exp(S - m[:, None]), 0.0)
        err = np.where(vis, np.maximum(rel * p, floor), 0.0)
        den = p.sum(axis=1)
        out[a:a + r.size] = (err @ absv) / np.where(den > 0, den, 1.0)[:, None]
    return out


def forward(q, k, v, scale, causal=False, block_mask=None, chunk=1024):
    """[B, H, N, d] inputs -> O [B, H, N, d], LSE [B, H, N] (fp64)."""
    B, H, N, d = q.shape
    O = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            O[b, h], lse[b, h] = forward_head(q[b, h], k[b, h], v[b, h], scale, causal, block_mask, chunk=chunk)
    return O, lse


def backward_head(q, k, v, do, scale, causal=False, block_mask=None, dq_rows=None, dkv_cols=None, chunk=1024):
    """Gradients of L = sum(O * dO) for one head.

    dq_rows:  query rows whose dQ is returned (None = all).
    dkv_cols: key rows whose dK, dV are returned (None = all; an empty list skips dK/dV).
    Returns (dQ [len(dq_rows), d], dK [len(dkv_cols), d], dV [len(dkv_cols), d]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    N, d = q.shape
    dq_rows = np.arange(N) if dq_rows is None else np.asarray(dq_rows, dtype=np.int64)
    dkv_cols = np.arange(N) if dkv_cols is None else np.asarray(dkv_cols, dtype=np.int64)
    dQ = np.zeros((dq_rows.size, d))
    dK = np.zeros((dkv_cols.size, d))
    dV = np.zeros((dkv_cols.size, d))
    want_row = np.zeros(N, dtype=bool)
    want_row[dq_rows] = True
    row_pos = np.full(N, -1, dtype=np.int64)
    row_pos[dq_rows] = np.arange(dq_rows.size)
    # dK and dV sum over every query row; dQ of a row needs only that row's P, dP and D, so
    # without dK/dV columns only the requested rows are visited
    visit = np.arange(N) if dkv_cols.size else np.unique(dq_rows)
    for a in range(0, visit.size, chunk):
        r = visit[a:a + chunk]
        P, _, _ = _softmax_rows(_scores(q, k, r, scale, causal, block_mask))
        dP = do[r] @ v.T
        D = (P * dP).sum(axis=1)
        dS = P * (dP - D[:, None])
        if dkv_cols.size:
            dV += P[:, dkv_cols].T @ do[r]
            dK += scale * (dS[:, dkv_cols].T @ q[r])
        sel = want_row[r]
        if sel.any():
            dQ[row_pos[r[sel]]] = scale * (dS[sel] @ k)
    return dQ, dK, dV


def backward(q, k, v, do, scale, causal=False, block_mask=None, chunk=1024):
    """[B, H, N, d] inputs -> dQ, dK, dV [B, H, N, d] (fp64)."""
    dQ = np.zeros(q.shape)
    dK = np.zeros(q.shape)
    dV = np.zeros(q.shape)
    B, H = q.shape[:2]
    for b in range(B):
        for h in range(H):
            dQ[b, h], dK[b, h], dV[b, h] = backward_head(q[b, h], k[b, h], v[b, h], do[b, h], scale, causal,
                                                         block_mask, chunk=chunk)
    return dQ, dK, dV


def s_matrix_bytes(N: int, elem_bytes: int = 4) -> int:
    """Bytes of one materialised N x N score matrix, the quadratic term that standard attention
    writes to HBM [P2 "The Quadratic Memory Bottleneck"]."""
    return N * N * elem_bytes
