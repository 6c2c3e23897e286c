"""Checks that pin the fp64 oracle to facts outside itself.

Each `check_*` takes the oracle's callables and raises AssertionError when a fact fails, so the
same checks run against the real oracle (test_oracle.py) and against copies with planted
mistakes (test_oracle_mutations.py).  The facts come from the definition of softmax attention
[P2 "The Quadratic Memory Bottleneck", "The Trick: Online Softmax"], from calculus (central
finite differences), and from brute force in plain Python scalars.

Page keys: [P2] "FlashAttention: how a memory trick unlocked today's giant AI models" (khetwal.com);
[P3] "How FlashAttention Eliminates Transformer Memory Bottlenecks" (Galileo blog).
"""
from __future__ import annotations

import math

import numpy as np

BLOCK = 128


# ----------------------------------------------------------------------------- brute force
def brute_force_head(q, k, v, scale, causal=False, block_mask=None, rows=None):
    """Plain-Python scalar attention for small inputs: math.exp, math.fsum, explicit loops."""
    N, d = len(q), len(q[0])
    dv = len(v[0])
    rows = range(N) if rows is None else rows
    O, L = [], []
    for i in rows:
        s = []
        for j in range(len(k)):
            ok = (not causal or j <= i) and (block_mask is None or block_mask[i // BLOCK][j // BLOCK] != 0)
            s.append(scale * math.fsum(float(q[i][c]) * float(k[j][c]) for c in range(d)) if ok else None)
        vis = [x for x in s if x is not None]
        if not vis:
            O.append([0.0] * dv)
            L.append(-math.inf)
            continue
        m = max(vis)
        e = [math.exp(x - m) if x is not None else 0.0 for x in s]
        den = math.fsum(e)
        O.append([math.fsum(e[j] * float(v[j][c]) for j in range(len(k))) / den for c in range(dv)])
        L.append(m + math.log(den))
    return np.array(O), np.array(L)


def check_brute_force(forward_head, seed=0):
    rng = np.random.default_rng(seed)
    for N in (1, 2, 3, 5, 8):
        for d in (1, 3, 4):
            q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
            for causal in (False, True):
                for scale in (0.7, -0.7):  # a negative scale reverses which keys dominate
                    O, L = forward_head(q, k, v, scale, causal)
                    Ob, Lb = brute_force_head(q.tolist(), k.tolist(), v.tolist(), scale, causal)
                    assert np.abs(O - Ob).max() <= 1e-13, ("brute force O", N, d, causal, scale)
                    assert np.abs(L - Lb).max() <= 1e-13, ("brute force LSE", N, d, causal, scale)


def check_brute_force_masked(forward_head, seed=1):
    """Block mask semantics at 128x128 granularity, with an asymmetric mask, against brute force
    over a sample of rows spanning every block row (rows of mask block 1 see only block 2 and
    block 0 sees itself; block 2 row sees blocks 0 and 1)."""
    rng = np.random.default_rng(seed)
    N, d = 300, 2
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    mask = np.array([[1, 0, 0], [0, 0, 1], [1, 1, 0]], dtype=np.uint8)
    rows = [0, 5, 127, 128, 129, 200, 255, 256, 257, 299]
    for causal in (False, True):
        O, L = forward_head(q, k, v, 0.9, causal, mask, rows=np.array(rows))
        Ob, Lb = brute_force_head(q.tolist(), k.tolist(), v.tolist(), 0.9, causal, mask.tolist(), rows)
        fin = np.isfinite(Lb)
        assert np.array_equal(np.isfinite(L), fin), ("masked dead rows", causal)
        assert np.abs(O - Ob).max() <= 1e-13, ("masked brute force O", causal)
        assert np.abs(L[fin] - Lb[fin]).max() <= 1e-13, ("masked brute force LSE", causal)


# ----------------------------------------------------------------------------- invariants
def check_probabilities_sum_to_one(probabilities, seed=2):
    rng = np.random.default_rng(seed)
    N, d = 260, 8
    q, k = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    mask = np.array([[1, 0, 1], [1, 1, 0], [0, 1, 1]], dtype=np.uint8)
    for causal, bm in ((False, None), (True, None), (False, mask), (True, mask)):
        P = probabilities(q, k, 0.3, causal, bm)
        assert np.all(P >= 0)
        assert np.abs(P.sum(axis=1) - 1.0).max() <= 1e-12, ("rows of P sum to 1", causal, bm is not None)


def check_identical_keys(forward_head, seed=3):
    """All keys equal => every visible score in a row is equal => O_i is the mean of the
    visible V_j, and LSE_i = scale q_i.k + ln(#visible)."""
    rng = np.random.default_rng(seed)
    N, d = 50, 6
    q, v = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    kk = rng.standard_normal(d)
    k = np.tile(kk, (N, 1))
    for causal in (False, True):
        O, L = forward_head(q, k, v, 0.5, causal)
        for i in range(N):
            n = i + 1 if causal else N
            assert np.abs(O[i] - v[:n].mean(axis=0)).max() <= 1e-12, ("identical keys O", causal, i)
            assert abs(L[i] - (0.5 * q[i] @ kk + math.log(n))) <= 1e-12, ("identical keys LSE", causal, i)


def check_one_hot_dominant(forward_head, seed=4):
    """Q_i = c K_{j*} with a score gap of >= 40 nats returns V_{j*} (to e^-40 N max|V|)."""
    rng = np.random.default_rng(seed)
    N, d = 64, 16
    k = rng.standard_normal((N, d))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((N, d))
    q = rng.standard_normal((N, d))
    target = rng.permutation(N)
    scale = 0.25
    for i in range(N):
        j = target[i]
        s = k @ k[j]  # scores of c*k_j against all keys, before c
        gap = s[j] - np.max(np.delete(s, j))
        c = 40.0 / (scale * gap) + 1.0
        q[i] = c * k[j]
    O, _ = forward_head(q, k, v, scale, False)
    tol = math.exp(-40) * N * np.abs(v).max() + 1e-13
    assert np.abs(O - v[target]).max() <= tol, "one-hot dominant row"


def check_causal_row0_and_small_n(forward_head, seed=5):
    rng = np.random.default_rng(seed)
    N, d = 40, 5
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    O, L = forward_head(q, k, v, 0.8, True)
    assert np.array_equal(O[0], v[0]), "causal row 0 returns V[0] exactly"
    assert abs(L[0] - 0.8 * (q[0] @ k[0])) <= 1e-13, "causal row 0 LSE"
    # N = 1: O = V, LSE = scale q.k
    O1, L1 = forward_head(q[:1], k[:1], v[:1], 0.8, False)
    assert np.abs(O1 - v[:1]).max() <= 1e-15 and abs(L1[0] - 0.8 * q[0] @ k[0]) <= 1e-13, "N=1"
    # N = 2: P_i0 = sigmoid(S_i0 - S_i1)
    O2, L2 = forward_head(q[:2], k[:2], v[:2], 0.8, False)
    for i in range(2):
        s0, s1 = 0.8 * q[i] @ k[0], 0.8 * q[i] @ k[1]
        p0 = 1.0 / (1.0 + math.exp(-(s0 - s1)))
        assert np.abs(O2[i] - (p0 * v[0] + (1 - p0) * v[1])).max() <= 1e-13, "N=2 sigmoid"
        assert abs(L2[i] - (max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))))) <= 1e-13, "N=2 LSE"


def check_causal_is_prefix_attention(forward_head, seed=6):
    rng = np.random.default_rng(seed)
    N, d = 30, 4
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    O, L = forward_head(q, k, v, 0.6, True)
    for i in (1, 7, 29):
        Ob, Lb = brute_force_head(q[i:i + 1].tolist(), k[:i + 1].tolist(), v[:i + 1].tolist(), 0.6)
        assert np.abs(O[i] - Ob[0]).max() <= 1e-13 and abs(L[i] - Lb[0]) <= 1e-13, ("causal prefix", i)


def check_permutation_and_shift(forward_head, seed=7):
    rng = np.random.default_rng(seed)
    N, d = 70, 8
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    O, L = forward_head(q, k, v, 0.4, False)
    perm = rng.permutation(N)
    Op, Lp = forward_head(q, k[perm], v[perm], 0.4, False)
    assert np.abs(O - Op).max() <= 1e-13 and np.abs(L - Lp).max() <= 1e-12, "key permutation"
    u = rng.standard_normal(d)
    Os, Ls = forward_head(q, k + u, v, 0.4, False)
    assert np.abs(O - Os).max() <= 1e-12, "key shift leaves O"
    assert np.abs(Ls - (L + 0.4 * q @ u)).max() <= 1e-12, "key shift moves LSE by scale q.u"


def check_mask_equivalences(forward_head, seed=8):
    rng = np.random.default_rng(seed)
    N, d = 300, 4
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    ones = np.ones((3, 3), dtype=np.uint8)
    O, L = forward_head(q, k, v, 0.5, False)
    O1, L1 = forward_head(q, k, v, 0.5, False, ones)
    assert np.abs(O - O1).max() == 0 and np.abs(L - L1).max() == 0, "all-ones mask equals dense"
    mask = np.array([[1, 0, 1], [0, 1, 1], [1, 1, 0]], dtype=np.uint8)
    Om, Lm = forward_head(q, k, v, 0.5, False, mask)
    for i in (3, 140, 290):
        cols = np.array([j for j in range(N) if mask[i // BLOCK][j // BLOCK]])
        Og, Lg = forward_head(q[i:i + 1], k[cols], v[cols], 0.5, False)
        assert np.abs(Om[i] - Og[0]).max() <= 1e-13 and abs(Lm[i] - Lg[0]) <= 1e-13, ("gathered keys", i)
    # a row with no visible key: O = 0, LSE = -inf
    dead = np.array([[1, 0, 0], [0, 0, 0], [1, 1, 1]], dtype=np.uint8)
    Od, Ld = forward_head(q, k, v, 0.5, False, dead)
    assert np.all(Od[128:256] == 0) and np.all(np.isneginf(Ld[128:256])), "fully masked rows"
    assert np.all(np.isfinite(Ld[:128])) and np.all(np.isfinite(Ld[256:])), "live rows finite"


def check_tiled_twin(forward_head, tiled_forward_head, seed=9):
    """The online-softmax tiled loop reaches the materialised definition (exactness)."""
    rng = np.random.default_rng(seed)
    N, d = 290, 8
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    mask = np.array([[1, 0, 1], [1, 1, 0], [0, 1, 1]], dtype=np.uint8)
    for causal, bm in ((False, None), (True, None), (False, mask), (True, mask)):
        O, L = forward_head(q, k, v, 0.35, causal, bm)
        for bq, bk in ((1, 1), (3, 16), (16, 3), (128, 128), (64, 128)):
            Ot, Lt = tiled_forward_head(q, k, v, 0.35, causal, bm, bq, bk)
            assert np.abs(O - Ot).max() <= 1e-13, ("tiled twin O", causal, bm is not None, bq, bk)
            fin = np.isfinite(L)
            assert np.array_equal(fin, np.isfinite(Lt)) and np.abs(L[fin] - Lt[fin]).max() <= 1e-13


# ----------------------------------------------------------------------------- backward
def _loss(forward_head, q, k, v, do, scale, causal, bm):
    O, _ = forward_head(q, k, v, scale, causal, bm)
    return float(np.sum(O * do))


def check_finite_differences(forward_head, backward_head, seed=10, h=1e-6):
    rng = np.random.default_rng(seed)
    cases = [(N, d, c) for N in (1, 2, 3, 5, 8, 13) for d in (1, 2, 4, 8) for c in (False, True)
             if not (N >= 8 and d >= 8 and not c)]
    for N, d, causal in cases:
        q, k, v, do = (rng.standard_normal((N, d)) for _ in range(4))
        scale = 0.75 if (N + d) % 2 else -0.75  # both signs of the scale
        dQ, dK, dV = backward_head(q, k, v, do, scale, causal, None)
        for name, X, G in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
            for idx in np.ndindex(*X.shape):
                old = X[idx]
                X[idx] = old + h
                lp = _loss(forward_head, q, k, v, do, scale, causal, None)
                X[idx] = old - h
                lm = _loss(forward_head, q, k, v, do, scale, causal, None)
                X[idx] = old
                fd = (lp - lm) / (2 * h)
                assert abs(fd - G[idx]) <= 1e-7 * max(1.0, abs(G[idx])), ("finite difference", name, N, d, causal, idx)


def check_finite_differences_masked(forward_head, backward_head, seed=11, h=1e-6):
    """Block-masked case (with a fully masked row block), on a sample of elements."""
    rng = np.random.default_rng(seed)
    N, d = 260, 2
    q, k, v, do = (rng.standard_normal((N, d)) for _ in range(4))
    mask = np.array([[1, 0, 1], [0, 0, 0], [1, 1, 0]], dtype=np.uint8)
    for causal in (False, True):
        dQ, dK, dV = backward_head(q, k, v, do, 0.6, causal, mask)
        assert np.all(dQ[128:256] == 0), "dead rows get zero dQ"
        for name, X, G in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
            for r in (0, 77, 127, 130, 256, 259):
                for c in range(d):
                    old = X[r, c]
                    X[r, c] = old + h
                    lp = _loss(forward_head, q, k, v, do, 0.6, causal, mask)
                    X[r, c] = old - h
                    lm = _loss(forward_head, q, k, v, do, 0.6, causal, mask)
                    X[r, c] = old
                    fd = (lp - lm) / (2 * h)
                    assert abs(fd - G[r, c]) <= 1e-6 * max(1.0, abs(G[r, c])), ("masked FD", name, causal, r, c)


def check_backward_invariants(forward_head, backward_head, probabilities, seed=12):
    rng = np.random.default_rng(seed)
    N, d = 90, 8
    q, k, v, do = (rng.standard_normal((N, d)) for _ in range(4))
    for causal in (False, True):
        dQ, dK, dV = backward_head(q, k, v, do, 0.45, causal, None)
        # sum over keys of dV equals sum over queries of dO (each P row sums to 1)
        assert np.abs(dV.sum(axis=0) - do.sum(axis=0)).max() <= 1e-11, ("sum dV", causal)
        # sum over keys of dK is zero (each dS row sums to zero)
        assert np.abs(dK.sum(axis=0)).max() <= 1e-11, ("sum dK", causal)
        # rowsum(P * dP) = rowsum(dO * O)
        P = probabilities(q, k, 0.45, causal)
        O, _ = forward_head(q, k, v, 0.45, causal)
        assert np.abs((P * (do @ v.T)).sum(axis=1) - (do * O).sum(axis=1)).max() <= 1e-12, ("D identity", causal)
        if causal:
            assert np.all(dQ[0] == 0), "causal row 0 has zero dQ"
    # N = 1: dV = dO, dQ = dK = 0
    dQ, dK, dV = backward_head(q[:1], k[:1], v[:1], do[:1], 0.45, False, None)
    assert np.abs(dV - do[:1]).max() <= 1e-15 and np.all(dQ == 0) and np.all(dK == 0), "N=1 backward"


def check_sampled_backward(backward_head, seed=13):
    rng = np.random.default_rng(seed)
    N, d = 300, 4
    q, k, v, do = (rng.standard_normal((N, d)) for _ in range(4))
    mask = np.array([[1, 0, 1], [1, 1, 0], [0, 1, 1]], dtype=np.uint8)
    dQ, dK, dV = backward_head(q, k, v, do, 0.5, True, mask, chunk=64)
    rows = np.array([0, 99, 200, 299])
    cols = np.array([1, 128, 257])
    sq, sk, sv = backward_head(q, k, v, do, 0.5, True, mask, dq_rows=rows, dkv_cols=cols, chunk=37)
    assert np.abs(sq - dQ[rows]).max() <= 1e-12 and np.abs(sk - dK[cols]).max() <= 1e-12
    assert np.abs(sv - dV[cols]).max() <= 1e-12, "sampled backward equals full"
    # dQ rows alone (no dK/dV columns: only the requested rows are visited), unsorted
    sel = [299, 5, 200, 99, 130]
    sq2, sk2, sv2 = backward_head(q, k, v, do, 0.5, True, mask, dq_rows=np.array(sel), dkv_cols=[], chunk=2)
    assert np.abs(sq2 - dQ[sel]).max() <= 1e-12 and sk2.shape == (0, 4) and sv2.shape == (0, 4)
