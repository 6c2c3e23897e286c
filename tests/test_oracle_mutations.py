"""Plant plausible mistakes in copies of the oracle (CPU only) and check that the pins catch each.

A pin suite that still passed with a dropped scale, a transposed operand, an off-by-one causal
mask, a swapped block-mask index, a log2 statistic or a wrong backward sign would not pin
anything.  The real oracle is not modified: each case wraps or replaces functions locally.
"""
import numpy as np
import pytest

import oracle
from oracle import attention as A
from tests import pins


def _forward_with_scores(scores_fn):
    def forward_head(q, k, v, scale, causal=False, block_mask=None, rows=None, chunk=1024):
        q = np.asarray(q, float)
        k = np.asarray(k, float)
        v = np.asarray(v, float)
        rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
        P, l, _ = A._softmax_rows(scores_fn(q, k, rows, scale, causal, block_mask))
        return P @ v, l
    return forward_head


def _scores_no_scale(q, k, rows, scale, causal, bm):
    return A._scores(q, k, rows, 1.0, causal, bm)


def _scores_causal_strict(q, k, rows, scale, causal, bm):
    S = scale * (q[rows] @ k.T)
    vis = A.visible(rows, np.arange(k.shape[0]), False, bm)
    if causal:
        vis &= np.arange(k.shape[0])[None, :] < rows[:, None]
    return np.where(vis, S, -np.inf)


def _scores_mask_transposed(q, k, rows, scale, causal, bm):
    bmT = None if bm is None else np.asarray(bm).T
    return A._scores(q, k, rows, scale, causal, bmT)


def _scores_q_for_k(q, k, rows, scale, causal, bm):
    # transposed operand: scores built from K rows against Q
    S = scale * (k[rows] @ q.T)
    vis = A.visible(rows, np.arange(k.shape[0]), causal, bm)
    return np.where(vis, S, -np.inf)


def _scores_abs_scale(q, k, rows, scale, causal, bm):
    # the sign of the scale lost
    return A._scores(q, k, rows, abs(scale), causal, bm)


def _forward_log2_lse(q, k, v, scale, causal=False, block_mask=None, rows=None, chunk=1024):
    O, L = oracle.forward_head(q, k, v, scale, causal, block_mask, rows, chunk)
    return O, L / np.log(2.0)


FORWARD_MUTANTS = {
    "dropped scale": _forward_with_scores(_scores_no_scale),
    "strict causal": _forward_with_scores(_scores_causal_strict),
    "transposed block mask": _forward_with_scores(_scores_mask_transposed),
    "transposed operand": _forward_with_scores(_scores_q_for_k),
    "log2 statistic": _forward_log2_lse,
    "sign of scale lost": _forward_with_scores(_scores_abs_scale),
}


def _all_forward_pins(fwd):
    pins.check_brute_force(fwd)
    pins.check_brute_force_masked(fwd)
    pins.check_identical_keys(fwd)
    pins.check_causal_row0_and_small_n(fwd)
    pins.check_one_hot_dominant(fwd)


@pytest.mark.parametrize("name", sorted(FORWARD_MUTANTS))
def test_forward_mutant_is_caught(name):
    with pytest.raises(AssertionError):
        _all_forward_pins(FORWARD_MUTANTS[name])


def _bwd_sign(q, k, v, do, scale, causal=False, block_mask=None, **kw):
    dq, dk, dv = oracle.backward_head(q, k, v, do, scale, causal, block_mask, **kw)
    return dq, -dk, dv


def _bwd_no_scale(q, k, v, do, scale, causal=False, block_mask=None, **kw):
    dq, dk, dv = oracle.backward_head(q, k, v, do, scale, causal, block_mask, **kw)
    return dq / scale, dk, dv


def _bwd_no_D(q, k, v, do, scale, causal=False, block_mask=None, **kw):
    # dS = P * dP (the rowsum term dropped)
    q, k, v, do = (np.asarray(x, float) for x in (q, k, v, do))
    P = oracle.probabilities(q, k, scale, causal, block_mask)
    dP = do @ v.T
    dS = P * dP
    return scale * dS @ k, scale * dS.T @ q, P.T @ do


BACKWARD_MUTANTS = {"dK sign": _bwd_sign, "dQ scale": _bwd_no_scale, "dropped D": _bwd_no_D}


@pytest.mark.parametrize("name", sorted(BACKWARD_MUTANTS))
def test_backward_mutant_is_caught(name):
    with pytest.raises(AssertionError):
        pins.check_finite_differences(oracle.forward_head, BACKWARD_MUTANTS[name])
