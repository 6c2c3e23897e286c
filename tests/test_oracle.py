"""Pins of the fp64 oracle (CPU only).  See tests/pins.py for what each check establishes."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads
from tests import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_brute_force():
    pins.check_brute_force(oracle.forward_head)


def test_brute_force_block_mask():
    pins.check_brute_force_masked(oracle.forward_head)


def test_probabilities_sum_to_one():
    pins.check_probabilities_sum_to_one(oracle.probabilities)


def test_identical_keys_mean_of_v():
    pins.check_identical_keys(oracle.forward_head)


def test_one_hot_dominant_row():
    pins.check_one_hot_dominant(oracle.forward_head)


def test_causal_row0_and_closed_forms():
    pins.check_causal_row0_and_small_n(oracle.forward_head)


def test_causal_is_prefix_attention():
    pins.check_causal_is_prefix_attention(oracle.forward_head)


def test_permutation_and_shift_invariance():
    pins.check_permutation_and_shift(oracle.forward_head)


def test_mask_equivalences_and_dead_rows():
    pins.check_mask_equivalences(oracle.forward_head)


def test_tiled_online_softmax_equals_definition():
    pins.check_tiled_twin(oracle.forward_head, oracle.tiled_forward_head)


def test_backward_finite_differences():
    pins.check_finite_differences(oracle.forward_head, oracle.backward_head)


def test_backward_finite_differences_block_mask():
    pins.check_finite_differences_masked(oracle.forward_head, oracle.backward_head)


def test_backward_invariants():
    pins.check_backward_invariants(oracle.forward_head, oracle.backward_head, oracle.probabilities)


def test_sampled_backward_matches_full():
    pins.check_sampled_backward(oracle.backward_head)


def test_batched_wrappers_match_heads():
    rng = np.random.default_rng(14)
    q, k, v, do = (rng.standard_normal((2, 3, 40, 4)) for _ in range(4))
    O, L = oracle.forward(q, k, v, 0.5, True, chunk=16)
    dQ, dK, dV = oracle.backward(q, k, v, do, 0.5, True, chunk=16)
    for b in range(2):
        for h in range(3):
            o, l = oracle.forward_head(q[b, h], k[b, h], v[b, h], 0.5, True)
            g = oracle.backward_head(q[b, h], k[b, h], v[b, h], do[b, h], 0.5, True)
            assert np.abs(O[b, h] - o).max() <= 1e-14 and np.abs(L[b, h] - l).max() <= 1e-14
            for a, c in zip((dQ, dK, dV), g):
                assert np.abs(a[b, h] - c).max() <= 1e-13


def test_s_matrix_size_against_pages():
    """The pages print the size of one fp32 N x N score matrix; the bench uses this helper for the
    traffic that exact tiled attention avoids."""
    with open(os.path.join(GOLDEN, "s_matrix_sizes.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        got = oracle.s_matrix_bytes(case["N"], 4)
        if "approx_bytes" in case:
            assert abs(got - case["approx_bytes"]) <= case["rel_tol"] * case["approx_bytes"], case
        if "min_bytes" in case:
            assert got > case["min_bytes"], case


# ----------------------------------------------------------------------------- input generator
def test_bf16_rounding_is_round_to_nearest_even():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(15)
    x = rng.standard_normal(100000).astype(np.float32) * np.float32(3.0)
    # exact ties: low 16 bits = 0x8000 with both parities of bit 16
    ties = (np.arange(2000, dtype=np.uint32) << 17 | 0x3F800000 | 0x8000).view(np.float32)
    ties_odd = ((np.arange(2000, dtype=np.uint32) << 17) | 0x3F810000 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, ties_odd, np.array([0.0, -0.0, 1e-40, 3.4e38, -3.4e38], np.float32)])
    ours = workloads.round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = workloads.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_workload_recipe_is_seeded_and_shaped():
    t1 = workloads.make("bert", B=1, H=2, N=64)
    t2 = workloads.make("bert", B=1, H=2, N=64)
    assert t1.q.shape == (1, 2, 64, 64) and t1.q.dtype == np.uint16
    assert all(np.array_equal(getattr(t1, n), getattr(t2, n)) for n in ("q", "k", "v", "do"))
    assert not np.array_equal(t1.q, t1.k)
    sp = workloads.make("sparse", B=1, H=1, N=8192, with_do=False)
    m = sp.block_mask
    assert m.shape == (64, 64)
    i = np.arange(64)
    assert np.all(m[i, i] == 1) and np.all(m[:, 0] == 1) and np.all(m[i[3:], i[3:] - 3] == 1)
    fixed = ((i[None] <= i[:, None]) & (i[None] >= i[:, None] - 3)) | (i[None] == 0)
    extra_frac = (m.astype(bool) & ~fixed).sum() / (~fixed).sum()
    assert 0.07 < extra_frac < 0.13


def test_flop_convention():
    assert workloads.flops_fwd(1, 1, 256, 64, False) == 4 * 256 * 256 * 64
    assert workloads.flops_fwd(1, 32, 16384, 128, True) == 4 * 32 * 16384 ** 2 * 128 / 2
    m = np.eye(4, dtype=np.uint8)
    assert workloads.flops_fwd(2, 3, 512, 64, False, m) == 4 * 6 * 64 * 128 * 128 * 4
    assert workloads.flops_bwd(1, 1, 256, 64, False) == 2.5 * workloads.flops_fwd(1, 1, 256, 64, False)
