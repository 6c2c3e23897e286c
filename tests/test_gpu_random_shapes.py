"""GPU parity on seeded random shapes: B, H, ragged N, head dimension, dtype, causal flag, a
random 128 x 128 block mask and the scale (both signs) drawn from seeded generators, forward and
backward of every head compared with the fp64 oracle at the same tolerances as the other parity
tests.  The sizes stay small enough that the oracle finishes each case in well under a second."""
import math

import numpy as np
import pytest

import workloads
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

CASES = 48


def _draw(i):
    rng = np.random.default_rng(9000 + i)
    B = int(rng.integers(1, 3))
    H = int(rng.integers(1, 4))
    # ragged lengths around the 64-key tile, the 128-row block and their multiples
    N = int(rng.choice([int(rng.integers(1, 64)), int(rng.integers(64, 300)), int(rng.integers(300, 640))]))
    d = int(rng.choice([64, 128]))
    dtype = "fp32" if rng.random() < 0.25 else "bf16"
    causal = bool(rng.random() < 0.5)
    masked = bool(rng.random() < 0.4)
    scale = float(rng.uniform(0.3, 1.5)) / math.sqrt(d)
    if np.random.default_rng(7000 + i).random() < 0.5:  # a generator of its own: the draws above stay as they were
        scale = -scale
    return B, H, N, d, dtype, causal, masked, scale


@pytest.fixture(scope="module")
def dev():
    return G.device()


@pytest.mark.parametrize("i", range(CASES))
def test_random_shape(dev, i):
    B, H, N, d, dtype, causal, masked, scale = _draw(i)
    t = workloads.random_case(B, H, N, d, dtype, seed=9100 + i, mask_density=0.5 if masked else None,
                              mask_seed=9200 + i)
    if t.block_mask is not None:
        np.fill_diagonal(t.block_mask, 1)  # every query block keeps at least its own keys
    G.say(f"[case] random {i}: B={B} H={H} N={N} d={d} {dtype} causal={causal} mask={masked} "
          f"scale={scale:.4f}")
    res = G.run_lib(t, scale, causal, dev, True)
    G.compare_heads(t, res, scale, causal, [(b, h) for b in range(B) for h in range(H)], True)
