"""The checking build (-DFA_CHECK): every asynchronous copy into LDS first fills its destination
with NaN, and the paired dK/dV kernel poisons each P exchange slot once it is consumed, so a read
that runs ahead of its copy or of the barrier that publishes it carries NaN into the results.
The small-N sweep and the other entry points run against that build here, compared with the oracle
(the same bar as the parity tests; any NaN fails)."""
import math

import numpy as np
import pytest

import workloads
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def check_lib():
    import exact_io_aware_flash_amd as fa
    from exact_io_aware_flash_amd import build as B

    G.device()
    path = B.variant_path("check")
    if not fa.os.path.exists(path):
        pytest.fail(f"{path} missing: build it with python -m exact_io_aware_flash_amd.build")
    return fa.load(path)


@pytest.fixture
def on_check_build(check_lib, monkeypatch):
    import exact_io_aware_flash_amd as fa

    monkeypatch.setattr(fa, "_lib", check_lib)
    yield


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode", ["dense", "causal", "mask", "causal+mask"])
def test_sentinel_small_n_sweep(on_check_build, d, mode):
    dev = G.device()
    causal = "causal" in mode
    for N in (1, 63, 65, 129, 300, 1000):
        t = workloads.random_case(1, 2, N, d, "bf16", seed=4100 + N, mask_density=0.6 if "mask" in mode else None,
                                  mask_seed=4200 + N)
        if t.block_mask is not None:
            np.fill_diagonal(t.block_mask, 1)
        G.say(f"[case] check build N={N} d={d} {mode}")
        res = G.run_lib(t, 1.0 / math.sqrt(d), causal, dev)
        G.compare_heads(t, res, 1.0 / math.sqrt(d), causal, heads=[(0, 0), (0, 1)])


def test_sentinel_other_entry_points(on_check_build):
    """Split-key forward, the wave-specialised forward, the one-pass backward and the MX-FP8
    forward through the checking build (several tiles, ragged N)."""
    import torch

    import exact_io_aware_flash_amd as fa

    dev = G.device()
    t = workloads.random_case(1, 2, 1000, 128, "bf16", seed=4300)
    q, k, v, do = (G.to_dev(x, "bf16", dev) for x in (t.q, t.k, t.v, t.do))
    for causal in (False, True):
        o, lse = fa.fwd_splitkv(q, k, v, 0.09, causal, None, 3)
        o2, lse2 = fa.fwd_pingpong(q, k, v, 0.09, causal)
        dq, dk, dv = fa.bwd_onepass(q, k, v, o2, lse2, do, 0.09, causal)
        torch.cuda.synchronize()
        G.compare_heads(t, {"o": o, "lse": lse}, 0.09, causal, heads=[(0, 0)], backward=False)
        G.compare_heads(t, {"o": o2, "lse": lse2, "dq": dq, "dk": dk, "dv": dv}, 0.09, causal, heads=[(0, 1)])
    # MX-FP8 forward: the check build against the normal build (same kernels, same inputs)
    Q8, K8, V8 = fa.mxfp8_quantize(q), fa.mxfp8_quantize(k), fa.mxfp8_quantize(v, transposed=True)
    o8, l8 = fa.fwd_mxfp8(Q8, K8, V8, 0.09, True)
    torch.cuda.synchronize()
    assert not torch.isnan(o8).any().item() and not torch.isnan(l8).any().item()
    ref = fa.load(fa.LIB_PATH)
    saved = fa._lib
    fa._lib = ref
    try:
        o8r, l8r = fa.fwd_mxfp8(Q8, K8, V8, 0.09, True)
        torch.cuda.synchronize()
    finally:
        fa._lib = saved
    assert torch.equal(o8, o8r) and torch.equal(l8, l8r)
