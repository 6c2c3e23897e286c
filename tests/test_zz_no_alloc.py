"""flash_attn_bwd_noalloc (the backward for callers that cannot allocate device memory) against
flash_attn_bwd, both called through the C ABI: two calls in a row on one device, the second with
a smaller input (the fixed scratch keeps the first call's contents, which must not leak into the
second), then the largest accepted size.  The same kernels run in both entry points, so the
results must be bitwise equal."""
import ctypes
import math

import numpy as np
import pytest

import workloads
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return G.device()


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _both(L, q, k, v, do, scale, causal, mask):
    """(reference through flash_attn_bwd with a caller workspace, result of flash_attn_bwd_noalloc)"""
    import torch

    import exact_io_aware_flash_amd as fa

    B, H, N, d = q.shape
    o, lse = fa.fwd(q, k, v, scale, causal, mask)
    nan = lambda: torch.full_like(q, float("nan"))
    ref = [nan(), nan(), nan()]
    ws = fa.new_workspace(B, H, N, d, q.device)
    st = L.flash_attn_bwd(_p(q), _p(k), _p(v), _p(o), _p(do), _p(lse), *(_p(x) for x in ref), _p(ws),
                          ws.numel(), B, H, N, d, scale, int(causal), _p(mask) if mask is not None else None, None)
    assert st == fa.FA_OK, fa.status_string(st)
    got = [nan(), nan(), nan()]
    st = L.flash_attn_bwd_noalloc(_p(q), _p(k), _p(v), _p(o), _p(do), _p(lse), *(_p(x) for x in got), B, H, N, d,
                                  scale, int(causal), _p(mask) if mask is not None else None, None)
    assert st == fa.FA_OK, fa.status_string(st)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_bwd_two_calls(dev):
    import torch

    import exact_io_aware_flash_amd as fa

    L = fa.lib()
    cases = [
        # the larger call first, then a smaller one with another head dimension and a block mask
        (2, 4, 1000, 128, True, None, 0.09),
        (1, 2, 300, 64, False, 0.6, -0.125),
    ]
    for i, (B, H, N, d, causal, dens, scale) in enumerate(cases):
        G.say(f"[case] noalloc call {i}: B={B} H={H} N={N} d={d} causal={causal} mask={dens} scale={scale}")
        t = workloads.random_case(B, H, N, d, "bf16", seed=2500 + i, mask_density=dens, mask_seed=2600 + i)
        if t.block_mask is not None:
            np.fill_diagonal(t.block_mask, 1)
        q, k, v, do = (G.to_dev(x, "bf16", dev) for x in (t.q, t.k, t.v, t.do))
        mask = torch.from_numpy(t.block_mask).to(dev) if t.block_mask is not None else None
        ref, got = _both(L, q, k, v, do, scale, causal, mask)
        for name, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert not torch.isnan(b).any().item(), f"{name}: unwritten elements"
            assert torch.equal(a, b), f"call {i}: {name} differs from flash_attn_bwd"
        # and both are the oracle's to the bf16 bar on one head
        o, lse = fa.fwd(q, k, v, scale, causal, mask)
        G.compare_heads(t, {"o": o, "lse": lse, "dq": got[0], "dk": got[1], "dv": got[2]}, scale, causal,
                        heads=[(0, 1)])


def test_noalloc_largest_size(dev):
    """B * H * N = FA_NOALLOC_MAX_ROWS exactly is accepted and matches flash_attn_bwd; one more
    row is refused before anything is enqueued."""
    import torch

    import exact_io_aware_flash_amd as fa

    L = fa.lib()
    B, H, N, d = 1, 1024, 4096, 64
    assert B * H * N == fa.NOALLOC_MAX_ROWS
    G.say(f"[case] noalloc largest: B={B} H={H} N={N} d={d} causal")
    g = torch.Generator(device=dev)
    g.manual_seed(2700)
    mk = lambda: torch.randn((B, H, N, d), device=dev, generator=g).to(torch.bfloat16)
    q, k, v, do = mk(), mk(), mk(), mk()
    ref, got = _both(L, q, k, v, do, 1.0 / math.sqrt(d), True, None)
    for name, a, b in zip(("dq", "dk", "dv"), ref, got):
        assert torch.equal(a, b), f"largest: {name} differs from flash_attn_bwd"
    st = L.flash_attn_bwd_noalloc(_p(q), _p(k), _p(v), _p(q), _p(do), _p(q), *(_p(x) for x in got), B, H + 1, N - 1,
                                  d, 0.125, 1, None, None)
    assert st == fa.FA_ERR_SCRATCH
