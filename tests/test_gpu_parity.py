"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle, element by element.

Tolerances: max-abs 1e-5 for fp32 inputs, 2e-2 for bf16 inputs (fp32 accumulation; for bf16
outputs half a bf16 ulp of the reference value is added, the output's own storage rounding),
1e-3 for LSE.  Full-size workloads are run on the device in full; the oracle checks
sampled heads, rows and key columns of them.
"""
import math
import time

import numpy as np
import pytest

import workloads
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return G.device()


def _run_and_compare(name, t, scale, causal, dev, heads, backward=True, rows=None, cols=None):
    G.say(f"[case] {name}: shape={t.q.shape} dtype={t.dtype} causal={causal} "
          f"mask={'yes' if t.block_mask is not None else 'no'} bwd={backward}")
    t0 = time.time()
    res = G.run_lib(t, scale, causal, dev, backward)
    G.say(f"  device done in {time.time() - t0:.1f}s")
    G.compare_heads(t, res, scale, causal, heads, backward, rows, cols)
    return res


# ------------------------------------------------------------------------------ the workloads
def test_tiny_fp32_exact(dev):
    w = workloads.WORKLOADS["tiny"]
    t = workloads.make(w)
    _run_and_compare("tiny fp32", t, w.scale, w.causal, dev, heads=[(0, 0)])


def test_bert_shaped_full(dev):
    w = workloads.WORKLOADS["bert"]
    t = workloads.make(w)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    _run_and_compare("bert", t, w.scale, w.causal, dev, heads)


def _run_every_tile(name, w, t, dev, seed, kv_heads, backward=True):
    G.say(f"[case] {name}: shape={t.q.shape} causal={w.causal} mask={'yes' if t.block_mask is not None else 'no'} "
          f"bwd={backward} (one row per query tile on every head; one key per key block on {len(kv_heads)} heads)")
    t0 = time.time()
    res = G.run_lib(t, w.scale, w.causal, dev, backward)
    G.say(f"  device done in {time.time() - t0:.1f}s")
    G.compare_every_tile(t, res, w.scale, w.causal, seed, kv_heads, backward)


def _spread_heads(B, H, n):
    """n heads spread over the (b, h) grid, first and last included."""
    idx = np.unique(np.linspace(0, B * H - 1, n).round().astype(int))
    return {(int(i) // H, int(i) % H) for i in idx}


def test_gpt2_shaped_causal(dev):
    w = workloads.WORKLOADS["gpt2"]
    t = workloads.make(w)
    _run_every_tile("gpt2", w, t, dev, seed=30, kv_heads=_spread_heads(w.B, w.H, 8))


def test_long_context_causal_every_tile(dev):
    w = workloads.WORKLOADS["long"]
    t = workloads.make(w)
    _run_every_tile("long", w, t, dev, seed=40, kv_heads=_spread_heads(w.B, w.H, 8))


def test_long_context_64k_forward_every_tile(dev):
    w = workloads.WORKLOADS["long64k"]
    t = workloads.make(w, with_do=False)
    _run_every_tile("long64k fwd", w, t, dev, seed=50, kv_heads=set(), backward=False)


def test_head_major_schedule_sampled(dev):
    """B*H = 16 heads of N = 8192, d = 128, causal: two heads per XCD group, each with as many
    tiles as the XCD holds workgroups or more, so every grid runs head by head, and the forward
    alternates its key direction by cohort."""
    t = workloads.random_case(2, 8, 8192, 128, "bf16", seed=900)
    rows = G.sample_rows(8192, 40, seed=901)
    cols = G.sample_rows(8192, 40, seed=902)
    _run_and_compare("head-major N=8192 d=128", t, 1.0 / math.sqrt(128), True, dev, heads=[(0, 0), (1, 7)],
                     rows=rows, cols=cols)


@pytest.mark.parametrize("d", [64, 128])
def test_head_major_equal_tiles_sampled(dev, d):
    """Non-causal heads whose tiles carry equal work run head by head even when a head has fewer
    tiles than the XCD holds workgroups: B*H = 16 heads of N = 2048 (8 to 16 tiles per head)."""
    t = workloads.random_case(2, 8, 2048, d, "bf16", seed=910 + d)
    rows = G.sample_rows(2048, 40, seed=911)
    cols = G.sample_rows(2048, 40, seed=912)
    _run_and_compare(f"head-major equal tiles N=2048 d={d}", t, 1.0 / math.sqrt(d), False, dev,
                     heads=[(0, 0), (0, 5), (1, 2), (1, 7)], rows=rows, cols=cols)


def test_block_sparse(dev):
    w = workloads.WORKLOADS["sparse"]
    t = workloads.make(w)
    _run_every_tile("sparse", w, t, dev, seed=60, kv_heads=_spread_heads(w.B, w.H, 8))


# ------------------------------------------------------------------------------ sweeps and edges
SMALL_N = [1, 2, 3, 17, 63, 64, 65, 127, 128, 129, 255, 300]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("mode", ["dense", "causal", "mask", "causal+mask"])
def test_small_n_sweep(dev, d, dtype, mode):
    causal = "causal" in mode
    for N in SMALL_N:
        t = workloads.random_case(1, 2, N, d, dtype, seed=100 + N,
                                  mask_density=0.6 if "mask" in mode else None, mask_seed=200 + N)
        if t.block_mask is not None:
            np.fill_diagonal(t.block_mask, 1)
        _run_and_compare(f"sweep N={N} d={d} {dtype} {mode}", t, 1.0 / math.sqrt(d), causal, dev,
                         heads=[(0, 0), (0, 1)])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_multi_tile(dev, d, causal):
    t = workloads.random_case(2, 3, 1000, d, "bf16", seed=300 + d, mask_density=0.5, mask_seed=301)
    np.fill_diagonal(t.block_mask, 1)
    _run_and_compare(f"ragged N=1000 d={d}", t, 0.1, causal, dev, heads=[(0, 0), (1, 2)])
    t.block_mask = None
    _run_and_compare(f"ragged dense N=1000 d={d}", t, 0.1, causal, dev, heads=[(0, 1), (1, 0)])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("mode", ["dense", "causal", "mask", "causal+mask"])
def test_negative_scale(dev, d, dtype, mode):
    """A negative scale (S = scale Q K^T reverses which keys dominate): forward and backward
    against the oracle, one and several tiles, ragged tails."""
    causal = "causal" in mode
    for N in (63, 300, 1000):
        t = workloads.random_case(1, 2, N, d, dtype, seed=1700 + N + d,
                                  mask_density=0.6 if "mask" in mode else None, mask_seed=1800 + N)
        if t.block_mask is not None:
            np.fill_diagonal(t.block_mask, 1)
        _run_and_compare(f"negative scale N={N} d={d} {dtype} {mode}", t, -1.0 / math.sqrt(d), causal, dev,
                         heads=[(0, 0), (0, 1)])


def test_negative_scale_long_sampled(dev):
    """Negative scale on a long causal head (N = 8192, d = 128: many tiles, the running maximum
    moving), sampled rows and key columns."""
    t = workloads.random_case(1, 8, 8192, 128, "bf16", seed=1900)
    rows = G.sample_rows(8192, 40, seed=1901)
    cols = G.sample_rows(8192, 40, seed=1902)
    _run_and_compare("negative scale N=8192 d=128", t, -1.0 / math.sqrt(128), True, dev, heads=[(0, 0), (0, 5)],
                     rows=rows, cols=cols)


@pytest.mark.gpu
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mult", [16.0, 64.0])
def test_sharp_softmax_forward(dev, d, mult):
    """Scores far larger than the workloads' (scale = mult / sqrt(d), both signs): most rows are
    close to one-hot, LSE reaches a few hundred, and the running maximum moves past the rescale
    threshold many times along a row. Forward only, against the oracle at the stated bars: the
    bf16 backward rounds dS, whose error grows with the scores and leaves the stated bar at such
    scales (an error budget of the rounding alone, not of the kernels)."""
    for i, (causal, dens, sign) in enumerate(((False, None, 1.0), (True, None, -1.0), (False, 0.5, 1.0))):
        t = workloads.random_case(1, 2, 700, d, "bf16", seed=2300 + 10 * i + d, with_do=False, mask_density=dens)
        _run_and_compare(f"sharp softmax x{mult:g} d={d} causal={causal} mask={dens}", t, sign * mult / math.sqrt(d),
                         causal, dev, heads=[(0, 0), (0, 1)], backward=False)


@pytest.mark.gpu
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_flat_softmax(dev, d, causal):
    """scale = 1e-3: every row nearly uniform over the keys it sees (LSE close to the log of their
    count, P close to its mean everywhere), forward and backward."""
    t = workloads.random_case(1, 2, 700, d, "bf16", seed=2400 + d + int(causal))
    _run_and_compare(f"flat softmax d={d} causal={causal}", t, 1e-3, causal, dev, heads=[(0, 0), (0, 1)])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_dead_rows(dev, dtype, d):
    """Rows that see no key: O = 0, LSE = -inf, no gradient (a zero mask row; and causal with a
    mask that only allows later blocks)."""
    N = 384
    t = workloads.random_case(1, 2, N, d, dtype, seed=400 + d)
    t.block_mask = np.array([[1, 0, 0], [0, 0, 0], [1, 1, 1]], dtype=np.uint8)
    res = _run_and_compare(f"dead rows {dtype} d={d}", t, 1.0 / math.sqrt(d), False, dev, heads=[(0, 0), (0, 1)])
    o = G.host_f64(res["o"])
    assert np.all(o[:, :, 128:256] == 0)
    assert np.all(np.isneginf(res["lse"][:, :, 128:256].cpu().numpy()))
    assert np.all(G.host_f64(res["dq"])[:, :, 128:256] == 0)
    t.block_mask = np.array([[0, 1, 1], [1, 0, 1], [1, 1, 1]], dtype=np.uint8)
    res = _run_and_compare(f"dead rows causal {dtype} d={d}", t, 1.0 / math.sqrt(d), True, dev,
                           heads=[(0, 0), (0, 1)])
    assert np.all(np.isneginf(res["lse"][:, :, 0:128].cpu().numpy()))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_empty_key_block(dev, d, causal):
    """A key block that no query block sees (an empty mask column): its workgroup has no query
    tile at all, and dK, dV of its keys are exactly zero; the other blocks match the oracle."""
    N = 3 * 128 - 40  # ragged last block
    t = workloads.random_case(1, 2, N, d, "bf16", seed=450 + d)
    t.block_mask = np.array([[1, 0, 0], [1, 0, 1], [1, 0, 1]], dtype=np.uint8)
    res = _run_and_compare(f"empty key block d={d} causal={causal}", t, 1.0 / math.sqrt(d), causal, dev,
                           heads=[(0, 0), (0, 1)])
    assert np.all(G.host_f64(res["dk"])[:, :, 128:256] == 0)
    assert np.all(G.host_f64(res["dv"])[:, :, 128:256] == 0)


def test_invariants_on_device_outputs(dev):
    """Second witnesses on the device results: identical keys give the mean of the visible V;
    causal row 0 returns V[0] exactly; sums of dV and dK over keys."""
    import torch

    import exact_io_aware_flash_amd as fa

    N, d = 256, 64
    t = workloads.random_case(1, 1, N, d, "bf16", seed=500)
    t.k[:] = t.k[:, :, :1, :]
    q = G.to_dev(t.q, "bf16", dev)
    k = G.to_dev(t.k, "bf16", dev)
    v = G.to_dev(t.v, "bf16", dev)
    do = G.to_dev(t.do, "bf16", dev)
    for causal in (False, True):
        o, lse = fa.fwd(q, k, v, 0.125, causal)
        vv = G.host_f64(v)[0, 0]
        ref = np.cumsum(vv, 0) / np.arange(1, N + 1)[:, None] if causal else np.tile(vv.mean(0), (N, 1))
        G.check(f"identical keys causal={causal}", G.host_f64(o)[0, 0], ref, G.TOL_BF16, True)
        if causal:
            assert np.array_equal(G.host_f64(o)[0, 0, 0], vv[0]), "causal row 0 must return V[0]"
        dq, dk, dv = fa.bwd(q, k, v, o, lse, do, 0.125, causal)
        torch.cuda.synchronize()
        dvs, dos = G.host_f64(dv)[0, 0].sum(0), G.host_f64(do)[0, 0].sum(0)
        assert np.abs(dvs - dos).max() < 0.05 * math.sqrt(N), "sum_j dV_j = sum_i dO_i"
        assert np.abs(G.host_f64(dk)[0, 0].sum(0)).max() < 0.05 * math.sqrt(N), "sum_j dK_j = 0"


@pytest.mark.parametrize("causal", [False, True])
def test_dominant_score_on_device_outputs(dev, causal):
    """Second witness on the device results (one-hot dominant row): with Q_i = 10 K_j* for one
    visible key j* per row, the score of j* exceeds every other visible score by tens of nats, so
    O_i = V_j* (up to the bf16 rounding of P and of O) and LSE_i = scale Q_i K_j* (the other keys
    add about e^-40 to the sum).  Several tiles, a ragged tail, d = 128."""
    import torch

    import exact_io_aware_flash_amd as fa

    N, d = 300, 128
    scale = 1.0 / math.sqrt(d)
    t = workloads.random_case(1, 1, N, d, "bf16", seed=520, with_do=False)
    rng = np.random.default_rng(521)
    jstar = np.array([rng.integers(0, i + 1) if causal else rng.integers(0, N) for i in range(N)])
    # Q_i = 10 K_j*, rounded to bf16 (the inputs are bf16 bit patterns); the reference reads the
    # device copy back
    t.q[0, 0] = workloads.round_to_bf16_bits(10.0 * workloads.bf16_bits_to_f32(t.k[0, 0, jstar]))
    q, k, v = (G.to_dev(x, "bf16", dev) for x in (t.q, t.k, t.v))
    o, lse = fa.fwd(q, k, v, scale, causal)
    torch.cuda.synchronize()
    qh, kh, vh = (G.host_f64(x)[0, 0] for x in (q, k, v))
    s = scale * qh @ kh.T
    if causal:
        s = np.where(np.tril(np.ones((N, N), bool)), s, -np.inf)
    gap = s[np.arange(N), jstar] - np.max(np.where(np.eye(N, dtype=bool)[jstar], -np.inf, s), axis=1)
    assert gap.min() > 40.0, gap.min()  # the construction holds (causal row 0 sees one key: gap inf)
    G.check(f"dominant row O causal={causal}", G.host_f64(o)[0, 0], vh[jstar], G.TOL_BF16, True)
    G.check(f"dominant row LSE causal={causal}", G.host_f64(lse)[0, 0], s[np.arange(N), jstar], G.TOL_LSE, False)


def test_bitwise_reproducible(dev):
    import torch

    t = workloads.random_case(2, 4, 700, 128, "bf16", seed=600)
    a = G.run_lib(t, 0.09, True, dev)
    b = G.run_lib(t, 0.09, True, dev)
    for kname in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(a[kname], b[kname]), kname


def test_non_default_stream(dev):
    import torch

    import exact_io_aware_flash_amd as fa

    t = workloads.random_case(1, 2, 300, 64, "bf16", seed=700)
    q, k, v = (G.to_dev(x, "bf16", dev) for x in (t.q, t.k, t.v))
    ref_o, ref_l = fa.fwd(q, k, v, 0.125, True)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, l = fa.fwd(q, k, v, 0.125, True)
    s.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)


def test_explicit_stream_argument(dev):
    """stream= passed explicitly (not the current stream): the binding's internal temporaries
    (the backward's workspace, the split-key partials) stay reserved for that stream while its
    kernels run, though allocations and kernels on the current stream follow in between."""
    import torch

    import exact_io_aware_flash_amd as fa

    t = workloads.random_case(2, 4, 2000, 128, "bf16", seed=710)
    q, k, v, do = (G.to_dev(x, "bf16", dev) for x in (t.q, t.k, t.v, t.do))
    ref_o, ref_l = fa.fwd(q, k, v, 0.09, True)
    ref_g = fa.bwd(q, k, v, ref_o, ref_l, do, 0.09, True)
    ref_s = fa.fwd_splitkv(q, k, v, 0.09, True, None, 4)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    o, l = fa.fwd(q, k, v, 0.09, True, stream=s)
    s.synchronize()
    g = fa.bwd(q, k, v, o, l, do, 0.09, True, stream=s)
    so = fa.fwd_splitkv(q, k, v, 0.09, True, None, 4, stream=s)
    # allocations and writes on the current stream while the kernels on s may still run
    junk = [torch.full((1 << 20,), 3.0, device=dev) for _ in range(8)]
    for j in junk:
        j.mul_(2.0)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)
    for a, b in zip(g, ref_g):
        assert torch.equal(a, b)
    assert torch.equal(so[0], ref_s[0]) and torch.equal(so[1], ref_s[1])


def test_graph_capture_replays(dev):
    """The library's launches (forward, the three backward stages, the allocation-free backward)
    captured into one HIP graph: every replay, with eager work and synchronisations between
    replays, equals the eager results bitwise."""
    import torch

    import exact_io_aware_flash_amd as fa

    t = workloads.random_case(2, 4, 777, 128, "bf16", seed=760)
    q, k, v, do = (G.to_dev(x, "bf16", dev) for x in (t.q, t.k, t.v, t.do))
    o, lse = fa.fwd(q, k, v, 0.1, True)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, 0.1, True)
    torch.cuda.synchronize()
    go, gl = torch.empty_like(o), torch.empty_like(lse)
    gq, gk, gv, nq, nk, nv = (torch.empty_like(q) for _ in range(6))
    ws = fa.new_workspace(2, 4, 777, 128, dev)
    # warm: the launchers' one-time queries and the scratch lookup of the allocation-free entry
    # point run eagerly, outside the capture
    fa.fwd(q, k, v, 0.1, True, out=go, lse=gl)
    fa.bwd_noalloc(q, k, v, go, gl, do, nq, nk, nv, 0.1, True)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.fwd(q, k, v, 0.1, True, out=go, lse=gl)
        fa.bwd_preprocess(q, go, do, ws)
        fa.bwd_dkdv(q, k, v, do, gl, ws, 0.1, True, None, gk, gv)
        fa.bwd_dq(q, k, v, do, gl, ws, 0.1, True, None, gq)
        fa.bwd_noalloc(q, k, v, go, gl, do, nq, nk, nv, 0.1, True)
    for r in range(3):
        for x in (go, gl, gq, gk, gv, nq, nk, nv):
            x.fill_(float("nan"))
        junk = torch.randn(1 << 20, device=dev).sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(go, o) and torch.equal(gl, lse), f"replay {r}: forward"
        for a, b in ((gq, dq), (gk, dk), (gv, dv), (nq, dq), (nk, dk), (nv, dv)):
            assert torch.equal(a, b), f"replay {r}: backward"
        del junk


def test_invalid_call_leaves_outputs_untouched(dev):
    import ctypes

    import torch

    import exact_io_aware_flash_amd as fa

    q = torch.randn(1, 1, 128, 64, device=dev).to(torch.bfloat16)
    o = torch.full_like(q, 7.0)
    lse = torch.full((1, 1, 128), 3.0, device=dev)
    L = fa.lib()
    p = lambda x: ctypes.c_void_p(x.data_ptr())
    st = L.flash_attn_fwd(p(q), p(q), p(q), p(o), p(lse), 1, 1, 128, 96, 0.125, 0, None, None)
    assert st == fa.FA_ERR_HEADDIM
    st = L.flash_attn_fwd(p(q), p(q), p(q), p(o), p(lse), 1, 1, 128, 64, float("nan"), 0, None, None)
    assert st == fa.FA_ERR_SCALE
    torch.cuda.synchronize()
    assert torch.all(o == 7.0) and torch.all(lse == 3.0)
    with pytest.raises(fa.FlashAttnError):
        fa.fwd(q, q, q, scale=0.0)


def test_backward_stages_equal_bwd(dev):
    import torch

    import exact_io_aware_flash_amd as fa

    t = workloads.random_case(2, 3, 777, 128, "bf16", seed=800, mask_density=0.5, mask_seed=801)
    np.fill_diagonal(t.block_mask, 1)
    q, k, v, do = (G.to_dev(x, "bf16", dev) for x in (t.q, t.k, t.v, t.do))
    mask = torch.from_numpy(t.block_mask).to(dev)
    for causal, bm in ((False, None), (True, None), (True, mask)):
        o, lse = fa.fwd(q, k, v, 0.1, causal, bm)
        dq, dk, dv = fa.bwd(q, k, v, o, lse, do, 0.1, causal, bm)
        ws = fa.bwd_preprocess(q, o, do)
        dk2, dv2 = fa.bwd_dkdv(q, k, v, do, lse, ws, 0.1, causal, bm)
        dq2 = fa.bwd_dq(q, k, v, do, lse, ws, 0.1, causal, bm)
        torch.cuda.synchronize()
        assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)


def test_autograd_wrapper(dev):
    """attention() as a torch.autograd operation: its forward equals fwd() and its gradients equal
    bwd() bit for bit, and both match the oracle."""
    import torch

    import exact_io_aware_flash_amd as fa

    t = workloads.random_case(1, 2, 300, 64, "bf16", seed=1100)
    q, k, v, do = (G.to_dev(x, "bf16", dev) for x in (t.q, t.k, t.v, t.do))
    qa, ka, va = (x.clone().requires_grad_(True) for x in (q, k, v))
    o = fa.attention(qa, ka, va, 0.125, True)
    o.backward(do)
    o_ref, lse_ref = fa.fwd(q, k, v, 0.125, True)
    dq_ref, dk_ref, dv_ref = fa.bwd(q, k, v, o_ref, lse_ref, do, 0.125, True)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o_ref)
    assert torch.equal(qa.grad, dq_ref) and torch.equal(ka.grad, dk_ref) and torch.equal(va.grad, dv_ref)
    res = {"o": o.detach(), "lse": lse_ref, "dq": qa.grad, "dk": ka.grad, "dv": va.grad}
    G.compare_heads(t, res, 0.125, True, heads=[(0, 0), (0, 1)])


# ------------------------------------------------------------------------------ one-pass backward
@pytest.mark.parametrize("mode", ["dense", "causal", "mask", "causal+mask"])
def test_onepass_backward_matches_oracle(dev, mode):
    """The one-pass backward (dQ by float32 atomics): dV bitwise equal to flash_attn_bwd's, dQ, dK
    and dV within the bar of the oracle; ragged N from one tile to many, both signs of scale."""
    import torch

    import exact_io_aware_flash_amd as fa

    causal = "causal" in mode
    for N, scale in ((1, 0.09), (65, 0.09), (300, -0.09), (1000, 0.09), (2049, 0.11)):
        t = workloads.random_case(1, 2, N, 128, "bf16", seed=3300 + N, mask_density=0.6 if "mask" in mode else None,
                                  mask_seed=3400 + N)
        if t.block_mask is not None:
            np.fill_diagonal(t.block_mask, 1)
        G.say(f"[case] onepass N={N} {mode} scale={scale}")
        q, k, v, do = (G.to_dev(x, "bf16", dev) for x in (t.q, t.k, t.v, t.do))
        mask = torch.from_numpy(t.block_mask).to(dev) if t.block_mask is not None else None
        o, lse = fa.fwd(q, k, v, scale, causal, mask)
        nan = lambda: torch.full_like(q, float("nan"))
        dq, dk, dv = fa.bwd_onepass(q, k, v, o, lse, do, scale, causal, mask, dq=nan(), dk=nan(), dv=nan())
        rq, rk, rv = fa.bwd(q, k, v, o, lse, do, scale, causal, mask)
        torch.cuda.synchronize()
        for name, x in (("dq", dq), ("dk", dk), ("dv", dv)):
            assert not torch.isnan(x).any().item(), f"{name}: unwritten elements"
        # dV is the same sum of the same bf16 P in the same order; dK may differ by rounding (the
        # two-kernel path forms dS from the bf16 P its waves exchange, this kernel from fp32 P)
        assert torch.equal(dv, rv), "dV differs from flash_attn_bwd"
        G.compare_heads(t, {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}, scale, causal, heads=[(0, 0), (0, 1)])


def test_onepass_backward_long_every_tile(dev):
    """The long-context workload through the one-pass backward, every query tile of every head."""
    import torch

    import exact_io_aware_flash_amd as fa

    w = workloads.WORKLOADS["long"]
    t = workloads.make(w)
    q, k, v, do = (G.to_dev(x, "bf16", dev) for x in (t.q, t.k, t.v, t.do))
    o, lse = fa.fwd(q, k, v, w.scale, True)
    dq, dk, dv = fa.bwd_onepass(q, k, v, o, lse, do, w.scale, True)
    torch.cuda.synchronize()
    res = {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
    G.compare_every_tile(t, res, w.scale, True, seed=45, kv_heads={(0, 3), (0, 30)})


# ------------------------------------------------------------------------------ wave-specialised forward
@pytest.mark.parametrize("causal", [False, True])
def test_pingpong_forward_equals_fwd_and_oracle(dev, causal):
    """The wave-specialised forward computes the same products and sums in the same order as the
    interleaved one: bitwise equal outputs; and both match the oracle (ragged N from one tile to
    several, both signs of the scale)."""
    import torch

    import exact_io_aware_flash_amd as fa

    for N, scale in ((1, 0.09), (65, 0.09), (300, -0.09), (1000, 0.09), (2049, 0.11)):
        G.say(f"[case] pingpong N={N} causal={causal} scale={scale}")
        t = workloads.random_case(2, 2, N, 128, "bf16", seed=2900 + N, with_do=False)
        q, k, v = (G.to_dev(x, "bf16", dev) for x in (t.q, t.k, t.v))
        nan = lambda shape, dt: torch.full(shape, float("nan"), dtype=dt, device=dev)
        o, lse = fa.fwd_pingpong(q, k, v, scale, causal, out=nan(q.shape, q.dtype), lse=nan(q.shape[:3], torch.float32))
        o2, lse2 = fa.fwd(q, k, v, scale, causal)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(lse, lse2), "pingpong differs from flash_attn_fwd"
        G.compare_heads(t, {"o": o, "lse": lse}, scale, causal, heads=[(0, 0), (1, 1)], backward=False)


def test_pingpong_long_sampled(dev):
    import torch

    import exact_io_aware_flash_amd as fa

    w = workloads.WORKLOADS["long"]
    t = workloads.random_case(1, 8, w.N, 128, "bf16", seed=2950, with_do=False)
    q, k, v = (G.to_dev(x, "bf16", dev) for x in (t.q, t.k, t.v))
    o, lse = fa.fwd_pingpong(q, k, v, w.scale, True)
    o2, lse2 = fa.fwd(q, k, v, w.scale, True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    rows = G.sample_rows(w.N, 40, seed=2951)
    G.compare_heads(t, {"o": o, "lse": lse}, w.scale, True, heads=[(0, 0), (0, 7)], backward=False, rows=rows)


# ------------------------------------------------------------------------------ split-key forward
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode", ["dense", "causal", "mask", "causal+mask"])
def test_splitkv_matches_oracle(dev, d, mode):
    """Split-key forward (partials per key range, log-sum-exp merge) against the oracle, for
    split counts below, at and above the number of 128-key blocks."""
    import torch

    import exact_io_aware_flash_amd as fa

    causal = "causal" in mode
    for N, splits in ((1, 1), (127, 3), (300, 2), (300, 5), (1000, 3), (1000, 8)):
        t = workloads.random_case(1, 2, N, d, "bf16", seed=1200 + N + splits,
                                  mask_density=0.6 if "mask" in mode else None, mask_seed=1300 + N)
        if t.block_mask is not None:
            np.fill_diagonal(t.block_mask, 1)
        G.say(f"[case] splitkv N={N} d={d} {mode} splits={splits}")
        q, k, v = (G.to_dev(x, "bf16", dev) for x in (t.q, t.k, t.v))
        mask = torch.from_numpy(t.block_mask).to(dev) if t.block_mask is not None else None
        nan = lambda shape, dt: torch.full(shape, float("nan"), dtype=dt, device=dev)
        o, lse = fa.fwd_splitkv(q, k, v, 1.0 / math.sqrt(d), causal, mask, splits,
                                out=nan(q.shape, q.dtype), lse=nan(q.shape[:3], torch.float32))
        torch.cuda.synchronize()
        assert not torch.isnan(o).any().item() and not torch.isnan(lse).any().item()
        G.compare_heads(t, {"o": o, "lse": lse}, 1.0 / math.sqrt(d), causal, heads=[(0, 0), (0, 1)], backward=False)


def test_splitkv_negative_scale(dev):
    import torch

    import exact_io_aware_flash_amd as fa

    t = workloads.random_case(1, 2, 1000, 128, "bf16", seed=1250, with_do=False)
    q, k, v = (G.to_dev(x, "bf16", dev) for x in (t.q, t.k, t.v))
    for causal in (False, True):
        o, lse = fa.fwd_splitkv(q, k, v, -0.1, causal, None, 3)
        torch.cuda.synchronize()
        G.compare_heads(t, {"o": o, "lse": lse}, -0.1, causal, heads=[(0, 0), (0, 1)], backward=False)


def test_splitkv_long_head_sampled(dev):
    """Few heads and a long causal sequence (the case the split-key form is for): B=1, H=2,
    N=16384, d=128 with 8 key ranges, sampled rows against the oracle."""
    import torch

    import exact_io_aware_flash_amd as fa

    N = 16384
    t = workloads.random_case(1, 2, N, 128, "bf16", seed=1400, with_do=False)
    q, k, v = (G.to_dev(x, "bf16", dev) for x in (t.q, t.k, t.v))
    o, lse = fa.fwd_splitkv(q, k, v, 1.0 / math.sqrt(128), True, None, 8)
    torch.cuda.synchronize()
    rows = G.sample_rows(N, 40, seed=1401)
    G.compare_heads(t, {"o": o, "lse": lse}, 1.0 / math.sqrt(128), True, heads=[(0, 0), (0, 1)], backward=False,
                    rows=rows)


def test_merge_of_oracle_partials(dev):
    """The merge kernel alone: partial results of the oracle over disjoint key ranges (one of them
    empty, so every row has a dead part) combine into the oracle's attention over all keys."""
    import torch

    import exact_io_aware_flash_amd as fa
    import oracle

    N, d = 200, 64
    t = workloads.random_case(1, 1, N, d, "bf16", seed=1500, with_do=False)
    q, k, v = (G._head(t, x, 0, 0) for x in ("q", "k", "v"))
    cuts = [(0, 37), (37, 150), (150, 150), (150, 200)]
    o_parts, l_parts = [], []
    for lo, hi in cuts:
        if hi > lo:
            O, L = oracle.forward_head(q, k[lo:hi], v[lo:hi], 0.125, False, None)
        else:
            O, L = np.zeros((N, d)), np.full(N, -np.inf)
        o_parts.append(O)
        l_parts.append(L)
    op = torch.from_numpy(np.stack(o_parts).astype(np.float32)).to(dev)
    lp = torch.from_numpy(np.stack(l_parts).astype(np.float32)).to(dev)
    o, lse = fa.merge(op, lp)
    torch.cuda.synchronize()
    O, L = oracle.forward_head(q, k, v, 0.125, False, None)
    G.check("merge O", G.host_f64(o), O, G.TOL_BF16, True)
    G.check_lse("merge LSE", lse.cpu().numpy(), L)
    # all parts dead: O = 0, LSE = -inf
    o2, lse2 = fa.merge(torch.zeros_like(op), torch.full_like(lp, float("-inf")))
    torch.cuda.synchronize()
    assert torch.all(o2 == 0) and torch.all(torch.isneginf(lse2))
