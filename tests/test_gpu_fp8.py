"""GPU parity of the MX-FP8 path, through the C ABI.

* Device quantisation (flash_attn_mxfp8_quantize_rows / _vt) against oracle/mx.py: bit-exact
  codes and scale bytes (integer work).
* The FP8 forward against the fp64 oracle evaluated on the dequantised inputs (the exact
  attention of what the kernel is given).  Tolerance per O element: the bound on the rounding
  of P to E4M3 (oracle.p_rounding_bound: sum_j max(2^-4 p_j, 2^-10) |v_j| / sum_j p_j), plus
  half a bf16 ulp of the value (the output's own rounding), plus 1e-4 for fp32 accumulation.
  LSE: 1e-3 (the row sums use P in fp32).
"""
import numpy as np
import pytest

import workloads
from oracle import mx
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return G.device()


def _bf16_dev(bits, dev):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def _quantize_all(t, dev):
    import exact_io_aware_flash_amd as fa

    q, k, v = (_bf16_dev(getattr(t, n), dev) for n in ("q", "k", "v"))
    return fa.mxfp8_quantize(q), fa.mxfp8_quantize(k), fa.mxfp8_quantize(v, transposed=True)


def _vt_scales_natural(sc, N):
    """device V^T scales [Np/32, 32, d/32] (key block, feature % 32, feature / 32) -> [nkb, d]"""
    nkb = sc.shape[0]
    d = sc.shape[1] * sc.shape[2]
    return np.ascontiguousarray(sc.transpose(0, 2, 1)).reshape(nkb, d)[: (N + 31) // 32]


def _check_head_quantisation(t, Q8, K8, V8, b, h):
    """device codes and scales of head (b, h) equal the host quantiser's; returns the
    dequantised q, k, v (fp64) the oracle works on"""
    N = t.q.shape[2]
    out = []
    for name, X in (("q", Q8), ("k", K8)):
        codes, scales = mx.quantize(t.as_f64(name)[b, h], axis=-1)
        dc, ds = X.codes[b, h].cpu().numpy(), X.scales[b, h].cpu().numpy()
        assert np.array_equal(dc, codes), f"{name} codes differ at {np.argwhere(dc != codes)[:4].tolist()}"
        assert np.array_equal(ds, scales), f"{name} scales differ at {np.argwhere(ds != scales)[:4].tolist()}"
        out.append(mx.dequantize(codes, scales, axis=-1))
    vc, vs = mx.quantize(t.as_f64("v")[b, h], axis=0)
    dct = V8.codes[b, h].cpu().numpy()
    assert np.array_equal(dct[:, :N].T, vc), "V^T codes differ"
    assert not dct[:, N:].any(), "V^T padding columns must be zero"
    ds = _vt_scales_natural(V8.scales[b, h].cpu().numpy(), N)
    assert np.array_equal(ds, vs), f"V^T scales differ at {np.argwhere(ds != vs)[:4].tolist()}"
    out.append(mx.dequantize(vc, vs, axis=0))
    return out


def _fp8_case(name, t, scale, causal, dev, heads, rows=None):
    import torch

    import exact_io_aware_flash_amd as fa
    import oracle

    B, H, N, d = t.q.shape
    G.say(f"[case] fp8 {name}: shape={t.q.shape} causal={causal} mask={'yes' if t.block_mask is not None else 'no'}")
    Q8, K8, V8 = _quantize_all(t, dev)
    mask = torch.from_numpy(t.block_mask).to(dev) if t.block_mask is not None else None
    o = torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    fa.fwd_mxfp8(Q8, K8, V8, scale, causal, mask, out=o, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any().item() and not torch.isnan(lse).any().item(), "unwritten outputs"
    worst = 0.0
    for (b, h) in heads:
        qd, kd, vd = _check_head_quantisation(t, Q8, K8, V8, b, h)
        r = np.arange(N) if rows is None else np.asarray(rows)
        O, L = oracle.forward_head(qd, kd, vd, scale, causal, t.block_mask, rows=r)
        bound = oracle.p_rounding_bound(qd, kd, vd, scale, causal, t.block_mask, rows=r)
        got = G.host_f64(o[b, h][r])
        err = np.abs(got - O)
        lim = bound + G.bf16_half_ulp(O) * (O != 0) + 1e-4
        ratio = float((err / lim).max()) if err.size else 0.0
        worst = max(worst, ratio)
        G.say(f"  O[{b},{h}]: max|err| {err.max():.3e}  max bound {bound.max():.3e}  max err/limit {ratio:.3f}  "
              f"mean|err| {err.mean():.2e}")
        bad = ~(err <= lim)
        if bad.any():
            i = np.unravel_index(np.argmax(np.where(bad, err / lim, -1)), err.shape)
            raise AssertionError(f"O[{b},{h}]: {int(bad.sum())} elements beyond the bound; worst at row {r[i[0]]} "
                                 f"feature {i[1]}: got {got[i]} ref {O[i]} limit {lim[i]:.3e}")
        G.check_lse(f"LSE[{b},{h}]", lse[b, h][r].cpu().numpy(), L)
    return worst


def _blocks_with_exponents(shape, seed):
    """bf16 bit patterns [..., d] whose 32-element blocks span the whole bf16 range (each block
    N(0,1) times 2^s, s from -133 to 126), plus crafted blocks: zeros, one nonzero, signed zeros,
    E4M3 ties (normal and subnormal) at scale 1, and a block whose scaled maximum exceeds 448."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape)
    nblk = x.size // 32
    xb = x.reshape(nblk, 32)
    s = rng.integers(-133, 127, size=nblk)
    xb *= np.exp2(s.astype(np.float64))[:, None]
    special = [
        np.zeros(32),
        np.r_[np.zeros(31), 3.0],
        np.r_[-0.0, 0.0, -0.0, np.zeros(28), 1.0],
        # amax 256 -> scale 2^0: ties between neighbouring codes resolve to the even code
        np.r_[256.0, 1.0625, 1.1875, -1.0625, -1.1875, 2.0 ** -10, 3 * 2.0 ** -10, -(2.0 ** -10), 5 * 2.0 ** -10,
              17.0, 19.0, 36.0, 232.0, 248.0, np.full(18, 0.5)],
        # amax 1.9 * 2^8 -> scale 2^0, scaled value 486.4 clamps to 448; 464 and 470 too
        np.r_[486.4, 464.0, 470.0, -480.0, 440.0, 444.0, np.full(26, 7.0)],
        np.r_[2.0 ** -133, 2.0 ** -134, np.zeros(30)],  # bf16 subnormals only
    ]
    for i, blk in enumerate(special):
        xb[i * 7 % nblk] = blk
    bits = workloads.round_to_bf16_bits(xb.reshape(shape).astype(np.float32))
    return bits


@pytest.mark.parametrize("d", [64, 128])
def test_quantize_rows_bit_exact(dev, d):
    import exact_io_aware_flash_amd as fa

    shape = (1, 2, 96, d)
    bits = _blocks_with_exponents(shape, 40 + d)
    G.say(f"[case] quantize rows d={d}")
    X = fa.mxfp8_quantize(_bf16_dev(bits, dev))
    xf = workloads.bf16_bits_to_f32(bits).astype(np.float64)
    codes, scales = mx.quantize(xf, axis=-1)
    dc, ds = X.codes.cpu().numpy(), X.scales.cpu().numpy()
    assert np.array_equal(ds, scales), f"scales differ at {np.argwhere(ds != scales)[:4].tolist()}"
    diff = np.argwhere(dc != codes)
    assert diff.size == 0, f"codes differ at {diff[:4].tolist()}: {[(hex(dc[tuple(i)]), hex(codes[tuple(i)])) for i in diff[:4]]}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 200, 256])
def test_quantize_vt_bit_exact(dev, d, N):
    import exact_io_aware_flash_amd as fa

    bits = _blocks_with_exponents((1, 2, N, d), 50 + N + d) if N >= 32 else workloads.gaussian((1, 2, N, d), 7, 1,
                                                                                                 "bf16")[0]
    G.say(f"[case] quantize V^T d={d} N={N}")
    V8 = fa.mxfp8_quantize(_bf16_dev(bits, dev), transposed=True)
    vf = workloads.bf16_bits_to_f32(bits).astype(np.float64)
    npad = fa.mxfp8_vt_cols(N)
    assert V8.codes.shape == (1, 2, d, npad)
    for h in range(2):
        vc, vs = mx.quantize(vf[0, h], axis=0)
        dct = V8.codes[0, h].cpu().numpy()
        assert np.array_equal(dct[:, :N].T, vc)
        assert not dct[:, N:].any()
        sc = V8.scales[0, h].cpu().numpy()
        assert np.array_equal(_vt_scales_natural(sc, N), vs)
        # key blocks wholly past N are zero blocks: scale byte 0 (2^-127)
        assert not _vt_scales_natural(sc, npad)[(N + 31) // 32:].any()


CASES = [
    # name, B, H, N, d, causal, mask density
    ("dense ragged", 1, 2, 200, 64, False, None),
    ("causal ragged", 1, 2, 333, 128, True, None),
    ("dense tiles", 2, 1, 640, 128, False, None),
    ("causal tiles", 1, 2, 512, 64, True, None),
    ("sparse", 1, 2, 700, 128, False, 0.5),
    ("sparse causal", 1, 1, 900, 64, True, 0.6),
    ("one key", 1, 1, 1, 128, False, None),
    ("tail in first tile", 1, 1, 65, 64, True, None),
]


@pytest.mark.parametrize("name,B,H,N,d,causal,dens", CASES, ids=[c[0] for c in CASES])
def test_fwd_mxfp8_matches_oracle(dev, name, B, H, N, d, causal, dens):
    t = workloads.random_case(B, H, N, d, "bf16", seed=3000 + N + d, with_do=False, mask_density=dens,
                              mask_seed=77)
    heads = [(b, h) for b in range(B) for h in range(H)]
    worst = _fp8_case(name, t, 1.0 / np.sqrt(d), causal, dev, heads)
    assert worst <= 1.0


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_mxfp8_negative_scale(dev, causal):
    # a negative scale flips the sign of the Q codes (exact in E4M3)
    t = workloads.random_case(1, 2, 700, 128, "bf16", seed=3050, with_do=False)
    worst = _fp8_case("negative scale", t, -1.0 / np.sqrt(128), causal, dev, [(0, 0), (0, 1)])
    assert worst <= 1.0


def test_fwd_mxfp8_dead_rows(dev):
    # a block mask with an empty block row (non-causal): those queries see no key
    t = workloads.random_case(1, 2, 384, 64, "bf16", seed=3101, with_do=False)
    t.block_mask = np.ones((3, 3), dtype=np.uint8)
    t.block_mask[1, :] = 0
    _fp8_case("dead rows", t, 0.125, False, dev, [(0, 0), (0, 1)])


def test_fwd_mxfp8_long_sampled(dev):
    # the long-context shape (N = 16384, d = 128, causal) on 8 heads: B*H a multiple of 8 takes the
    # XCD remap and, with 128 query tiles per head, the head-major order; sampled rows of 2 heads
    t = workloads.random_case(1, 8, 16384, 128, "bf16", seed=1004, with_do=False)
    rows = G.sample_rows(16384, 48, seed=9)
    _fp8_case("long sampled", t, 1.0 / np.sqrt(128), True, dev, [(0, 0), (0, 7)], rows=rows)


def test_fwd_mxfp8_remapped_grid(dev):
    # B*H = 16 (remapped grid, level order), d = 64, non-causal, every row compared on 2 heads
    t = workloads.random_case(2, 8, 1024, 64, "bf16", seed=3201, with_do=False)
    _fp8_case("remapped grid", t, 0.125, False, dev, [(0, 3), (1, 6)])


@pytest.mark.parametrize("i", range(16))
def test_fwd_mxfp8_random_shape(dev, i):
    # seeded random shapes: B, H, ragged N, d, causal flag, a random block mask and a scale of
    # either sign, every head against the oracle within the P-rounding bound
    rng = np.random.default_rng(5000 + i)
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    N = int(rng.choice([int(rng.integers(1, 64)), int(rng.integers(64, 300)), int(rng.integers(300, 700))]))
    d = int(rng.choice([64, 128]))
    causal, masked = bool(rng.random() < 0.5), bool(rng.random() < 0.4)
    scale = float(rng.uniform(0.3, 1.5)) / np.sqrt(d) * (1 if rng.random() < 0.5 else -1)
    t = workloads.random_case(B, H, N, d, "bf16", seed=5100 + i, with_do=False,
                              mask_density=0.5 if masked else None, mask_seed=5200 + i)
    if t.block_mask is not None:
        np.fill_diagonal(t.block_mask, 1)  # every query block keeps at least its own keys
    worst = _fp8_case(f"random {i}: N={N} d={d} scale={scale:.4f}", t, scale, causal, dev,
                      [(b, h) for b in range(B) for h in range(H)])
    assert worst <= 1.0
