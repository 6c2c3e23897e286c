"""Pins of the host MX-FP8 quantiser (oracle/mx.py) to the OCP Microscaling Formats v1.0
definitions: the E4M3 code table, round-to-nearest-even by brute force over every finite code,
saturation, the shared-exponent rule and the resulting error bound."""
import numpy as np
import pytest

from oracle import mx

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_e4m3_code_table():
    # values fixed by the format: bias 7, 3 mantissa bits, subnormals m/8 * 2^-6, S.1111.111 NaN
    want = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 / 8 * 2.0 ** -6, 0x08: 2.0 ** -6, 0x38: 1.0, 0x39: 1.125,
            0x3C: 1.5, 0x40: 2.0, 0x7E: 448.0, 0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0, 0x77: 240.0, 0x78: 256.0}
    for c, v in want.items():
        assert mx.e4m3_decode(np.uint8(c)) == v, hex(c)
    assert np.isnan(mx.e4m3_decode(np.uint8(0x7F))) and np.isnan(mx.e4m3_decode(np.uint8(0xFF)))
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    v = mx.e4m3_decode(finite)
    assert np.nanmax(np.abs(v)) == 448.0 and len(np.unique(np.abs(v))) == 127


def test_e4m3_round_trip():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(mx.e4m3_encode(mx.e4m3_decode(codes)), codes)


def _brute_force_encode(x):
    """Nearest finite E4M3 value by search over the whole code table, ties to the even code,
    magnitudes past the largest finite value clamped to it."""
    pos = np.arange(0, 0x7F, dtype=np.uint8)  # 0x00 .. 0x7E: every non-negative finite code
    vals = mx.e4m3_decode(pos)
    out = []
    for xv in np.asarray(x, dtype=np.float64).ravel():
        a = min(abs(xv), 448.0)
        d = np.abs(vals - a)
        best = np.flatnonzero(d == d.min())
        c = int(pos[best[0]]) if len(best) == 1 else int(pos[[b for b in best if pos[b] % 2 == 0][0]])
        out.append(c | (0x80 if np.signbit(xv) else 0))
    return np.array(out, dtype=np.uint8)


def test_e4m3_encode_is_nearest_even_by_brute_force():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(3000) * np.exp2(rng.integers(-12, 10, 3000)),
        mx.e4m3_decode(np.arange(0, 0x7E, dtype=np.uint8)) * 1.0625,      # exact ties in the normal range
        (np.arange(1, 16) + 0.5) * 2.0 ** -10,                              # ties among subnormals
        np.array([448.0, 460.0, 464.0, 479.9, 1e6, -1e6, 2.0 ** -11, -2.0 ** -11, 0.0]),
    ])
    assert np.array_equal(mx.e4m3_encode(x), _brute_force_encode(x))


def test_shared_exponent_and_block_layout():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((5, 96)) * np.exp2(rng.integers(-20, 20, (5, 1)))
    codes, scales = mx.quantize(x, axis=-1)
    assert codes.shape == x.shape and scales.shape == (5, 3)
    amax = np.abs(x.reshape(5, 3, 32)).max(-1)
    assert np.array_equal(scales.astype(np.int64) - 127, np.floor(np.log2(amax)).astype(np.int64) - 8)
    # the largest element of every block lands in [256, 448] (its binade is 2^8, then clamped)
    top = np.abs(mx.e4m3_decode(codes)).reshape(5, 3, 32).max(-1)
    assert np.all((top >= 256) & (top <= 448))
    # axis handling: blocks along axis 0 are the transposed blocks along the last axis
    c0, s0 = mx.quantize(x.T, axis=0)
    assert np.array_equal(c0, codes.T) and np.array_equal(s0, scales.T)


def test_dequantised_error_bound_and_zero_blocks():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((64, 128))
    codes, scales = mx.quantize(x)
    deq = mx.dequantize(codes, scales)
    X = np.repeat(np.exp2(scales.astype(np.float64) - 127), 32, axis=-1)
    scaled = np.abs(x) / X
    inside = scaled <= 448
    err = np.abs(deq - x)
    assert np.all(err[inside] <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * X)[inside] + 1e-300)
    assert np.all(np.abs(deq[~inside]) == 448 * X[~inside])
    z, zs = mx.quantize(np.zeros((2, 64)))
    assert np.all(z == 0) and np.all(zs == 0)


def _head(seed, N=48, d=8):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((N, d)), rng.standard_normal((N, d)), rng.standard_normal((N, d))


@pytest.mark.parametrize("causal", [False, True])
def test_p_rounding_bound_is_attained_by_worst_perturbation(causal):
    # the bound is the triangle inequality: the perturbation p'_j = p_j + sign(v_jf) max(2^-4 p_j,
    # 2^-10) reaches it exactly for feature f, and random admissible perturbations stay inside
    import oracle
    q, k, v = _head(11)
    scale = 0.7
    rows = np.arange(q.shape[0])
    bound = oracle.p_rounding_bound(q, k, v, scale, causal)
    O, _ = oracle.forward_head(q, k, v, scale, causal)
    S = scale * (q @ k.T)
    vis = oracle.visible(rows, rows, causal, None)
    S = np.where(vis, S, -np.inf)
    p = np.where(vis, np.exp(S - S.max(axis=1, keepdims=True)), 0.0)
    err = np.where(vis, np.maximum(2.0 ** -4 * p, 2.0 ** -10), 0.0)
    for f in range(v.shape[1]):
        pw = p + err * np.sign(v[:, f])[None, :]
        got = (pw @ v[:, f]) / p.sum(axis=1)
        assert np.allclose(np.abs(got - O[:, f]), bound[:, f], rtol=1e-12, atol=1e-15)
    rng = np.random.default_rng(5)
    for _ in range(20):
        pw = p + err * rng.uniform(-1, 1, p.shape)
        dev = np.abs((pw @ v) / p.sum(axis=1, keepdims=True) - O)
        assert np.all(dev <= bound * (1 + 1e-12) + 1e-15)


@pytest.mark.parametrize("c", [1.0, 3.7, 2.0 ** 8])
def test_p_rounding_bound_covers_e4m3_rounding_of_p(c):
    # P held as c p (1 <= c <= 2^8, so every value stays <= 448) and rounded to E4M3 in the
    # numerator: the error stays within the bound, and uses a fair part of it (not vacuous)
    import oracle
    q, k, v = _head(12, N=200, d=16)
    scale = 1.3
    bound = oracle.p_rounding_bound(q, k, v, scale, True)
    O, _ = oracle.forward_head(q, k, v, scale, True)
    P = oracle.probabilities(q, k, scale, True)
    p = P / P.max(axis=1, keepdims=True)
    pq = mx.e4m3_decode(mx.e4m3_encode(c * p)) / c
    got = (pq @ v) / p.sum(axis=1, keepdims=True)
    dev = np.abs(got - O)
    assert np.all(dev <= bound * (1 + 1e-12))
    assert dev.max() > 0.05 * bound.max()
