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
