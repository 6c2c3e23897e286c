"""MX-FP8 quantisation on the host: E4M3 elements with one power-of-two (E8M0) scale per block of
32 consecutive elements, as the OCP Microscaling Formats (MX) specification v1.0 defines them
(section 5, "MX-compliant formats", and section 6.3, "Conversion from vectors of scalar floats").
Test infrastructure (see the package header): it supplies the quantised inputs of the FP8
forward's oracle and the expected codes of the device quantiser.

The pages name FP8 attention (FlashAttention-3 reaching about 1.2 PFLOP/s in FP8, "How
FlashAttention Bypasses the GPU Memory Bottleneck to Enable Long-Context AI") but fix no format;
the reading taken is OCP MXFP8 with E4M3 elements, the block-scaled FP8 format gfx950's matrix
cores multiply natively.

E4M3 (the OCP "FN" variant): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent
field 0 holds the subnormals m/8 * 2^-6; the code S.1111.111 is NaN; there are no infinities;
the largest finite magnitude is 1.75 * 2^8 = 448.  E8M0: an unsigned biased exponent, value
2^(e - 127), 0xFF = NaN.

Conversion of a block V_1..V_32 (spec 6.3): shared_exp = floor(log2(max_i |V_i|)) - emax_elem,
with emax_elem = 8 for E4M3 (the exponent of its largest normal); X = 2^shared_exp; each element
is V_i / X rounded to nearest, ties to even, and clamped to +-448.  A block of zeros takes the
smallest scale.  The scale exponent is held to [-127, 127].
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E4M3_MAX = 448.0
EMAX_ELEM = 8
NAN_CODE = 0x7F


def e4m3_decode(codes) -> np.ndarray:
    """float64 values of E4M3 codes (uint8); NaN for S.1111.111."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    field = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(field.astype(np.float64) - 7.0)
    sub = m / 8.0 * 2.0 ** -6
    v = sign * np.where(field == 0, sub, normal)
    return np.where((c & 0x7F) == NAN_CODE, np.nan, v)


def e4m3_encode(x) -> np.ndarray:
    """E4M3 codes (uint8) of float values: round to nearest, ties to even, clamp to +-448."""
    x = np.asarray(x, dtype=np.float64)
    sign = (np.signbit(x)).astype(np.int64) << 7
    a = np.abs(x)
    # normal range: a = (1 + f) 2^e, e >= -6; round f to 3 bits (np.rint is ties-to-even)
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64)
    e = np.maximum(e, -6)
    frac = a / np.exp2(e.astype(np.float64))  # in [1, 2) for normals, [0, 1) below 2^-6
    is_sub = a < 2.0 ** -6
    m_norm = np.rint((frac - 1.0) * 8.0).astype(np.int64)
    e_n = e + (m_norm == 8)
    m_norm = np.where(m_norm == 8, 0, m_norm)
    code_norm = ((e_n + 7) << 3) | m_norm
    # subnormals: a / 2^-9 rounded to an integer 0..8 (8 is the smallest normal, code 0x08)
    code_sub = np.rint(a * 2.0 ** 9).astype(np.int64)
    code = np.where(is_sub, code_sub, code_norm)
    code = np.where(a > E4M3_MAX, 0x7E, code)       # saturate
    code = np.where(code > 0x7E, 0x7E, code)        # rounding up past 448 also saturates
    code = np.where(np.isnan(x), NAN_CODE, code | sign)
    return code.astype(np.uint8)


def scale_exponent(amax) -> np.ndarray:
    """Shared exponent of blocks with largest magnitude amax (int64, in [-127, 127])."""
    amax = np.asarray(amax, dtype=np.float64)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 2.0 ** -200))).astype(np.int64) - EMAX_ELEM
    return np.clip(e, -127, 127)


def quantize(x, axis: int = -1):
    """MX-FP8 quantisation of x in blocks of 32 along `axis` (its length a multiple of 32, or
    padded with zeros to one).  Returns (codes uint8, same shape as x; scale bytes uint8, the
    block axis shortened 32-fold) with scale byte = shared exponent + 127."""
    x = np.moveaxis(np.asarray(x, dtype=np.float64), axis, -1)
    n = x.shape[-1]
    nb = (n + BLOCK - 1) // BLOCK
    pad = nb * BLOCK - n
    xp = np.concatenate([x, np.zeros(x.shape[:-1] + (pad,))], axis=-1) if pad else x
    blocks = xp.reshape(x.shape[:-1] + (nb, BLOCK))
    e = scale_exponent(np.abs(blocks).max(axis=-1))
    codes = e4m3_encode(blocks / np.exp2(e.astype(np.float64))[..., None])
    codes = codes.reshape(x.shape[:-1] + (nb * BLOCK,))[..., :n]
    return np.moveaxis(codes, -1, axis), np.moveaxis((e + 127).astype(np.uint8), -1, axis)


def dequantize(codes, scales, axis: int = -1) -> np.ndarray:
    """float64 values of MX-FP8 data quantised along `axis`."""
    c = np.moveaxis(np.asarray(codes), axis, -1)
    s = np.moveaxis(np.asarray(scales), axis, -1)
    n = c.shape[-1]
    scale = np.exp2(s.astype(np.float64) - 127.0)
    scale = np.repeat(scale, BLOCK, axis=-1)[..., :n]
    return np.moveaxis(e4m3_decode(c) * scale, -1, axis)
