"""Storage encoders for synthetic inputs: bf16, fp8 e4m3 with a per-row scale, MXFP4.

These only produce input bits; decoding and all arithmetic on them live on each
side separately (the oracle decodes from the format definitions, the HIP path in
hardware).  Formats:

* bf16: the top 16 bits of an IEEE binary32, round-to-nearest-even.
* fp8 e4m3 (OCP 8-bit floating point, "E4M3"): 1 sign, 4 exponent (bias 7),
  3 mantissa bits; no infinities; 0x7F / 0xFF are NaN; max finite 448.
  Row-scaled storage: scale = amax(row) / 448 (fp32), code = e4m3(x / scale)
  with round-to-nearest-even and saturation to +-448.
* MXFP4 (OCP Microscaling v1.0): blocks of 32 e2m1 elements (1 sign, 2 exponent
  with bias 1, 1 mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6) sharing one E8M0
  scale 2^(e-127).  Shared exponent = floor(log2(amax)) - 2; elements are
  x / 2^X rounded to nearest even and saturated to +-6.  Two elements per
  byte, element 2i in the low nibble.
"""
from __future__ import annotations

import numpy as np

FP8_MAX = 448.0


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest-even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _e4m3_encode_abs(a: np.ndarray) -> np.ndarray:
    """|value| (float64, already within [0, inf)) -> 7-bit magnitude code, RNE, saturating."""
    a = np.minimum(a, FP8_MAX)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormals: multiples of 2^-9
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)
    nrm = ~sub
    mant, ex = np.frexp(a[nrm])          # a = mant * 2^ex, mant in [0.5, 1)
    e = ex - 1                            # a = (2*mant) * 2^e, 2*mant in [1, 2)
    q = np.rint((2.0 * mant - 1.0) * 8.0).astype(np.int64)
    carry = q == 8
    q[carry] = 0
    e = e + carry
    c = ((e + 7) << 3) | q
    code[nrm] = np.minimum(c, 0x7E)
    return code


def fp8_e4m3_encode(v: np.ndarray) -> np.ndarray:
    """float32 values (already scaled) -> uint8 e4m3 codes."""
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    mag = _e4m3_encode_abs(np.abs(v))
    sign = (np.signbit(v) & (mag != 0)).astype(np.int64) << 7
    return (mag | sign).astype(np.uint8)


def fp8_rowscale_encode(x: np.ndarray):
    """Quantize rows (last axis) to e4m3 with scale = amax/448.  Returns (codes uint8, scale float32)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / np.float32(FP8_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = (x / safe[..., None]).astype(np.float32)
    return fp8_e4m3_encode(q), scale


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """float64 values (already divided by the block scale) -> 4-bit codes, RNE, saturating at 6."""
    a = np.abs(v)
    code = ((a > 0.25).astype(np.int64) + (a >= 0.75) + (a > 1.25) + (a >= 1.75)
            + (a > 2.5) + (a >= 3.5) + (a > 5.0))
    sign = (np.signbit(v) & (code != 0)).astype(np.int64) << 3
    return (code | sign).astype(np.uint8)


def mxfp4_encode(x: np.ndarray):
    """Quantize the last axis (a multiple of 32) to MXFP4.

    Returns (packed uint8 [..., n/2], e8m0 scales uint8 [..., n/32]).
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    n = x.shape[-1]
    assert n % 32 == 0
    blk = x.reshape(x.shape[:-1] + (n // 32, 32))
    amax = np.max(np.abs(blk), axis=-1)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    X = np.where(amax > 0, ex - 1 - 2, -127)       # floor(log2 amax) - emax(e2m1)
    X = np.clip(X, -127, 127)
    codes = e2m1_encode(np.ldexp(blk, -X[..., None]))
    codes = codes.reshape(x.shape)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, (X + 127).astype(np.uint8)
