"""Oracle-side number formats -- TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Decoders (and the encoders used to check the step's quantized cache writes) are
written from the format definitions, independently of any other code here:

* bf16: IEEE binary32 with the low 16 bits zero.
* OCP fp8 E4M3: sign | 4-bit exponent (bias 7) | 3-bit mantissa; exponent 0 is
  subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinities.
* OCP MX e2m1: sign | 2-bit exponent (bias 1) | 1-bit mantissa; exponent 0 is
  subnormal (m/2 * 2^0).  E8M0 scale: 2^(e-127), 0xFF is NaN.

The low-precision indexer formats are named by "【论文解读】DeepSeek-V4"
(wkq9411.github.io), section 二(四) "FP4 量化感知训练" (MXFP4 for the indexer QK
path); the pages give no bit layout, so the OCP definitions above are the reading.
Encoders pick the nearest representable value by search over the full value
table, ties to the even code, saturating at the largest finite magnitude.
"""
from __future__ import annotations

import numpy as np


def decode_bf16(bits) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def encode_bf16(x) -> np.ndarray:
    """float64 -> bf16 bits of the nearest bfloat16 value (8 significant bits), ties to the even significand.

    Used where the step stores a float32 result in a bf16 cache: the oracle keeps
    the same storage format, rounding its own float64 value once.
    """
    x = np.asarray(x, dtype=np.float64)
    _, ex = np.frexp(x)                                   # |x| = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex.astype(np.int64) - 1, -126)         # binade; subnormals share the 2^-126 ulp grid
    ulp = np.ldexp(1.0, e - 7)
    v = np.rint(x / ulp) * ulp                             # rint rounds half to even
    return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _fp8_e4m3_table() -> np.ndarray:
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        mt = code & 0x7
        if e == 0xF and mt == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = s * (mt / 8.0) * 2.0 ** (1 - 7)
        else:
            vals[code] = s * (1.0 + mt / 8.0) * 2.0 ** (e - 7)
    return vals


_FP8 = _fp8_e4m3_table()


def fp8_e4m3_values() -> np.ndarray:
    """All 256 code values (NaN for the two NaN codes)."""
    return _FP8.copy()


def decode_fp8_e4m3(codes) -> np.ndarray:
    return _FP8[np.asarray(codes, dtype=np.uint8)]


def _e2m1_table() -> np.ndarray:
    vals = np.empty(16, dtype=np.float64)
    for code in range(16):
        s = -1.0 if code & 0x8 else 1.0
        e = (code >> 1) & 0x3
        mt = code & 0x1
        vals[code] = s * (mt / 2.0) * 2.0 ** (1 - 1) if e == 0 else s * (1.0 + mt / 2.0) * 2.0 ** (e - 1)
    return vals


_E2M1 = _e2m1_table()


def e2m1_values() -> np.ndarray:
    return _E2M1.copy()


def decode_e2m1(codes) -> np.ndarray:
    return _E2M1[np.asarray(codes, dtype=np.uint8) & 0xF]


def decode_e8m0(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    out = np.ldexp(1.0, c - 127).astype(np.float64)
    return np.where(c == 255, np.nan, out)


def decode_mxfp4(packed, scales) -> np.ndarray:
    """packed uint8 [..., n/2] (element 2i low nibble) + E8M0 [..., n/32] -> float64 [..., n]."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = decode_e2m1(p & 0xF)
    hi = decode_e2m1(p >> 4)
    vals = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.float64)
    vals[..., 0::2] = lo
    vals[..., 1::2] = hi
    n = vals.shape[-1]
    sc = decode_e8m0(scales)
    return (vals.reshape(vals.shape[:-1] + (n // 32, 32)) * sc[..., None]).reshape(vals.shape)


def encode_fp8_rope_rows(x: np.ndarray, rope_dims: int):
    """Prepared KV rows [..., c] in the mixed storage the pages give for KV entries ("【论文解读】DeepSeek-V4",
    section 一(三)4, item 1; "DeepseekV4论文解析" on numerical precision): the RoPE dims in bf16, the others
    in fp8.  Returns (bytes [..., c + R] uint8, scale [...]): the first c - R values as e4m3 codes of
    value/scale with scale = amax/448 of those values (as encode_fp8_rows), then the R RoPE values as
    little-endian bf16."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1] - rope_dims
    codes, scale = encode_fp8_rows(x[..., :n])
    bf = np.ascontiguousarray(encode_bf16(x[..., n:])).view(np.uint8)
    return np.concatenate([codes, bf], axis=-1), scale


def decode_fp8_rope_rows(data, scale, rope_dims: int) -> np.ndarray:
    """Exact float64 values of rows stored by encode_fp8_rope_rows (c = bytes - R)."""
    data = np.ascontiguousarray(np.asarray(data, dtype=np.uint8))
    n = data.shape[-1] - 2 * rope_dims
    fp = decode_fp8_e4m3(data[..., :n]) * np.asarray(scale, dtype=np.float32).astype(np.float64)[..., None]
    bf = decode_bf16(np.ascontiguousarray(data[..., n:]).view(np.uint16))
    return np.concatenate([fp, bf], axis=-1)


def dequant_rows(data, scale, fmt: str) -> np.ndarray:
    """Exact float64 values of stored indexer rows."""
    if fmt == "f32":
        return np.asarray(data, dtype=np.float32).astype(np.float64)
    if fmt == "bf16":
        return decode_bf16(data)
    if fmt == "fp8":
        return decode_fp8_e4m3(data) * np.asarray(scale, dtype=np.float32).astype(np.float64)[..., None]
    if fmt == "mxfp4":
        return decode_mxfp4(data, scale)
    raise ValueError(fmt)


def _nearest_code(x: np.ndarray, table: np.ndarray, max_code: int) -> np.ndarray:
    """Nearest non-negative table entry to |x| (codes 0..max_code), ties to the even code."""
    a = np.abs(x)
    vals = table[: max_code + 1]
    d = np.abs(a[..., None] - vals)                  # [..., ncodes]
    best = np.min(d, axis=-1, keepdims=True)
    ties = d == best
    # among tied codes pick an even one (there is at most one tie pair, adjacent codes)
    even = ties & ((np.arange(max_code + 1) % 2) == 0)
    pick = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(ties, axis=-1))
    return pick.astype(np.int64)


def encode_fp8_rows(x: np.ndarray):
    """float64 rows -> (e4m3 codes, scale) with scale = amax/448 and x/scale rounded nearest-even."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.max(np.abs(x), axis=-1)
    scale = amax / 448.0
    safe = np.where(scale > 0, scale, 1.0)
    v = np.clip(x / safe[..., None], -448.0, 448.0)
    mag = _nearest_code(v, _FP8, 0x7E)
    sign = (v < 0) & (mag != 0)
    return (mag | (sign.astype(np.int64) << 7)).astype(np.uint8), scale


def encode_mxfp4(x: np.ndarray):
    """float64 [..., n] -> (packed e2m1 [..., n/2], E8M0 [..., n/32]); X = floor(log2 amax) - 2."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    blk = x.reshape(x.shape[:-1] + (n // 32, 32))
    amax = np.max(np.abs(blk), axis=-1)
    X = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127).astype(np.int64)
    X = np.clip(X, -127, 127)
    v = np.clip(blk / np.ldexp(1.0, X)[..., None], -6.0, 6.0)
    mag = _nearest_code(v, _E2M1, 7)
    sign = (v < 0) & (mag != 0)
    codes = (mag | (sign.astype(np.int64) << 3)).reshape(x.shape)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8), (X + 127).astype(np.uint8)
