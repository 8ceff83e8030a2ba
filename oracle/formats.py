"""Cache number formats, decoded and encoded from their definitions in float64.

TEST INFRASTRUCTURE.  This package is the CPU oracle of the CSA2 hot path.  Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the library never does.

Formats (DeepSeek-V4.1-Flash pages: blog.4sapi.com section 5 "FP4 KV", and the
animattoys.com section on the FP4 main KV cache):

* E4M3 -- the OCP 8-bit float "E4M3FN": 1 sign bit, 4 exponent bits (bias 7),
  3 mantissa bits; exponent field 0 is subnormal, S.1111.111 is NaN, there is
  no infinity, the largest finite magnitude is 448.  The FP4 section states the
  format's range as 2688, which is 6 (E2M1 max) x 448, so the OCP "FN" variant
  (and not the FNUZ variant, max 240) is meant.
* E2M1 -- FP4: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; magnitudes
  {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* Main-KV row: 512 channels, E2M1 codes two per byte (channel 2i in the low
  nibble of byte i, channel 2i+1 in the high nibble), one E4M3 scale per 16
  channels (scale byte g covers channels 16g..16g+15), no second-level scale.
  The nibble order and the separate scale array are readings of ours: the pages
  give neither.
* bf16 -- the upper 16 bits of an IEEE binary32.

Encoders round to nearest, ties to the code with an even mantissa (which is the
even code), and saturate to the largest finite magnitude.

Main-KV quantisation (the producer of the cache; blog.4sapi.com section 5 and the
animattoys.com FP4 section give the format and that it is applied to the rotated
latent, not the rule for choosing a scale).  The reading taken here, per group of 16
channels of a bf16 row:
  amax  = max |x_c|;
  scale = E4M3(amax / 6), the quotient rounded to binary32 first (6 = the largest E2M1
          magnitude, so amax maps to the top of the FP4 range);
  code_c = E2M1(x_c / scale), the quotient rounded to binary32 first, ties to even,
          saturating at +-6, sign kept (-0 gives the negative-zero code);
  a group whose scale byte is 0 (amax / 6 rounds to zero) stores code 0 everywhere.
Both quotients are IEEE binary32 divisions, the precision in which the GPU kernel takes
the same integer decisions.  Parity: pinned by the round trip of exactly representable
rows, the error bound of the two roundings, the pages' range 2688 = 6 x 448 and the
special cases in tests/test_oracle_formats.py.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0


def _e4m3_table() -> np.ndarray:
    t = np.empty(256, np.float64)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 0xF, c & 0x7
        if e == 0xF and m == 0x7:
            v = np.nan
        elif e == 0:
            v = (m / 8.0) * 2.0 ** -6
        else:
            v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
        t[c] = -v if s else v
    return t


def _e2m1_table() -> np.ndarray:
    t = np.empty(16, np.float64)
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 0x3, c & 0x1
        v = (m / 2.0) if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1)
        t[c] = -v if s else v
    return t


E4M3_TABLE = _e4m3_table()
E2M1_TABLE = _e2m1_table()


def e4m3_value(codes) -> np.ndarray:
    """E4M3 bytes -> float64 values (NaN for 0x7F / 0xFF)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e2m1_value(nibbles) -> np.ndarray:
    """E2M1 4-bit codes (0..15) -> float64 values."""
    return E2M1_TABLE[np.asarray(nibbles, dtype=np.uint8) & 0xF]


def _round_to_codes(x, pos_values: np.ndarray, sign_bit: int, max_code: int) -> np.ndarray:
    """Nearest non-negative code for |x|, ties to the even code, saturating at max_code;
    the sign bit is set for negative inputs (and for -0)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    neg = np.signbit(x)
    hi = np.searchsorted(pos_values, a, side="left")        # first value >= a
    hi = np.minimum(hi, max_code)
    lo = np.maximum(hi - 1, 0)
    dlo = a - pos_values[lo]
    dhi = pos_values[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= pos_values[max_code], max_code, code)
    code = code.astype(np.uint8) | np.where(neg, sign_bit, 0).astype(np.uint8)
    return code


def e4m3_from_value(x) -> np.ndarray:
    """float64 -> E4M3 bytes: round to nearest even, saturate to +-448, NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    pos = E4M3_TABLE[:127]                       # codes 0..126: 0 .. 448, ascending
    code = _round_to_codes(np.nan_to_num(x, nan=0.0), pos, 0x80, 126)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def e2m1_from_value(x) -> np.ndarray:
    """float64 -> E2M1 nibble codes: round to nearest even, saturate to +-6."""
    pos = E2M1_TABLE[:8]
    return _round_to_codes(x, pos, 0x8, 7)


def bf16_value(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def kv_row_values(codes, scales) -> np.ndarray:
    """Main-KV rows -> float64 [..., 512].

    codes  [..., 256] uint8: two E2M1 codes per byte, even channel in the low nibble.
    scales [..., 32]  uint8: E4M3, scale g multiplies channels 16g .. 16g+15.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    lo = e2m1_value(codes & 0xF)
    hi = e2m1_value(codes >> 4)
    v = np.stack([lo, hi], axis=-1).reshape(codes.shape[:-1] + (2 * codes.shape[-1],))
    s = np.repeat(e4m3_value(scales), 16, axis=-1)
    return v * s


def kv_quantize_rows(x_bf16) -> "tuple[np.ndarray, np.ndarray]":
    """Rotated bf16 latent rows [..., 512] (uint16 bits) -> (codes [..., 256] uint8,
    scales [..., 32] uint8), by the reading in the module docstring."""
    bits = np.asarray(x_bf16, dtype=np.uint16)
    assert bits.shape[-1] == 512
    x = (bits.astype(np.uint32) << 16).view(np.float32)             # exact bf16 values
    g = x.reshape(bits.shape[:-1] + (32, 16))
    amax = np.max(np.abs(g), axis=-1)                                # exact
    s32 = (amax / np.float32(6.0)).astype(np.float32)               # binary32 division
    scales = e4m3_from_value(s32.astype(np.float64))
    sval = e4m3_value(scales).astype(np.float32)                     # exact in binary32
    safe = np.where(sval > 0, sval, np.float32(1.0))[..., None]
    q = (g / safe).astype(np.float32)                                # binary32 division
    codes16 = e2m1_from_value(q.astype(np.float64))
    codes16 = np.where((sval > 0)[..., None], codes16, np.uint8(0)).astype(np.uint8)
    c = codes16.reshape(bits.shape[:-1] + (512,))
    codes = (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
    return codes, scales
