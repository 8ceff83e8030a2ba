"""Pins of the oracle's number formats against things other than the oracle itself:
PyTorch's float8_e4m3fn / bfloat16 casts (a library's implementation of the same
OCP and bfloat16 definitions), literal tables of the formats, and the figures the
pages print (fp4 range 2688, KV latent L2 norm ~22.6)."""
import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def page_figures():
    out = {}
    with open(os.path.join(GOLDEN, "page_figures.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, value = line.split()[:2]
                out[name] = float(value)
    return out


def torch_e4m3_values():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_decode_matches_torch_all_codes():
    ref = torch_e4m3_values()
    got = F.e4m3_value(np.arange(256))
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    m = ~np.isnan(ref)
    assert np.array_equal(got[m], ref[m])
    # sign of zero
    assert np.signbit(got[0x80]) and not np.signbit(got[0x00])


def test_e4m3_literal_values():
    v = F.e4m3_value
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0
    assert v(0x01) == 2.0 ** -9 and v(0x07) == 7 * 2.0 ** -9
    assert v(0x08) == 2.0 ** -6 and v(0x38) == 1.0 and v(0x40) == 2.0
    assert np.isnan(v(0x7F)) and np.isnan(v(0xFF))
    assert np.nanmax(F.E4M3_TABLE) == F.E4M3_MAX == 448.0


def test_e2m1_literal_table():
    # OCP MX E2M1 magnitudes
    assert list(F.E2M1_TABLE[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(F.E2M1_TABLE[8:]) == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    assert np.signbit(F.E2M1_TABLE[8])


def test_fp4_range_is_page_figure():
    figs = page_figures()
    assert F.E2M1_MAX * F.E4M3_MAX == figs["fp4_format_range"] == 2688.0
    # FNUZ E4M3 (max 240) would give 1440, so the page's 2688 fixes the OCP "FN" variant
    assert 6.0 * 240.0 != figs["fp4_format_range"]


def test_kv_width_matches_page_norm():
    figs = page_figures()
    # a unit-RMS latent of width 512 has L2 norm sqrt(512) = 22.63
    assert abs(np.sqrt(512) - figs["kv_latent_l2_norm"]) < 0.05


def test_e4m3_encode_all_bf16_matches_torch_in_range():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = F.bf16_value(bits)
    got = F.e4m3_from_value(x)
    tb = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    ref = tb.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    in_range = np.isfinite(x) & (np.abs(x) < 464.0)
    assert np.array_equal(got[in_range], ref[in_range])
    # NaN inputs -> NaN code
    assert np.all((got[np.isnan(x)] & 0x7F) == 0x7F)
    # beyond the rounding range (and infinities) the oracle saturates to +-448
    big = ~np.isnan(x) & ~in_range
    assert np.all(got[big & (x > 0)] == 0x7E) and np.all(got[big & (x < 0)] == 0xFE)


def test_e4m3_roundtrip_every_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    assert np.array_equal(F.e4m3_from_value(F.e4m3_value(codes)), codes)


def test_e4m3_ties_to_even():
    # 1 + 1/16 lies halfway between 1.0 (code 0x38, even) and 1.125 (0x39)
    assert F.e4m3_from_value(1.0625) == 0x38
    # 1.1875 lies halfway between 1.125 (0x39) and 1.25 (0x3A, even)
    assert F.e4m3_from_value(1.1875) == 0x3A
    # 2^-10 lies halfway between 0 and the smallest subnormal 2^-9
    assert F.e4m3_from_value(2.0 ** -10) == 0x00
    assert F.e4m3_from_value(464.0) == 0x7E   # halfway 448 / 480: even code, 448


def test_e2m1_encode_ties_and_roundtrip():
    cases = {0.25: 0x0, 0.75: 0x2, 1.25: 0x2, 1.75: 0x4, 2.5: 0x4, 3.5: 0x6, 5.0: 0x6,
             7.0: 0x7, 100.0: 0x7, -0.3: 0x9, -5.0: 0xE}
    for x, c in cases.items():
        assert F.e2m1_from_value(x) == c, x
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(F.e2m1_from_value(F.e2m1_value(codes)), codes)


def test_bf16_decode_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = F.bf16_value(bits)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    m = ~np.isnan(ref)
    assert np.array_equal(got[m], ref[m])


def test_kv_row_nibble_order_and_scale_groups():
    codes = np.zeros(256, np.uint8)
    codes[0] = 0x2 | (0x7 << 4)     # channel 0 = 1.0, channel 1 = 6.0
    codes[8] = 0x9 | (0x3 << 4)     # channel 16 = -0.5, channel 17 = 1.5
    codes[255] = 0x5 << 4           # channel 511 = 3.0
    scales = np.full(32, 0x38, np.uint8)  # 1.0
    scales[1] = 0x40                      # channels 16..31 scaled by 2
    scales[31] = 0x30                     # channels 496..511 scaled by 0.5
    v = F.kv_row_values(codes, scales)
    expect = np.zeros(512)
    expect[0], expect[1], expect[16], expect[17], expect[511] = 1.0, 6.0, -1.0, 3.0, 1.5
    assert np.array_equal(v, expect)


def test_fp4_dequant_is_exact_in_bf16():
    # every (E2M1 code, finite E4M3 scale) product is representable in bfloat16
    e2 = F.E2M1_TABLE
    e4 = F.E4M3_TABLE[~np.isnan(F.E4M3_TABLE)]
    prod = (e2[:, None] * e4[None, :]).ravel()
    back = torch.from_numpy(prod).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(back, prod)
    assert np.abs(prod).max() == 2688.0


# ------------------------------------------------------------------ main-KV quantiser

def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """float values that are exact in bf16 -> their bit patterns (checked exact)."""
    b = torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16)
    assert np.array_equal(b.to(torch.float64).numpy(), np.asarray(x, np.float64))
    return b.view(torch.int16).numpy().view(np.uint16)


def test_kv_quantize_roundtrip_of_representable_rows():
    """A row whose every group holds a +-6 code is quantised back to the same bytes: its scale
    is exactly amax / 6 and every value is exactly code x scale (negative zeros included)."""
    rng = np.random.default_rng(5)
    e4 = np.arange(1, 127, dtype=np.uint8)                  # positive finite scales, subnormals too
    for _ in range(20):
        codes16 = rng.integers(0, 16, size=512).astype(np.uint8)
        top = rng.integers(0, 16, size=32) + 16 * np.arange(32)
        codes16[top] = np.where(rng.random(32) < 0.5, 7, 15)
        scales = rng.choice(e4, size=32)
        codes = (codes16[0::2] | (codes16[1::2] << 4)).astype(np.uint8)
        x = F.kv_row_values(codes, scales)
        c2, s2 = F.kv_quantize_rows(_bf16_bits(x))
        assert np.array_equal(s2, scales)
        assert np.array_equal(c2, codes)


def _e2m1_half_step(q: np.ndarray) -> np.ndarray:
    """Half the E2M1 spacing around |q| (q in [0, 6])."""
    a = np.abs(q)
    return np.where(a <= 2.0, 0.25, np.where(a <= 4.0, 0.5, 1.0))


def test_kv_quantize_error_bound_and_nearest_choice():
    """On latent-like rows (unit RMS, as after RMSNorm, with a few large channels), every code
    is a nearest E2M1 value of x / scale (brute force over the 8 magnitudes), the scale is
    amax / 6 within E4M3's relative rounding 2^-4, and |x - dequant| is within half a step of
    the grid (or the saturation gap amax - 6 * scale)."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    x[:, rng.integers(0, 512, 8)] *= 8.0                    # magnitudes up to ~10 and beyond
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    xv = F.bf16_value(bits)
    codes, scales = F.kv_quantize_rows(bits)
    s = F.e4m3_value(scales)                                   # [64, 32]
    g = xv.reshape(64, 32, 16)
    amax = np.abs(g).max(-1)
    assert np.all(np.abs(s - amax / 6) <= amax / 6 * 2.0 ** -4 * (1 + 1e-12))
    deq = F.kv_row_values(codes, scales).reshape(64, 32, 16)
    q = g / s[..., None]
    sat = np.abs(q) > 6.0
    bound = np.where(sat, np.abs(g) - 6 * s[..., None], s[..., None] * _e2m1_half_step(q))
    assert np.all(np.abs(deq - g) <= bound * (1 + 1e-6) + 1e-30)
    # nearest magnitude by brute force (distance to each of the 8 magnitudes)
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    got = np.abs(deq / s[..., None])
    dist = np.abs(np.abs(q)[..., None] - mags)
    assert np.all(np.abs(np.abs(np.minimum(np.abs(q), 6.0)) - got) <= dist.min(-1) + 1e-9)
    assert np.all(np.signbit(deq) == np.signbit(g))


def test_kv_quantize_ties_go_to_even_codes():
    # scale 1 (amax 6): values at the midpoints of the E2M1 grid
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    expect = np.array([0, 2, 2, 4, 4, 6, 6])                # even codes
    row = np.zeros(512, np.float32)
    row[0] = 6.0
    row[1:8] = mids
    row[8:15] = -mids
    codes, scales = F.kv_quantize_rows(_bf16_bits(row))
    c16 = np.stack([codes & 0xF, codes >> 4], -1).reshape(512)
    assert scales[0] == 0x38                                # 1.0
    assert np.array_equal(c16[1:8], expect)
    assert np.array_equal(c16[8:15], expect | 8)


def test_kv_quantize_range_saturation_and_zero_groups():
    figs = page_figures()
    row = np.zeros(512, np.float32)
    row[0] = figs["fp4_format_range"]          # 2688 = 6 x 448: the top of the format
    row[16] = 4096.0                    # beyond it: scale and code saturate
    row[17] = -4096.0
    row[32] = 2.0 ** -12                # amax / 6 rounds to a zero scale byte
    row[48] = -0.0                      # an all-zero group (one negative zero)
    row[64] = 6 * 2.0 ** -9             # the smallest subnormal scale, exactly
    codes, scales = F.kv_quantize_rows(_bf16_bits(row))
    c16 = np.stack([codes & 0xF, codes >> 4], -1).reshape(512)
    deq = F.kv_row_values(codes, scales)
    assert scales[0] == 0x7E and c16[0] == 7 and deq[0] == figs["fp4_format_range"]
    assert scales[1] == 0x7E and c16[16] == 7 and c16[17] == 15 and deq[16] == figs["fp4_format_range"]
    assert scales[2] == 0 and not c16[32:48].any()
    assert scales[3] == 0 and not c16[48:64].any()
    assert scales[4] == 0x01 and c16[64] == 7 and deq[64] == row[64]
