"""Pins for the oracle's number formats (CPU only).

The e4m3fn codec and the bf16 rounding are checked against torch's own
casts (``torch.float8_e4m3fn`` / ``torch.bfloat16``), an implementation
independent of the oracle's, exhaustively over every bf16 value and at every
rounding midpoint; the activation recipe is checked against the facts of the
per-token FP8 cast ("DeepEP 架构与实现笔记" §11) and the format's error bound.
"""
import numpy as np
import pytest
import torch

from oracle import formats as F


def _torch_e4m3(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def all_bf16_values():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_to_f32(bits)
    return v[np.isfinite(v)]


def test_e4m3_decode_table_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.all(both_nan | (ours == ref))
    assert np.nanmax(ours) == 448.0 and np.nanmin(ours) == -448.0
    assert ours[1] == 2.0 ** -9 and ours[8] == 2.0 ** -6   # smallest subnormal / normal
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF]) and ours[0x7E] == 448.0


def test_e4m3_encode_every_bf16_value_matches_torch():
    v = all_bf16_values()
    v = v[np.abs(v) <= 464.0]          # beyond the 448/480 midpoint torch returns NaN
    ours = F.e4m3_encode(v)
    ref = _torch_e4m3(v)
    # -0.0 and +0.0: both map to a zero code of the input's sign
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("scale", [1.0, 3.0, 448.0 / 7.3, 0.013, 1e-3, 2.0 ** -7])
def test_e4m3_encode_scaled_values_match_torch(scale):
    with np.errstate(over="ignore"):
        v = all_bf16_values().astype(np.float32) * np.float32(scale)
    v = v[np.abs(v) <= 464.0]
    assert np.array_equal(F.e4m3_encode(v), _torch_e4m3(v))


def test_e4m3_encode_midpoints_ties_to_even():
    # exact midpoints between every pair of adjacent positive codes (0..0x7D),
    # where round-to-nearest-even must pick the even code
    codes = np.arange(0, 0x7E, dtype=np.uint8)
    lo, hi = F.e4m3_decode(codes), F.e4m3_decode(codes + 1)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.all(mid.astype(np.float64) == (lo + hi) / 2)   # representable in fp32
    got = F.e4m3_encode(mid)
    want = np.where(codes % 2 == 0, codes, codes + 1).astype(np.uint8)
    assert np.array_equal(got, want)
    assert np.array_equal(got, _torch_e4m3(mid))
    assert np.array_equal(F.e4m3_encode(-mid), want | 0x80)


def test_e4m3_encode_random_fp32_matches_torch():
    rng = np.random.default_rng(7)
    v = (rng.standard_normal(200_000) * np.exp(rng.uniform(-14, 6, 200_000))).astype(np.float32)
    v = v[np.abs(v) <= 464.0]
    assert np.array_equal(F.e4m3_encode(v), _torch_e4m3(v))


def test_e4m3_encode_saturates():
    assert F.e4m3_encode(np.array([449.0, 470.0, 1e6, -1e6])).tolist() == [0x7E, 0x7E, 0x7E, 0xFE]


def test_bf16_rounding_matches_torch_on_random_and_edges():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(100_000).astype(np.float32) * np.float32(1e3),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 3.4e38, 1e-40, np.inf, -np.inf],
                 np.float32)])
    # ties: exactly halfway between two bf16 values
    base = F.bf16_to_f32(rng.integers(0, 0x7F00, 1000).astype(np.uint16))
    ties = (base.view(np.uint32) + np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.f32_to_bf16(x), ref)
    assert np.isnan(F.bf16_to_f32(F.f32_to_bf16(np.array([np.nan], np.float32))))[0]


def test_quant_recipe_facts():
    # a group whose amax is 448 has scale 1 and encodes its values exactly
    row = np.zeros((1, 128), np.float32)
    row[0, :4] = [448.0, -2.0, 0.5, 2.0 ** -9]
    codes, scales = F.quant_fp8_groups(row)
    assert scales[0, 0] == np.float32(1.0)
    assert np.array_equal(F.e4m3_decode(codes[0, :4]), [448.0, -2.0, 0.5, 2.0 ** -9])
    # amax is clamped at 1e-4: an all-zero group gets scale 1e-4/448 and zero codes
    codes, scales = F.quant_fp8_groups(np.zeros((2, 256), np.float32))
    assert np.all(codes == 0)
    assert np.all(scales == np.float32(np.float32(1e-4) / np.float32(448.0)))
    # each group of 128 gets its own scale; the group's max maps to +-448
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 384)).astype(np.float32)
    x[:, 128:256] *= 100
    codes, scales = F.quant_fp8_groups(x)
    assert scales.shape == (5, 3)
    amax = np.abs(x.reshape(5, 3, 128)).max(axis=2)
    assert np.allclose(scales, amax / 448.0, rtol=1e-7)
    top = np.abs(F.e4m3_decode(codes)).reshape(5, 3, 128).max(axis=2)
    assert np.all(top == 448.0)


def test_quant_roundtrip_within_format_error_bound():
    # e4m3 keeps 3 mantissa bits: relative rounding error <= 2^-4 in the normal
    # range; below it the absolute error is <= half a subnormal step * scale
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((64, 512)) * rng.uniform(0.01, 50, (64, 1))).astype(np.float32)
    codes, scales = F.quant_fp8_groups(x)
    back = F.dequant_fp8_groups(codes, scales)
    s = np.repeat(scales.astype(np.float64), 128, axis=1)
    err = np.abs(back - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(err <= bound)


def test_quant_matches_torch_cast_recipe():
    # the recipe written with torch ops in fp32 (amax, 448/amax, product, cast)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((32, 768)).astype(np.float32) * np.float32(3)
    codes, scales = F.quant_fp8_groups(x)
    t = torch.from_numpy(x).view(32, 6, 128)
    amax = t.abs().amax(dim=2).clamp(min=1e-4)
    # 448/amax as the IEEE fp32 quotient (float64 division rounded once to
    # fp32); torch's CPU scalar/tensor division is not correctly rounded
    inv = (448.0 / amax.double()).float()
    ref_codes = (t * inv[:, :, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(codes, ref_codes.reshape(32, 768).numpy())
    assert np.array_equal(scales, (amax / 448.0).numpy())


def test_quant_tie_case_uses_ieee_quotient():
    # a group with amax 2.875 and an element -1.078125: 448/2.875 rounds to the
    # fp32 value whose product with -1.078125 is exactly -168.0, halfway
    # between e4m3 codes 160 and 176, so ties-to-even gives -160
    g = np.zeros((1, 128), np.float32)
    g[0, 0], g[0, 1] = 2.875, -1.078125
    inv = np.float32(448.0) / np.float32(2.875)
    assert np.float32(-1.078125) * inv == np.float32(-168.0)
    codes, _ = F.quant_fp8_groups(g)
    assert F.e4m3_decode(codes[0, 1:2])[0] == -160.0


def test_block_dequant_layout():
    # one scale per 128x128 (out, in) block
    codes = np.full((256, 384), 0x38, np.uint8)          # 0x38 encodes 1.0
    sc = np.arange(6, dtype=np.float32).reshape(2, 3) + 1
    v = F.dequant_fp8_blocks(codes, sc)
    assert F.e4m3_decode(np.array([0x38]))[0] == 1.0
    assert v[0, 0] == 1 and v[0, 128] == 2 and v[0, 383] == 3 and v[128, 0] == 4 and v[255, 383] == 6
