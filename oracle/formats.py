"""Number formats used on the path, written from their definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* bf16: the upper 16 bits of an IEEE binary32; narrowing rounds to nearest,
  ties to even.
* OCP FP8 E4M3 ("e4m3fn", the ``float8_e4m3fn`` type the FP8 cast of
  "DeepEP 架构与实现笔记" §11 produces): 1 sign bit, 4 exponent bits with bias
  7, 3 mantissa bits, no infinities, only S.1111.111 is NaN, so the largest
  finite magnitude is 1.75 * 2^8 = 448.  Exponent field 0 holds subnormals
  m * 2^-9.  Narrowing rounds to nearest, ties to even; this codec saturates
  magnitudes beyond 448 to 448 (the activation recipe never produces them).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


# ---------------------------------------------------------------- bf16

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32, exact."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (NaN stays NaN)."""
    x = np.ascontiguousarray(x, np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> 16).astype(np.uint16) | np.uint16(0x0040))
    return r


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 value rounded to the nearest bf16, returned as fp32."""
    return bf16_to_f32(f32_to_bf16(x))


# ---------------------------------------------------------------- e4m3fn

def _e4m3_value(c: int) -> float:
    """Value of one e4m3fn code, from the field definitions."""
    sign = -1.0 if c & 0x80 else 1.0
    ex, man = (c >> 3) & 0xF, c & 0x7
    if ex == 15 and man == 7:
        return float("nan")
    if ex == 0:
        return sign * man * 2.0 ** -9
    return sign * (1.0 + man / 8.0) * 2.0 ** (ex - 7)


_E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], np.float64)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """e4m3fn codes (uint8) -> exact values as float64 (table of all 256 codes)."""
    return _E4M3_TABLE[np.asarray(codes, np.uint8)]


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """fp32 (or fp64) values -> e4m3fn codes, round to nearest even, saturating.

    For |v| >= 2^-6 with 2^e <= |v| < 2^(e+1) the representable neighbours are
    spaced 2^(e-3); below 2^-6 they are the subnormals spaced 2^-9.  Dividing
    by that spacing is exact in float64, so ``rint`` (ties to even) gives the
    rounded significand n directly, and the code is (e+7)*8 + (n-8) in the
    normal range (a carry n == 16 lands on the next binade by itself) or n
    in the subnormal range (n == 8 is the smallest normal's code)."""
    v = np.asarray(x, np.float64)
    a = np.abs(v)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)
    out = np.zeros(v.shape, np.int64)
    sub = a < 2.0 ** -6
    out[sub] = np.rint(a[sub] / 2.0 ** -9).astype(np.int64)
    nrm = ~sub
    if nrm.any():
        an = a[nrm]
        e = np.floor(np.log2(an)).astype(np.int64)
        # guard log2 rounding at exact powers of two
        e = np.where(np.exp2(e.astype(np.float64)) > an, e - 1, e)
        e = np.where(np.exp2(e + 1.0) <= an, e + 1, e)
        n = np.rint(an / np.exp2(e - 3.0)).astype(np.int64)
        code = (e + 7) * 8 + (n - 8)
        out[nrm] = np.minimum(code, 0x7E)        # saturate at 448
    out = np.where(np.isnan(v), 0x7F, out)
    return (out | sign).astype(np.uint8)


# ---------------------------------------------------------------- activation quantisation

def quant_fp8_groups(x: np.ndarray, group: int = 128):
    """Per-row, per-128-column FP8 quantisation of activations.

    Follows the per-token FP8 cast of "DeepEP 架构与实现笔记" §11: for each row
    and each group of 128 consecutive columns, amax = max|x| clamped below at
    1e-4; values are multiplied by 448/amax and cast to e4m3fn; the fp32 scale
    is amax/448.  Reading: amax, the factor 448/amax and the product are fp32
    (each a single IEEE fp32 operation), as the page states the scale is FP32.

    Returns (codes uint8 [n, C], scales fp32 [n, C/128])."""
    x = np.ascontiguousarray(x, np.float32)
    n, c = x.shape
    assert c % group == 0
    blocks = x.reshape(n, c // group, group)
    amax = np.maximum(np.abs(blocks).max(axis=2), np.float32(1e-4)).astype(np.float32)
    inv = (np.float32(448.0) / amax).astype(np.float32)
    prod = (blocks * inv[:, :, None]).astype(np.float32)
    codes = e4m3_encode(prod).reshape(n, c)
    scales = (amax / np.float32(448.0)).astype(np.float32)
    return codes, scales


def dequant_fp8_groups(codes: np.ndarray, scales: np.ndarray, group: int = 128) -> np.ndarray:
    """codes [n, C] with scales [n, C/128] -> exact float64 values."""
    n, c = codes.shape
    v = e4m3_decode(codes).reshape(n, c // group, group)
    return (v * scales.astype(np.float64)[:, :, None]).reshape(n, c)


def dequant_fp8_blocks(codes: np.ndarray, scales: np.ndarray, blk: int = 128) -> np.ndarray:
    """Weight codes [N, K] with per-128x128-block scales [N/128, K/128] ->
    exact float64 values ("SGLang Expert Compute Backend" §3.5: one weight
    scale per 128x128 (N, K) block)."""
    n, k = codes.shape
    v = e4m3_decode(codes).reshape(n // blk, blk, k // blk, blk)
    return (v * scales.astype(np.float64)[:, None, :, None]).reshape(n, k)
