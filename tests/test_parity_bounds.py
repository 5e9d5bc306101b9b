"""CPU checks of the per-element comparison rules the GPU parity tests use
(tests/parity_bounds.py): results inside the arithmetic's error bounds pass,
and the mistakes a kernel could plausibly make -- a wrong row, a dropped
K group, a code two e4m3 steps off, a code one step off away from a rounding
midpoint, a wrong group scale -- fail.  The planted mistakes are made here,
on the CPU, from the oracle's own results."""
import numpy as np
import pytest

import parity_bounds as PB
from oracle import formats as F
from oracle import moe


def _fp8_operands(rng, n, N, K):
    a = rng.standard_normal((n, K)).astype(np.float32)
    codes, sc = F.quant_fp8_groups(a)
    a_vals = F.dequant_fp8_groups(codes, sc)
    w = (rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)
    wc, ws = F.quant_fp8_groups(w)          # per-row groups: any exact fp8 weights will do
    w_vals = F.dequant_fp8_groups(wc, ws)
    return a_vals, w_vals


@pytest.fixture(scope="module")
def case():
    rng = np.random.default_rng(11)
    n, I, K = 48, 256, 1024
    a, w13 = _fp8_operands(rng, n, 2 * I, K)
    g_ref = moe.gemm_w13(a, w13)
    bound = PB.eps("fp8", K) * PB.abs_dot(a, w13)
    # a GPU-like result: the exact dot products moved by up to half the bound
    g_gpu = (g_ref + rng.uniform(-0.5, 0.5, g_ref.shape) * bound).astype(np.float32)
    return dict(rng=rng, n=n, I=I, K=K, a=a, w13=w13, g_ref=g_ref, bound=bound, g_gpu=g_gpu)


def test_eps_is_far_below_a_plausible_mistake(case):
    # one dropped 128-wide K group changes a dot product by |P_g|, about
    # sqrt(128) typical products; the bound is ~1e-4 of sum |a w|
    assert PB.eps("fp8", 7168) < 2e-4
    assert PB.eps("bf16", 4096) < 2e-5
    assert PB.eps("f32", 1024) < 5e-5


def test_g_within_bound_passes_and_mistakes_fail(case):
    c = case
    rep = PB.check_values(c["g_gpu"], c["g_ref"], c["bound"], "f32", "G")
    assert rep["worst_ratio"] <= 1.0
    # a row computed from another row's activations
    bad = c["g_gpu"].copy()
    bad[3] = moe.gemm_w13(c["a"][4:5], c["w13"])[0]
    with pytest.raises(AssertionError):
        PB.check_values(bad, c["g_ref"], c["bound"], "f32", "G")
    # one K group of 128 left out of one element's sum
    bad = c["g_gpu"].copy()
    bad[7, 11] -= float(c["a"][7, 256:384] @ c["w13"][11, 256:384])
    with pytest.raises(AssertionError):
        PB.check_values(bad, c["g_ref"], c["bound"], "f32", "G")


def _gpu_like_z(g_gpu, I):
    z = moe.silu_mul(g_gpu, I)
    return F.quant_fp8_groups(z)


def test_fp8_z_from_a_g_within_bound_passes(case):
    c = case
    codes, scales = _gpu_like_z(c["g_gpu"], c["I"])
    rep = PB.check_z(codes, scales, "fp8", c["g_ref"], c["bound"], c["I"], "Z")
    assert rep["codes_differing"] >= 0
    # the oracle's own Z passes with zero differing codes
    rc, rs = _gpu_like_z(c["g_ref"], c["I"])
    rep = PB.check_z(rc, rs, "fp8", c["g_ref"], c["bound"], c["I"], "Z")
    assert rep["codes_differing"] == 0


def _step(code, k):
    """The e4m3 code k steps up (k > 0) or down from `code` by value."""
    vals = PB._E4M3_VALUES
    i = int(np.searchsorted(vals, F.e4m3_decode(np.uint8(code))))
    return F.e4m3_encode(np.array([vals[i + k]]))[0]


def test_fp8_z_planted_mistakes_fail(case):
    c = case
    I = c["I"]
    codes, scales = _gpu_like_z(c["g_ref"], I)
    z_ref, tol = PB.z_interval(c["g_ref"], c["bound"], I)
    # far from any rounding midpoint: pick an element whose v sits near a code
    amax = np.maximum(np.abs(z_ref).reshape(len(z_ref), -1, 128).max(axis=2), 1e-4)
    v = z_ref / np.repeat(amax, 128, axis=1) * 448.0
    near = np.abs(v - F.e4m3_decode(F.e4m3_encode(v))) < 1e-3 * np.maximum(np.abs(v), 1)
    near &= np.abs(v) > 1.0
    r, col = np.argwhere(near)[0]
    for k in (1, 2, -2):
        bad = codes.copy()
        bad[r, col] = _step(bad[r, col], k)
        with pytest.raises(AssertionError):
            PB.check_z(bad, scales, "fp8", c["g_ref"], c["bound"], I, "Z")
    # a group scale off by 5 % (an amax taken over part of the group)
    bad_s = scales.copy()
    bad_s[2, 1] *= np.float32(1.05)
    with pytest.raises(AssertionError):
        PB.check_z(codes, bad_s, "fp8", c["g_ref"], c["bound"], I, "Z")
    # the scale of the neighbouring group
    bad_s = scales.copy()
    bad_s[5, 0] = scales[5, 1]
    with pytest.raises(AssertionError):
        PB.check_z(codes, bad_s, "fp8", c["g_ref"], c["bound"], I, "Z")


def test_bf16_values_rounding_and_mistakes(case):
    c = case
    rng = c["rng"]
    ref = c["g_ref"][:, :64]
    bound = c["bound"][:, :64]
    got = F.round_bf16((ref + rng.uniform(-1, 1, ref.shape) * bound).astype(np.float32))
    PB.check_values(got, ref, bound, "bf16", "out")
    bad = got.copy()
    bad[1, 2] = F.round_bf16(np.array([ref[1, 2] * 1.02 + 1e-3], np.float32))[0]
    with pytest.raises(AssertionError):
        PB.check_values(bad, ref, bound, "bf16", "out")


def test_bf16_and_f32_z(case):
    c = case
    I = c["I"]
    z = moe.silu_mul(c["g_gpu"], I)
    PB.check_z(F.f32_to_bf16(z), None, "bf16", c["g_ref"], c["bound"], I, "Z bf16")
    PB.check_z(z, None, "f32", c["g_ref"], c["bound"], I, "Z f32")
    bad = z.copy()
    bad[0, :] = z[1, :]
    with pytest.raises(AssertionError):
        PB.check_z(bad, None, "f32", c["g_ref"], c["bound"], I, "Z f32")
