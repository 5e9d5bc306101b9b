"""Per-element bounds for comparing the GPU path with the oracle.

The oracle evaluates every dot product in float64 and rounds once; the GPU
accumulates in fp32 on matrix cores.  A GPU result is accepted element by
element when it lies inside an interval derived from the arithmetic:

* a dot product  sum_k a_k w_k  of length K is within
      eps(dtype, K) * sum_k |a_k w_k|
  of the exact value.  eps counts one fp32 rounding (2^-24) per accumulation
  step of the kernel (one per matrix-core instruction, plus the fold of each
  128-wide FP8 scale group, plus the K-split partial sums), doubled, plus the
  instruction's own error: FP8 16x16x128 products are summed inside the
  matrix core below fp32 precision (measured relative L2 3.6e-5 of the sum
  on random codes, i.e. a few 1e-6 of sum |a w|), bounded here by 2^-13;
  bf16 and fp32 instructions by 2^-20 and 2^-22.  sum |a w| is |A| |W|^T.
* a stored bf16 / fp32 value is the correctly rounded image of an fp32
  value within that interval, so it may differ from the oracle's rounding by
  the interval plus one unit in the last place of the stored format.
* Z = SiLU(gate) * up moves by at most |SiLU'(gate)| |up| dg + |SiLU(gate)| du
  (|SiLU'| <= 1.1) when gate and up move by dg and du, plus the few fp32
  ulps of the kernels' hardware exp2 / reciprocal SiLU (2^-19 relative).
* an FP8 Z code is the round-to-nearest-even image of z * (448 / amax) for
  some z within the Z interval and amax within the group's interval, so it
  must lie between the codes of the interval's two ends: equal to the
  oracle's code except where the oracle's value sits within the interval of
  a rounding midpoint (for values much larger than the interval that is one
  e4m3 step; the report gives the largest step count seen).

Each check returns a small report (worst ratio, number of differing codes)
that the tests print."""
from __future__ import annotations

import numpy as np

from oracle import formats as F
from oracle import moe

U = 2.0 ** -24
_K_INST = {"fp8": 128, "bf16": 32, "f32": 4}
_INST_ERR = {"fp8": 2.0 ** -13, "bf16": 2.0 ** -20, "f32": 2.0 ** -22}
SILU_REL = 2.0 ** -19

# every finite e4m3fn value, ascending (+0 and -0 are one value)
_E4M3_VALUES = np.unique(F.e4m3_decode(np.arange(256, dtype=np.uint8))[
    ~np.isnan(F.e4m3_decode(np.arange(256, dtype=np.uint8)))])


def eps(dt: str, K: int) -> float:
    """Relative (to sum |a w|) error bound of one GPU dot product of length K."""
    steps = K // _K_INST[dt] + (K // 128 if dt == "fp8" else 0) + 16
    return _INST_ERR[dt] + 2 * steps * U


def abs_dot(a_vals: np.ndarray, w_vals: np.ndarray) -> np.ndarray:
    """|A| |W|^T in fp32 (a bound: its own rounding is scaled away by 1.01)."""
    return (np.abs(a_vals).astype(np.float32) @ np.abs(w_vals).astype(np.float32).T) * np.float32(1.01)


def ulp_f32(x: np.ndarray) -> np.ndarray:
    return np.spacing(np.abs(np.asarray(x, np.float32))).astype(np.float64)


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (bf16 keeps 16 fewer significand bits)."""
    return ulp_f32(x) * 65536.0


def _report(name, excess, n, extra=None):
    worst = float(np.max(excess)) if excess.size else 0.0
    rep = {"check": name, "elements": int(n), "worst_ratio": worst}
    if extra:
        rep.update(extra)
    return rep


def check_values(got: np.ndarray, ref32: np.ndarray, bound: np.ndarray, fmt: str, name: str) -> dict:
    """got (stored in fmt: 'f32' or 'bf16', given as values) against the
    oracle's fp32 result ref32 and the dot-product bound: assert
    |got - ref32| <= bound + ulp_fmt(|ref32| + bound) element by element."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref32, np.float64)
    assert got.shape == ref.shape == bound.shape, (got.shape, ref.shape, bound.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    ulp = ulp_bf16 if fmt == "bf16" else ulp_f32
    allow = bound + ulp(np.abs(ref) + bound)
    diff = np.abs(got - ref)
    ratio = diff / np.maximum(allow, 1e-300)
    rep = _report(name, ratio, got.size)
    bad = ratio > 1.0
    assert not bad.any(), (f"{name}: {int(bad.sum())} elements outside the bound; first at "
                           f"{np.argwhere(bad)[0].tolist()}: got {got[bad][0]!r} ref {ref[bad][0]!r} "
                           f"allow {allow[bad][0]!r}")
    return rep


def z_interval(g_ref: np.ndarray, g_bound: np.ndarray, I: int):
    """z_ref (fp32, the oracle's SiLU(gate)*up) and the per-element bound on
    a GPU z computed from a G within g_bound of the oracle's."""
    g = np.asarray(g_ref, np.float64)
    gate, up = g[:, :I], g[:, I:]
    dg, du = g_bound[:, :I], g_bound[:, I:]
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-gate))
    silu = gate * s
    z_ref = moe.silu_mul(np.asarray(g_ref, np.float32), I).astype(np.float64)
    tol = 1.1 * (np.abs(up) + du) * dg + np.abs(silu) * du + SILU_REL * np.abs(z_ref) \
        + 4 * ulp_f32(z_ref)
    return z_ref, tol


def check_z(z_got, z_scales_got, z_dt: str, g_ref, g_bound, I: int, name: str) -> dict:
    """The GPU's Z (FP8 codes + scales, bf16 bits, or fp32) against the
    oracle's G and its bound."""
    z_ref, tol = z_interval(g_ref, g_bound, I)
    if z_dt == "f32":
        return check_values(z_got, z_ref.astype(np.float32), tol, "f32", name)
    if z_dt == "bf16":
        return check_values(F.bf16_to_f32(z_got), z_ref.astype(np.float32), tol, "bf16", name)
    n = z_ref.shape[0]
    G = I // 128
    zr = np.abs(z_ref).reshape(n, G, 128)
    tz = tol.reshape(n, G, 128)
    # oracle recipe on z_ref
    codes_ref, sc_ref = F.quant_fp8_groups(z_ref.astype(np.float32))
    amax_ref = np.maximum(zr.max(axis=2), 1e-4)
    tol_amax = tz.max(axis=2)
    # scales: amax moves by at most the largest z bound of its group
    sc_got = np.asarray(z_scales_got, np.float64)
    sc_allow = tol_amax / 448.0 + 2 * ulp_f32(sc_ref)
    sc_ratio = np.abs(sc_got - sc_ref) / sc_allow
    assert np.all(sc_ratio <= 1.0), (f"{name}: {int((sc_ratio > 1).sum())} Z scales outside the bound, "
                                     f"worst ratio {sc_ratio.max():.3g}")
    # codes: v = z * 448/amax; the GPU's v is within tol_v of the oracle's
    inv = (448.0 / amax_ref)[:, :, None]
    v_ref = (z_ref.reshape(n, G, 128)) * inv
    tol_v = tz * inv + np.abs(v_ref) * (tol_amax / amax_ref)[:, :, None] * 1.01 \
        + 2 * ulp_f32(v_ref)
    lo = F.e4m3_decode(F.e4m3_encode(v_ref - tol_v))
    hi = F.e4m3_decode(F.e4m3_encode(v_ref + tol_v))
    got = F.e4m3_decode(np.asarray(z_got, np.uint8)).reshape(n, G, 128)
    out = (got < lo) | (got > hi)
    assert not out.any(), (f"{name}: {int(out.sum())} Z codes outside the rounding interval; first "
                           f"at {np.argwhere(out)[0].tolist()}")
    ref_v = F.e4m3_decode(codes_ref).reshape(n, G, 128)
    diff = got != ref_v
    steps = np.abs(np.searchsorted(_E4M3_VALUES, got) - np.searchsorted(_E4M3_VALUES, ref_v))
    return {"check": name, "elements": int(got.size), "codes_differing": int(diff.sum()),
            "max_code_steps": int(steps.max()) if steps.size else 0,
            "codes_differing_frac": float(diff.mean()),
            "scale_worst_ratio": float(sc_ratio.max()) if sc_ratio.size else 0.0,
            "scales_differing": int((sc_got != sc_ref).sum())}


def maxabs_over_rms(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if not ref.size:
        return 0.0
    rms = np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(got - ref)) / max(rms, 1e-30))


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
