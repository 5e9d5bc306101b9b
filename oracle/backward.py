"""Backward of the MoE path, computed plainly on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages cited (by title):
  [XT]  "XTuner Domino EP": the DeepEP part's complete run path (the backward
        consumes the saved handle, counts and routing permutation in reverse
        order), and the UltraEP part's backward sketch (combine backward, the
        grouped GEMMs' data and weight gradients, inverse permutation).
  [EP]  "SGLang、NCCL 与 MoE EP" §1.1 (y = sum_k w * expert_out, weights on
        outputs), whose derivative this is.

The pages fix the order of the steps, not their formulas; the formulas are
the derivatives of the forward definition in ``moe``:

  y[t]      = sum_{k local} w[t,k] * out[q(t,k)]
  out[q]    = Z[q] W2[e]^T,   Z = SiLU(gate) * up,   [gate | up] = G = A W13[e]^T
  A[q]      = x[t(q)]

so, for an upstream gradient dy [T, H]:

  d_out[q]  = w[t,k] * dy[t]                         (combine backward, a dispatch)
  d_w[t,k]  = <dy[t], out[q]>                        (router-weight gradient)
  dZ[q]     = d_out[q] W2[e]                         (data gradient of the down GEMM)
  d_up      = dZ * SiLU(gate)
  d_gate    = dZ * up * s * (1 + gate * (1 - s)),    s = sigmoid(gate)
  dA[q]     = [d_gate | d_up] W13[e]                 (data gradient of the gate/up GEMM)
  dx[t]     = sum_{k local} dA[q(t,k)]               (permute backward, an unweighted combine)
  dW2[e]    = sum_{q of e} d_out[q]^T Z[q]            (weight gradient of the down GEMM)
  dW13[e]   = sum_{q of e} [d_gate | d_up][q]^T A[q]  (weight gradient of the gate/up GEMM)

Readings:
  * one GPU's share: routes with no local row contribute nothing here, so
    their d_w is 0 and a token without a local route gets dx = 0;
  * dot products in float64 rounded once to fp32; elementwise steps in fp32;
    sums over routes in fp32 in k order (as the forward combine);
  * every gradient that the next step consumes is rounded to the storage
    format of the configuration (bf16 or fp32) before it is consumed, as the
    GPU path stores it;
  * G is the forward's fp32 G (the GPU path recomputes it with the gate/up GEMM);
  * weight gradients reduce over the expert's valid rows in float64 and are
    rounded once to fp32; an expert without rows gets zeros.
"""
from __future__ import annotations

import numpy as np

from . import formats as F
from .moe import buffer_values, dispatch_layout, gemm_w13, permute, silu, valid_rows


def to_format(v: np.ndarray, dt: str) -> np.ndarray:
    """Gradient values rounded to their storage format (bf16 RNE or fp32), as fp32."""
    return F.round_bf16(v) if dt == "bf16" else np.asarray(v, np.float32)


def combine_backward(dy: np.ndarray, out_rows: dict, slot_of: np.ndarray, weights: np.ndarray,
                     d_out_dt: str):
    """d_out[q] = w[t,k] * dy[t] for every local route (one fp32 product,
    rounded to d_out_dt); d_w[t,k] = <dy[t], out[q]> in float64, rounded to
    fp32, and 0 for routes without a local row.  ``out_rows`` maps row q to
    the forward's expert output (values of its storage format)."""
    T, K = slot_of.shape
    d_out = {}
    d_w = np.zeros((T, K), np.float32)
    for t in range(T):
        for k in range(K):
            q = int(slot_of[t, k])
            if q < 0:
                continue
            d_out[q] = to_format((np.float32(weights[t, k]) * dy[t]).astype(np.float32), d_out_dt)
            d_w[t, k] = np.float32(np.dot(dy[t].astype(np.float64), out_rows[q].astype(np.float64)))
    return d_out, d_w


def silu_mul_backward(g: np.ndarray, dz: np.ndarray) -> np.ndarray:
    """[d_gate | d_up] for Z = SiLU(gate) * up, in fp32.  g [m, 2I] is the
    forward's G, dz [m, I] the gradient of Z."""
    g = np.asarray(g, np.float32)
    dz = np.asarray(dz, np.float32)
    I = dz.shape[1]
    gate, up = g[:, :I], g[:, I:]
    with np.errstate(over="ignore"):
        s = (np.float32(1.0) / (np.float32(1.0) + np.exp(-gate))).astype(np.float32)
    d_up = (dz * silu(gate)).astype(np.float32)
    d_gate = (dz * up * s * (np.float32(1.0) + gate * (np.float32(1.0) - s))).astype(np.float32)
    return np.concatenate([d_gate, d_up], axis=1).astype(np.float32)


def permute_backward(d_rows: dict, slot_of: np.ndarray, H: int, dx_dt: str) -> np.ndarray:
    """dx[t] = sum over local routes k (increasing) of d_rows[q(t,k)], fp32,
    rounded to dx_dt; 0 for a token without a local route."""
    T, K = slot_of.shape
    dx = np.zeros((T, H), np.float32)
    for t in range(T):
        acc = np.zeros(H, np.float32)
        for k in range(K):
            q = int(slot_of[t, k])
            if q >= 0:
                acc = (acc + d_rows[q]).astype(np.float32)
        dx[t] = acc
    return to_format(dx, dx_dt)


def wgrad(b_rows: np.ndarray, a_rows: np.ndarray, N: int, K: int) -> np.ndarray:
    """C = B^T A over one expert's rows: B [m, N], A [m, K] -> [N, K], float64
    products rounded once to fp32 (zeros for m = 0)."""
    if len(b_rows) == 0:
        return np.zeros((N, K), np.float32)
    return (np.asarray(b_rows, np.float64).T @ np.asarray(a_rows, np.float64)).astype(np.float32)


def layer_backward(wl, dy: np.ndarray, ew) -> dict:
    """The whole backward for a workload (bf16 or fp32 weights): forward
    quantities recomputed by the forward oracle's own steps, then the steps
    above in the order the path runs them.  ``dy`` [T, H] fp32 values of the
    output format.  Returns every intermediate by row."""
    cfg = wl.cfg
    gdt = "bf16" if cfg.out_dt == "bf16" else "f32"        # storage format of the gradients
    lay = dispatch_layout(wl.ids, cfg.E, cfg.expert_begin, cfg.L, cfg.R)
    slot_of, counts, offsets = lay["slot_of"], lay["counts"], lay["offsets"]
    rows = valid_rows(counts, offsets)
    perm = permute(wl.x, cfg.act, lay["row_src"], cfg.K, cfg.buf_dt, rows)
    a_vals = buffer_values(perm["data"], cfg.buf_dt, perm.get("scales"))
    a_by = {int(q): a_vals[i] for i, q in enumerate(perm["rows"])}
    e_of = {int(q): int(np.searchsorted(offsets, q, side="right") - 1) for q in rows}
    # forward quantities per row
    from .moe import expert_mlp_rows
    fwd = expert_mlp_rows(cfg, a_by, e_of, ew)
    d_out, d_w = combine_backward(dy, fwd["out"], slot_of, wl.weights, gdt)
    dz, dg, da = {}, {}, {}
    dw2 = np.zeros((cfg.L, cfg.H, cfg.I), np.float32)
    dw13 = np.zeros((cfg.L, 2 * cfg.I, cfg.H), np.float32)
    by_e: dict[int, list] = {}
    for q, e in e_of.items():
        by_e.setdefault(e, []).append(q)
    for e, qs in sorted(by_e.items()):
        qs = sorted(qs)
        do = np.stack([d_out[q] for q in qs]).astype(np.float64)
        dz_e = to_format((do @ ew.w2(e)).astype(np.float32), gdt)
        g_e = np.stack([fwd["G"][q] for q in qs])
        dg_e = to_format(silu_mul_backward(g_e, dz_e), gdt)
        da_e = to_format((dg_e.astype(np.float64) @ ew.w13(e)).astype(np.float32), gdt)
        z_e = buffer_values(np.stack([fwd["Z"][q] for q in qs]), cfg.z_dt,
                            np.stack([fwd["Zs"][q] for q in qs]) if fwd["Zs"] else None)
        dw2[e] = wgrad(do, z_e, cfg.H, cfg.I)
        dw13[e] = wgrad(dg_e, np.stack([a_by[q] for q in qs]), 2 * cfg.I, cfg.H)
        for i, q in enumerate(qs):
            dz[q], dg[q], da[q] = dz_e[i], dg_e[i], da_e[i]
    dx = permute_backward(da, slot_of, cfg.H, gdt)
    return {"layout": lay, "rows": rows, "fwd": fwd, "d_out": d_out, "d_w": d_w, "dz": dz,
            "dg": dg, "da": da, "dx": dx, "e_of": e_of, "dw2": dw2, "dw13": dw13}


def gemm_w13_rows(a_by: dict, e_of: dict, ew) -> dict:
    """G rows of the forward (for tests that feed the GPU the oracle's G)."""
    out = {}
    by_e: dict[int, list] = {}
    for q, e in e_of.items():
        by_e.setdefault(e, []).append(q)
    for e, qs in sorted(by_e.items()):
        qs = sorted(qs)
        g = gemm_w13(np.stack([a_by[q] for q in qs]), ew.w13(e))
        for i, q in enumerate(qs):
            out[q] = g[i]
    return out
