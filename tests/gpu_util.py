"""Helpers for the GPU parity tests: moving seeded inputs to the device,
building a layer, comparing against the oracle."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def announce(*parts):
    """Print and flush what names the case before any GPU work."""
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, kind: str | None = None) -> torch.Tensor:
    """numpy -> device tensor; bf16 bit patterns become torch.bfloat16."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if kind == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    """device tensor -> numpy with bf16 as uint16 bits, fp8 as uint8."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def host_vals(t: torch.Tensor) -> np.ndarray:
    """device tensor -> numpy float32 values (bf16 decoded exactly)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.float().numpy()
    return t.numpy()


def layer_shape(cfg, BM=128):
    from combine_top_expert_amd.pipeline import LayerShape
    return LayerShape(T=cfg.T, K=cfg.K, E=cfg.E, expert_begin=cfg.expert_begin, L=cfg.L,
                      H=cfg.H, I=cfg.I, R=cfg.R, act=cfg.act, wdt=cfg.wdt, BM=BM)


def upload_weights(layer, wl):
    cfg = wl.cfg
    kind = "bf16" if cfg.wdt == "bf16" else None
    w13 = dev(wl.w["w13"], kind)
    w2 = dev(wl.w["w2"], kind)
    s13 = dev(wl.w["w13_scales"]) if cfg.wdt == "fp8" else None
    s2 = dev(wl.w["w2_scales"]) if cfg.wdt == "fp8" else None
    layer.set_weights(w13, w2, s13, s2)


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))


def maxabs_rel(got, ref) -> float:
    """max |got - ref| / max |ref|: the L-infinity counterpart of rel_l2."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if not ref.size:
        return 0.0
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def maxabs_over_rms(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    return float(np.max(np.abs(got - ref)) / max(rms, 1e-30)) if ref.size else 0.0


# Layer output bars (the layer's rel-L2 bar and the max-abs bar "after
# normalisation", read as max|dy| / RMS(y_ref)):
#  * rel-L2 of y against the oracle's y: <= 2e-2;
#  * max|dy| / RMS against the oracle's y: <= max(5e-2, 3 x floor), where
#    floor is the same figure between two evaluations of the oracle that
#    differ only in fp32 vs float64 dot products, measured on the same
#    tokens.  The figure is set by roundings, not by arithmetic error: one
#    bf16 unit of the largest outputs is 2^-8..2^-7 of a value several times
#    the RMS, and a G difference of a few fp32 ulps moves an FP8 Z code by a
#    whole step at a rounding midpoint, which reaches every output of its
#    row.  The full prefill shape's floor is 4.9e-2 (one bf16 unit at the
#    largest output); the GPU, whose FP8 matrix cores sum each 128-product
#    group below fp32 precision, reaches two units there.
# The arithmetic itself is checked element by element upstream: every G, Z
# and expert-output element within its bound (parity_bounds) and combine
# bit-exact on the GPU's expert outputs, so y is the correctly computed
# combine of correctly computed rows.
LAYER_REL_L2 = 2e-2
LAYER_MAXABS = 5e-2
FLOOR_FACTOR = 3.0


def check_layer(wl, layer, tokens=None, ew=None, stages=True, tag="", g=None):
    """The GPU layer (already run; its buffers still hold the pass) against
    the oracle: layout, every Z element against the oracle's G (FP8 codes
    and scales within the rounding interval), every expert-output element
    against the oracle's down GEMM on the GPU's Z, combine bit-exact on the
    GPU's expert outputs, and the layer bars above (max|dy|/RMS against the
    oracle run on the GPU's own Z is printed as well).  ``g``: a device G
    [rows_cap, 2I] from the same GEMM with the stored-G epilogue, checked
    element by element as well (the unfused layer's own G is used when
    present).  Returns the metrics."""
    import parity_bounds as PB
    from oracle import moe

    cfg = wl.cfg
    ew = ew or moe.ExpertWeights(cfg, wl.w)
    ref = moe.moe_layer(wl, tokens=tokens, ew=ew)
    sel = ref["tokens"]
    slot_of = ref["layout"]["slot_of"]
    if cfg.routing != "given":
        assert np.array_equal(layer.slot_of.cpu().numpy(), slot_of), "slot_of differs"
    rows = np.asarray(ref["perm"]["rows"], np.int64)
    offs, cnts = ref["layout"]["offsets"], ref["layout"]["counts"]
    e_of = np.searchsorted(offs, rows, side="right") - 1
    z_gpu = host_bits(layer.z)[rows]
    zs_gpu = layer.z_scales.cpu().numpy()[rows] if layer.z_scales is not None else None
    out_gpu = host_vals(layer.out)[rows]
    y_gpu = host_vals(layer.y)[sel]
    zv_gpu = moe.buffer_values(z_gpu, cfg.z_dt, zs_gpu)
    a_vals = moe.buffer_values(ref["perm"]["data"], cfg.buf_dt, ref["perm"].get("scales"))
    if g is None:
        g = getattr(layer, "g", None)
    g_gpu = g.cpu().numpy()[rows] if g is not None else None
    out_cond = {}
    rep = {"z": [], "out": [], "g": []}
    for e in np.unique(e_of):
        idx = np.nonzero(e_of == e)[0]
        w13, w2 = ew.w13(int(e)), ew.w2(int(e))
        o = moe.out_to_format(moe.gemm_w2(zv_gpu[idx], w2), cfg.out_dt)
        for j, q in enumerate(rows[idx]):
            out_cond[int(q)] = o[j]
        if stages:
            g_ref = np.stack([ref["mlp"]["G"][int(q)] for q in rows[idx]])
            g_bound = PB.eps(cfg.wdt, cfg.H) * PB.abs_dot(a_vals[idx], w13)
            if g_gpu is not None:
                rep["g"].append(PB.check_values(g_gpu[idx], g_ref, g_bound, "f32", f"G e{e}"))
            rep["z"].append(PB.check_z(z_gpu[idx], None if zs_gpu is None else zs_gpu[idx], cfg.z_dt,
                                       g_ref, g_bound, cfg.I, f"Z e{e}"))
            o_bound = PB.eps(cfg.wdt, cfg.I) * PB.abs_dot(zv_gpu[idx], w2)
            ref32 = moe.gemm_w2(zv_gpu[idx], w2)
            rep["out"].append(PB.check_values(out_gpu[idx], ref32, o_bound, cfg.out_dt, f"out e{e}"))
    # combine on the GPU's own expert outputs is bit-exact
    out_rows = {int(q): out_gpu[i] for i, q in enumerate(rows)}
    y_comb = moe.combine(out_rows, slot_of, wl.weights, cfg.out_dt, tokens=sel)
    assert np.array_equal(y_gpu, y_comb), "combine of the GPU's expert outputs differs"
    y_cond = moe.combine(out_cond, slot_of, wl.weights, cfg.out_dt, tokens=sel)
    y_ref = ref["y"]
    y32 = moe.moe_layer(wl, tokens=tokens, ew=ew, acc="f32")["y"]
    m = {
        "rel_l2": PB.rel_l2(y_gpu, y_ref),
        "maxabs_rms_given_gpu_z": PB.maxabs_over_rms(y_gpu, y_cond),
        "maxabs_rms": PB.maxabs_over_rms(y_gpu, y_ref),
        "floor_maxabs_rms": PB.maxabs_over_rms(y32, y_ref),
        "floor_rel_l2": PB.rel_l2(y32, y_ref),
        "tokens": int(len(sel)), "rows": int(len(rows)),
    }
    if stages and rep["z"] and cfg.z_dt == "fp8":
        m["z_codes_differing"] = int(sum(r["codes_differing"] for r in rep["z"]))
        m["z_codes"] = int(sum(r["elements"] for r in rep["z"]))
        m["z_max_code_steps"] = int(max(r["max_code_steps"] for r in rep["z"]))
        m["z_scales_differing"] = int(sum(r["scales_differing"] for r in rep["z"]))
    if stages and rep["out"]:
        m["out_worst_ratio"] = max(r["worst_ratio"] for r in rep["out"])
    if rep["g"]:
        m["g_worst_ratio"] = max(r["worst_ratio"] for r in rep["g"])
    print(f"[metric] {tag or cfg.name} " + " ".join(
        f"{k}={v:.3e}" if isinstance(v, float) else f"{k}={v}" for k, v in m.items()), flush=True)
    assert np.all(np.isfinite(y_gpu))
    assert m["rel_l2"] <= LAYER_REL_L2, m
    assert m["maxabs_rms"] <= max(LAYER_MAXABS, FLOOR_FACTOR * m["floor_maxabs_rms"]), m
    return m


# Matrix-core GEMM outputs against the oracle's fp64 dots, relative L2
# (per-element bounds are in parity_bounds): FP8 1e-4, bf16 / fp32 1e-5.
GEMM_REL_L2 = {"fp8": 1e-4, "bf16": 1e-5, "f32": 1e-5}
