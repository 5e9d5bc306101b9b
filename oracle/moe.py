"""The MoE hot path, computed plainly on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages cited (by title):
  [EP]  "SGLang、NCCL 与 MoE EP：从职责边界到执行机制"
  [ECB] "SGLang Expert Compute Backend：从接收布局到 Triton 专家计算"
  [DEP] "DeepEP 架构与实现笔记"

Stages, in the order the path runs them:
  dispatch_layout -> permute -> gemm_w13 -> silu_mul -> gemm_w2 -> combine
and ``moe_layer`` composing them.  Readings where the pages are silent:
  * rows of one expert are allocated in flattened (token, k) order -- the
    sequential dispatch_convert loop of [DEP] §9.4 -- rather than the atomic
    arrival order of [EP] §2.3.4, which the pages allow to vary;
  * a route that does not fit the capacity is never written; it is counted,
    flagged, and its slot is -1;  id -1 means "no route", any other id outside
    [0, E) is flagged as bad and skipped;
  * dot products are accumulated in float64 over exactly dequantised operands
    and rounded once to fp32; SiLU(gate)*up is evaluated in fp32; Z is then
    rounded to the format GEMM-2 consumes (FP8 groups, bf16, or fp32);
  * combine accumulates in fp32 in k order; a token with no local route is 0.
"""
from __future__ import annotations

import math

import numpy as np

from . import formats as F

FLAG_CAPACITY = 1
FLAG_BAD_EXPERT_ID = 2


# ============================================================== stage 1: layout

def dispatch_layout(topk_ids: np.ndarray, E_global: int, expert_begin: int, L: int, R: int,
                    BM: int = 128) -> dict:
    """Per-expert counts, offsets, (t,k) -> row slots and row -> (t,k) sources.

    [EP] §2.3.4: each local expert has a row allocator; a route to local
    expert e takes s = counter[e]++ and lands at flattened row q = e*M + s,
    so every expert's valid rows form a contiguous prefix of its capacity
    block.  [EP] §2.3.6: the reverse map keeps, for each (t, k), its row q, and
    -1 for top-k entries that are not local.  [DEP] §9.4 (dispatch_convert):
    walking tokens, then top-k positions, in order, m = expert_start[e]++;
    with exact-fit offsets (R == 0) expert_start is the prefix sum of counts
    ([ECB] §2.6 / §4.1 compact storage).  tile_offsets[e+1] - tile_offsets[e]
    = ceil(counts[e] / BM) is the number of BM-row tiles expert e contributes
    ([ECB] §2.4)."""
    ids = np.asarray(topk_ids, np.int64)
    T, K = ids.shape
    flags = 0
    true_counts = [0] * L
    # pass 1: count routes per local expert
    for t in range(T):
        for k in range(K):
            g = int(ids[t, k])
            if g == -1:
                continue
            if g < -1 or g >= E_global:
                flags |= FLAG_BAD_EXPERT_ID
                continue
            if expert_begin <= g < expert_begin + L:
                true_counts[g - expert_begin] += 1
    if R > 0:
        counts = [min(c, R) for c in true_counts]
        if any(c > R for c in true_counts):
            flags |= FLAG_CAPACITY
        offsets = [e * R for e in range(L + 1)]
        rows_cap = L * R
    else:
        counts = list(true_counts)
        offsets = [0]
        for c in counts:
            offsets.append(offsets[-1] + c)
        rows_cap = T * K
    # pass 2: place routes in (t, k) order
    expert_start = list(offsets[:L])
    slot_of = np.full((T, K), -1, np.int32)
    row_src = np.full(rows_cap, -1, np.int32)
    for t in range(T):
        for k in range(K):
            g = int(ids[t, k])
            if g < 0 or g >= E_global or not (expert_begin <= g < expert_begin + L):
                continue
            e = g - expert_begin
            m = expert_start[e]
            expert_start[e] += 1
            if m - offsets[e] >= counts[e]:
                continue                      # beyond capacity: not placed
            slot_of[t, k] = m
            row_src[m] = t * K + k
    tile_offsets = [0]
    for c in counts:
        tile_offsets.append(tile_offsets[-1] + -(-c // BM))
    dropped = int(sum(tc - c for tc, c in zip(true_counts, counts)))
    return {
        "counts": np.array(counts, np.int32),
        "offsets": np.array(offsets, np.int32),
        "slot_of": slot_of,
        "row_src": row_src,
        "tile_offsets": np.array(tile_offsets, np.int32),
        "flags": flags,
        "dropped": dropped,
        "rows_cap": rows_cap,
    }


def valid_rows(counts: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    """All valid row indices of an expert-major buffer, expert by expert."""
    return np.concatenate([np.arange(offsets[e], offsets[e] + counts[e])
                           for e in range(len(counts))] + [np.zeros(0, np.int64)]).astype(np.int64)


# ============================================================== stage 2: permute

def x_values(x: np.ndarray, act: str) -> np.ndarray:
    """Token activations as fp32 values (bf16 bit patterns decoded exactly)."""
    return F.bf16_to_f32(x) if act == "bf16" else np.asarray(x, np.float32)


def permute(x: np.ndarray, act: str, row_src: np.ndarray, K: int, buf_dt: str,
            rows: np.ndarray | None = None) -> dict:
    """Expert-major buffer: buf[q] = x[row_src[q] // K] for every valid q.

    [EP] §2.3.4 (recv_tokens[e, s, :] = the token's payload) and [DEP] §9.4
    (recv_x_all[m] = recv_x[token]).  With ``buf_dt == 'fp8'`` each row is
    then quantised per 128 columns ([EP] §2.3.5: FP8 [L,M,H] with fp32
    scales [L,M,H/128]; [DEP] §11 recipe).  Padding rows are not produced.

    Returns {"rows": q indices, "data": rows' contents (fp32 values, bf16
    bits, or e4m3 codes), "scales": fp32 [n, H/128] for fp8}."""
    if rows is None:
        rows = np.nonzero(row_src >= 0)[0]
    rows = np.asarray(rows, np.int64)
    src_tok = row_src[rows] // K
    out = {"rows": rows}
    if buf_dt == "fp8":
        codes, scales = F.quant_fp8_groups(x_values(x, act)[src_tok])
        out["data"], out["scales"] = codes, scales
    else:
        assert buf_dt == act
        out["data"] = np.asarray(x)[src_tok].copy()
    return out


def buffer_values(data: np.ndarray, dt: str, scales: np.ndarray | None = None) -> np.ndarray:
    """Rows of a buffer in format ``dt`` -> exact float64 values."""
    if dt == "fp8":
        return F.dequant_fp8_groups(data, scales)
    if dt == "bf16":
        return F.bf16_to_f32(data).astype(np.float64)
    return np.asarray(data, np.float32).astype(np.float64)


def weight_values(w: np.ndarray, wdt: str, scales: np.ndarray | None = None) -> np.ndarray:
    """One expert's stored weight [out, in] -> exact float64 values."""
    if wdt == "fp8":
        return F.dequant_fp8_blocks(w, scales)
    if wdt == "bf16":
        return F.bf16_to_f32(w).astype(np.float64)
    return np.asarray(w, np.float32).astype(np.float64)


# ============================================================== stages 3-5: expert MLP

def _dot_rows(a_vals: np.ndarray, w_vals: np.ndarray, acc: str) -> np.ndarray:
    """Every dot product of a row of A with a row of W, rounded to fp32.
    acc="f64": float64 dot products rounded once (the oracle's definition);
    acc="f32": the same operands summed in fp32 by the BLAS routine, an
    evaluation order a correct fp32 implementation may also take.  The second
    form only measures how much the format's roundings downstream react to
    fp32-level differences; no result is checked against it."""
    if acc == "f64":
        return (np.asarray(a_vals, np.float64) @ np.asarray(w_vals, np.float64).T).astype(np.float32)
    assert acc == "f32", acc
    return np.asarray(a_vals, np.float32) @ np.asarray(w_vals, np.float32).T


def gemm_w13(a_vals: np.ndarray, w13_vals: np.ndarray, acc: str = "f64") -> np.ndarray:
    """G = A W13^T for one expert's valid rows ([ECB] §1.1: X_e [m_e, H] ->
    gate/up GEMM -> [m_e, 2I]; weights stored [expert, out, in], §3.5).
    float64 dot products, rounded once to fp32."""
    return _dot_rows(a_vals, w13_vals, acc)


def silu(v: np.ndarray) -> np.ndarray:
    """SiLU(v) = v * sigmoid(v) = v / (1 + exp(-v)), evaluated in fp32."""
    v = np.asarray(v, np.float32)
    with np.errstate(over="ignore"):
        return (v / (np.float32(1.0) + np.exp(-v))).astype(np.float32)


def silu_mul(g: np.ndarray, I: int) -> np.ndarray:
    """Z = SiLU(gate) * up with gate the first I columns of G and up the last
    I ([ECB] §3.6: non-interleaved gate/up, first half gate).  fp32."""
    g = np.asarray(g, np.float32)
    assert g.shape[1] == 2 * I
    return (silu(g[:, :I]) * g[:, I:]).astype(np.float32)


def z_to_format(z: np.ndarray, z_dt: str) -> dict:
    """Round Z to what GEMM-2 consumes: FP8 groups of 128 ([ECB] §3.6: Z is
    re-quantised before the down GEMM with its own scales), bf16 (RNE) or fp32."""
    if z_dt == "fp8":
        codes, scales = F.quant_fp8_groups(z)
        return {"data": codes, "scales": scales}
    if z_dt == "bf16":
        return {"data": F.f32_to_bf16(z)}
    return {"data": np.asarray(z, np.float32)}


def gemm_w2(z_vals: np.ndarray, w2_vals: np.ndarray, acc: str = "f64") -> np.ndarray:
    """out = Z W2^T ([ECB] §1.1: [m_e, I] -> down GEMM -> [m_e, H]), float64
    dot products rounded once to fp32."""
    return _dot_rows(z_vals, w2_vals, acc)


def out_to_format(out: np.ndarray, out_dt: str) -> np.ndarray:
    """Expert output / combined output rounded to its storage format, as fp32."""
    return F.round_bf16(out) if out_dt == "bf16" else np.asarray(out, np.float32)


# ============================================================== stage 6: combine

def combine(out_rows: dict, slot_of: np.ndarray, weights: np.ndarray, y_dt: str,
            tokens: np.ndarray | None = None) -> np.ndarray:
    """y[t] = sum_k w[t,k] * out[slot_of[t,k]] over local routes.

    [EP] §1.1: the routed output is the router-weighted sum of the selected
    experts' outputs, weights applied to expert *outputs*; §2.3.6: combine
    follows the (t, k) -> q map back and weights by topk_weights[t, k].
    [DEP] §9.4 combine_convert: local weighted sum per original token.
    fp32 accumulation in k order; 0 for a token without a local route.
    ``out_rows`` maps row q -> fp32 output row (values already rounded to the
    expert-output format)."""
    T, K = slot_of.shape
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    H = len(next(iter(out_rows.values()))) if out_rows else 0
    y = np.zeros((len(tokens), H), np.float32)
    for i, t in enumerate(tokens):
        acc = np.zeros(H, np.float32)
        for k in range(K):
            q = int(slot_of[t, k])
            if q < 0:
                continue
            prod = (np.float32(weights[t, k]) * out_rows[q]).astype(np.float32)
            acc = (acc + prod).astype(np.float32)
        y[i] = acc
    return out_to_format(y, y_dt)


# ============================================================== the layer

class ExpertWeights:
    """Dequantised (float64) expert weights, made on first use and cached."""

    def __init__(self, cfg, w: dict, cache: bool = True):
        self.cfg, self.w, self.cache, self._c13, self._c2 = cfg, w, cache, {}, {}

    def _get(self, store: dict, name: str, e: int) -> np.ndarray:
        if e in store:
            return store[e]
        sc = self.w.get(name + "_scales")
        v = weight_values(self.w[name][e], self.cfg.wdt, None if sc is None else sc[e])
        if self.cache:
            store[e] = v
        return v

    def w13(self, e: int) -> np.ndarray:
        return self._get(self._c13, "w13", e)

    def w2(self, e: int) -> np.ndarray:
        return self._get(self._c2, "w2", e)


def expert_mlp_rows(cfg, a_vals_by_row: dict, expert_of_row: dict, ew: ExpertWeights,
                    acc: str = "f64") -> dict:
    """Run GEMM-1 -> SiLU*up -> Z rounding -> GEMM-2 on the given rows, each
    with its own expert's weights.  Returns per-row dicts of G (fp32), Z in
    its format, and the expert output (fp32 values of the output format).
    ``acc`` selects the dot products' accumulation (see _dot_rows)."""
    res = {"G": {}, "Z": {}, "Zs": {}, "out": {}}
    by_e: dict[int, list] = {}
    for q, e in expert_of_row.items():
        by_e.setdefault(e, []).append(q)
    for e, qs in sorted(by_e.items()):
        qs = sorted(qs)
        a = np.stack([a_vals_by_row[q] for q in qs])
        g = gemm_w13(a, ew.w13(e), acc)
        z = silu_mul(g, cfg.I)
        zf = z_to_format(z, cfg.z_dt)
        zv = buffer_values(zf["data"], cfg.z_dt, zf.get("scales"))
        out = out_to_format(gemm_w2(zv, ew.w2(e), acc), cfg.out_dt)
        for i, q in enumerate(qs):
            res["G"][q] = g[i]
            res["Z"][q] = zf["data"][i]
            if "scales" in zf:
                res["Zs"][q] = zf["scales"][i]
            res["out"][q] = out[i]
    return res


def moe_layer(wl, tokens=None, BM: int = 128, ew: ExpertWeights | None = None,
              acc: str = "f64") -> dict:
    """dispatch_layout -> permute -> expert MLP -> combine for a workload.

    ``tokens`` restricts the expert MLP and combine to the routes of those
    tokens (layout is always computed in full, it is cheap); the outputs for
    those tokens are then exactly what the full computation gives them.
    ``acc`` selects the dot products' accumulation (see _dot_rows)."""
    cfg = wl.cfg
    ew = ew or ExpertWeights(cfg, wl.w)
    if cfg.routing == "given":
        sh = wl.share
        counts, offsets, slot_of = sh["counts"], sh["offsets"], sh["slot_of"]
        lay = {"counts": counts, "offsets": offsets, "slot_of": slot_of}
        sel = np.arange(cfg.T) if tokens is None else np.asarray(tokens)
        rows = np.unique(slot_of[sel].ravel())
        rows = rows[rows >= 0]
        perm = {"rows": rows, "data": sh["buf"][rows]}
    else:
        lay = dispatch_layout(wl.ids, cfg.E, cfg.expert_begin, cfg.L, cfg.R, BM)
        slot_of = lay["slot_of"]
        sel = np.arange(cfg.T) if tokens is None else np.asarray(tokens)
        rows = np.unique(slot_of[sel].ravel())
        rows = rows[rows >= 0]
        perm = permute(wl.x, cfg.act, lay["row_src"], cfg.K, cfg.buf_dt, rows)
    a_vals = buffer_values(perm["data"], cfg.buf_dt, perm.get("scales"))
    offsets, counts = lay["offsets"], lay["counts"]
    e_of = {}
    for q in perm["rows"]:
        e = int(np.searchsorted(offsets, q, side="right") - 1)
        assert offsets[e] <= q < offsets[e] + counts[e]
        e_of[int(q)] = e
    a_by_row = {int(q): a_vals[i] for i, q in enumerate(perm["rows"])}
    mlp = expert_mlp_rows(cfg, a_by_row, e_of, ew, acc)
    y = combine(mlp["out"], slot_of, wl.weights, cfg.out_dt, tokens=sel)
    return {"layout": lay, "perm": perm, "mlp": mlp, "y": y, "tokens": sel}


def gemm_flops(H: int, I: int, rows: int) -> float:
    """Main GEMM FLOPs of the gated expert: 2*H*2I + 2*I*H = 6*H*I per routed
    row ([EP] §5.3, [ECB] §1.1)."""
    return 6.0 * H * I * rows


def m_tile_count(counts, BM: int) -> int:
    """Number of BM-row tiles over all experts ([ECB] §2.4, §4.3)."""
    return int(sum(math.ceil(int(c) / BM) for c in counts))
