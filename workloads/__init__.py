"""Seeded synthetic inputs for the MoE dispatch -> expert MLP -> combine path.

This module only *makes inputs*: routing ids and router weights, token
activations, and expert weights.  It holds none of the path's arithmetic
(no layout, no permutation, no activation quantisation, no GEMM, no combine),
so both the CPU oracle and the GPU tests/bench can consume the same bytes.

Every array is returned as numpy:
  * bf16 tensors as ``uint16`` bit patterns,
  * OCP e4m3fn tensors as ``uint8`` codes,
  * fp32 / int32 as themselves.

Workload shapes follow the worked examples and shapes the pages use:
  * ``toy_fp32``   -- the 112-token, 8-expert, top-2 routing with token 5
    sent to (E1, E6) at weights (0.25, 0.75) and every other token to
    (E0, E7) ("SGLang、NCCL 与 MoE EP", two guiding questions and §3.2),
    fp32 throughout, H=256, I=128, capacity 128.
  * ``share_bf16`` -- the two-expert expert-major buffer with counts [70, 12],
    R=128, H=256, I=128 ("SGLang Expert Compute Backend", §2.2-§2.4), bf16.
  * ``decode_fp8`` / ``prefill_fp8`` -- one GPU's 32-expert share of a
    256-expert top-8 layer with H=7168, I=2048 and block-wise (128x128) FP8
    weights (the block-FP8 expert GEMM of "SGLang Expert Compute Backend",
    §3.5), T=128 and T=8192.
  * ``skewed_bf16`` -- 64 local experts, top-6, Zipf-biased routing, H=4096,
    I=1408, bf16, exact-fit (compact) offsets ("SGLang Expert Compute
    Backend", §2.6 and §4.1).
Smaller variants with the same structure serve the parity tests.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np
import torch

__all__ = ["MoEConfig", "CONFIGS", "get_config", "make_routing", "make_activations",
           "make_weights", "make_share_buffer", "bf16_bits_from_f32", "Workload", "make_workload"]


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int                 # tokens submitted on this GPU
    K: int                 # top-k
    E: int                 # global experts
    expert_begin: int      # first global expert owned here
    L: int                 # local experts
    H: int                 # hidden size
    I: int                 # expert intermediate size
    R: int                 # capacity rows per local expert; 0 = exact-fit (compact)
    act: str               # "f32" | "bf16"   token activations
    wdt: str               # "f32" | "bf16" | "fp8"   expert weights
    routing: str           # "token5" | "softmax" | "given"
    bias: str = "none"     # "none" | "linear" | "zipf"  per-expert logit bias
    bias_alpha: float = 0.0
    seed: int = 1001

    @property
    def rows_cap(self) -> int:
        return self.L * self.R if self.R > 0 else self.T * self.K

    @property
    def buf_dt(self) -> str:
        """dtype of the expert-major receive buffer (GEMM-1 A operand)."""
        return "fp8" if self.wdt == "fp8" else self.act

    @property
    def z_dt(self) -> str:
        """dtype of the activated intermediate Z (GEMM-2 A operand)."""
        return "fp8" if self.wdt == "fp8" else ("f32" if self.wdt == "f32" else "bf16")

    @property
    def out_dt(self) -> str:
        """dtype of expert outputs and of the combined output."""
        return "f32" if self.act == "f32" else "bf16"

    def scaled(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


def _prefill_capacity(T: int, K: int, E: int) -> int:
    # capacity = ceil(T * top-k / experts * 2): twice the mean rows per expert
    return int(math.ceil(T * K / E * 2))


CONFIGS = {
    "toy_fp32": MoEConfig("toy_fp32", T=112, K=2, E=8, expert_begin=0, L=8, H=256, I=128,
                          R=128, act="f32", wdt="f32", routing="token5", seed=1001),
    "share_bf16": MoEConfig("share_bf16", T=82, K=1, E=2, expert_begin=0, L=2, H=256, I=128,
                            R=128, act="bf16", wdt="bf16", routing="given", seed=1002),
    "decode_fp8": MoEConfig("decode_fp8", T=128, K=8, E=256, expert_begin=0, L=32, H=7168,
                            I=2048, R=128, act="bf16", wdt="fp8", routing="softmax", seed=1003),
    "prefill_fp8": MoEConfig("prefill_fp8", T=8192, K=8, E=256, expert_begin=0, L=32, H=7168,
                             I=2048, R=_prefill_capacity(8192, 8, 256), act="bf16", wdt="fp8",
                             routing="softmax", bias="linear", bias_alpha=0.6, seed=1004),
    "skewed_bf16": MoEConfig("skewed_bf16", T=16384, K=6, E=64, expert_begin=0, L=64, H=4096,
                             I=1408, R=0, act="bf16", wdt="bf16", routing="softmax",
                             bias="zipf", bias_alpha=1.2, seed=1005),
}

# Reduced shapes with the same structure, used where the CPU oracle must
# cover every output element.  They still span several GEMM tiles in M and N
# and leave ragged row tails.
CONFIGS.update({
    "decode_fp8_small": CONFIGS["decode_fp8"].scaled(name="decode_fp8_small", T=64, H=512, I=384),
    "prefill_fp8_small": CONFIGS["prefill_fp8"].scaled(
        name="prefill_fp8_small", T=1024, E=32, L=8, H=512, I=384,
        R=_prefill_capacity(1024, 8, 32)),
    "skewed_bf16_small": CONFIGS["skewed_bf16"].scaled(name="skewed_bf16_small", T=1024, H=512,
                                                      I=384),
    "toy_bf16_fp8w": CONFIGS["toy_fp32"].scaled(name="toy_bf16_fp8w", act="bf16", wdt="fp8"),
})

# Reduced shapes with a few experts holding hundreds of rows each: several
# full GEMM row tiles per expert, ragged tails and near-empty experts
# (Zipf-biased routing); odd and single-stage K loops (FP8: H=128 is one
# 128-byte stage, I=384 three).
CONFIGS.update({
    "manyrow_bf16_small": CONFIGS["skewed_bf16"].scaled(
        name="manyrow_bf16_small", T=1024, K=2, E=4, L=4, H=384, I=256),
    "manyrow_fp8_small": CONFIGS["prefill_fp8"].scaled(
        name="manyrow_fp8_small", T=512, K=4, E=8, L=4, H=128, I=384, R=640,
        bias="zipf", bias_alpha=1.2),
    "manyrow_fp32_small": CONFIGS["toy_fp32"].scaled(
        name="manyrow_fp32_small", T=384, K=2, E=4, L=4, R=384, routing="softmax",
        bias="zipf", bias_alpha=1.2),
})

# The largest local expert count (L = 1024, the library's limit) with about
# two rows per expert: one short row tile per expert, many empty experts,
# and ids on both sides of the owned range [512, 1536) of 2048.
CONFIGS.update({
    "manyexpert_fp8_small": CONFIGS["prefill_fp8"].scaled(
        name="manyexpert_fp8_small", T=512, K=8, E=2048, expert_begin=512, L=1024, H=256, I=128,
        R=16, bias="none"),
    "manyexpert_bf16_small": CONFIGS["skewed_bf16"].scaled(
        name="manyexpert_bf16_small", T=512, K=8, E=2048, expert_begin=512, L=1024, H=256, I=128,
        R=0, bias="none"),
})


def get_config(name: str) -> MoEConfig:
    return CONFIGS[name]


# ----------------------------------------------------------------------------
# helpers

def _rng(seed: int, *stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, *stream]))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 through torch's cast (input recipe)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _fp8_block_quant(w: np.ndarray, blk: int = 128):
    """Make block-scaled e4m3fn weights from fp32 ones: one fp32 scale per
    128x128 (out, in) block, amax/448 per block, codes from torch's cast.
    This is how the synthetic FP8 weights are produced (input recipe)."""
    n, k = w.shape
    assert n % blk == 0 and k % blk == 0
    tw = torch.from_numpy(w)
    blocks = tw.view(n // blk, blk, k // blk, blk)
    amax = blocks.abs().amax(dim=(1, 3)).clamp(min=1e-4)            # [n/128, k/128]
    scale = amax / 448.0
    q = (blocks * (448.0 / amax)[:, None, :, None]).to(torch.float8_e4m3fn)
    codes = q.view(torch.uint8).reshape(n, k).numpy().copy()
    return codes, scale.numpy().astype(np.float32)


# ----------------------------------------------------------------------------
# routing

def make_routing(cfg: MoEConfig):
    """topk_ids [T,K] int32 (global expert ids) and topk_weights [T,K] fp32."""
    T, K, E = cfg.T, cfg.K, cfg.E
    if cfg.routing == "token5":
        # every token -> (E0, E7) at (0.5, 0.5); token 5 -> (E1, E6) at (0.25, 0.75)
        ids = np.tile(np.array([0, 7], np.int32), (T, 1))
        w = np.full((T, K), 0.5, np.float32)
        if T > 5:
            ids[5] = [1, 6]
            w[5] = [0.25, 0.75]
        return ids, w
    if cfg.routing == "softmax":
        rng = _rng(cfg.seed, 0)
        logits = rng.standard_normal((T, E), dtype=np.float32).astype(np.float64)
        e = np.arange(E, dtype=np.float64)
        if cfg.bias == "linear":
            # bias repeats every L experts so every GPU's share sees the same skew
            logits += cfg.bias_alpha * (e % cfg.L) / max(cfg.L - 1, 1)
        elif cfg.bias == "zipf":
            logits += -cfg.bias_alpha * np.log(e + 1.0)
        # top-k sorted by descending logit; ties go to the lower expert id
        order = np.argsort(-logits, axis=1, kind="stable")[:, :K]
        sel = np.take_along_axis(logits, order, axis=1)
        p = np.exp(sel - sel[:, :1])
        w = (p / p.sum(axis=1, keepdims=True)).astype(np.float32)   # renormalised softmax
        return order.astype(np.int32), w
    raise ValueError(f"routing {cfg.routing!r} has no generated ids")


def make_router_inputs(cfg: MoEConfig, seed_stream: int = 7):
    """Router logits [T,E] fp32 ~ N(0,1) and the per-expert fp32 bias of the
    workload's routing recipe (None without one): the inputs of the router
    top-k step, drawn from their own seeded stream."""
    logits = _rng(cfg.seed, seed_stream).standard_normal((cfg.T, cfg.E), dtype=np.float32)
    e = np.arange(cfg.E, dtype=np.float64)
    if cfg.bias == "linear":
        bias = cfg.bias_alpha * (e % cfg.L) / max(cfg.L - 1, 1)
    elif cfg.bias == "zipf":
        bias = -cfg.bias_alpha * np.log(e + 1.0)
    else:
        return logits, None
    return logits, bias.astype(np.float32)


# ----------------------------------------------------------------------------
# activations and weights

def make_activations(cfg: MoEConfig) -> np.ndarray:
    """x [T,H] ~ N(0,1): fp32, or bf16 bits."""
    x = _rng(cfg.seed, 1).standard_normal((cfg.T, cfg.H), dtype=np.float32)
    return x if cfg.act == "f32" else bf16_bits_from_f32(x)


def _one_expert(cfg: MoEConfig, which: int, e: int):
    if which == 0:
        n, k = 2 * cfg.I, cfg.H      # W13[e]: [2I, H]  (gate rows first, then up rows)
    else:
        n, k = cfg.H, cfg.I          # W2[e]:  [H, I]
    w = _rng(cfg.seed, 2 + which, e).standard_normal((n, k), dtype=np.float32)
    w *= np.float32(1.0 / math.sqrt(k))                 # N(0, 1/fan_in)
    if cfg.wdt == "f32":
        return w, None
    if cfg.wdt == "bf16":
        return bf16_bits_from_f32(w), None
    return _fp8_block_quant(w)


def make_weights(cfg: MoEConfig, experts=None, threads: int = 8):
    """Expert weights in storage order [expert, out, in].

    Returns dict with w13 [L,2I,H], w2 [L,H,I] and, for FP8, w13_scales
    [L,2I/128,H/128] and w2_scales [L,H/128,I/128] (fp32).  ``experts``
    restricts generation to a subset of local experts (others left zero)."""
    L = cfg.L
    experts = list(range(L)) if experts is None else list(experts)
    wdt = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[cfg.wdt]
    out = {"w13": np.zeros((L, 2 * cfg.I, cfg.H), wdt), "w2": np.zeros((L, cfg.H, cfg.I), wdt)}
    if cfg.wdt == "fp8":
        out["w13_scales"] = np.zeros((L, 2 * cfg.I // 128, cfg.H // 128), np.float32)
        out["w2_scales"] = np.zeros((L, cfg.H // 128, cfg.I // 128), np.float32)

    def job(args):
        which, e = args
        # each expert has its own random stream, so threading does not change values
        v, s = _one_expert(cfg, which, cfg.expert_begin + e)
        name = "w13" if which == 0 else "w2"
        out[name][e] = v
        if s is not None:
            out[name + "_scales"][e] = s

    jobs = [(which, e) for e in experts for which in (0, 1)]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(job, jobs))
    return out


def make_share_buffer(cfg: MoEConfig):
    """The given expert-major buffer of the two-expert share workload.

    Returns buf [L*R, H] bf16 bits with N(0,1) in valid rows and 0xFFFF (a
    bf16 NaN) in every padding row, counts [L], offsets [L+1], the token ->
    row map slot_of [T,1] (a seeded bijection of the valid rows onto tokens
    0..T-1) and router weights [T,1] ~ U(0,1)."""
    counts = np.array([70, 12], np.int32)
    L, R, H = cfg.L, cfg.R, cfg.H
    assert counts.sum() == cfg.T and len(counts) == L
    rng = _rng(cfg.seed, 1)
    buf = np.full((L * R, H), 0xFFFF, np.uint16)
    valid_rows = np.concatenate([e * R + np.arange(c) for e, c in enumerate(counts)])
    vals = rng.standard_normal((len(valid_rows), H), dtype=np.float32)
    buf[valid_rows] = bf16_bits_from_f32(vals)
    perm = _rng(cfg.seed, 4).permutation(len(valid_rows))
    slot_of = valid_rows[perm].astype(np.int32).reshape(cfg.T, 1)
    w = _rng(cfg.seed, 5).uniform(0.0, 1.0, (cfg.T, 1)).astype(np.float32)
    offsets = (np.arange(L + 1) * R).astype(np.int32)
    return {"buf": buf, "counts": counts, "offsets": offsets, "slot_of": slot_of, "weights": w}


@dataclass
class Workload:
    cfg: MoEConfig
    ids: np.ndarray | None
    weights: np.ndarray
    x: np.ndarray | None
    w: dict
    share: dict | None = None


def make_workload(name_or_cfg, experts=None) -> Workload:
    cfg = name_or_cfg if isinstance(name_or_cfg, MoEConfig) else get_config(name_or_cfg)
    w = make_weights(cfg, experts)
    if cfg.routing == "given":
        share = make_share_buffer(cfg)
        return Workload(cfg, None, share["weights"], None, w, share)
    ids, rw = make_routing(cfg)
    return Workload(cfg, ids, rw, make_activations(cfg), w)
