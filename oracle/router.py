"""Router top-k, computed plainly on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name this step but leave its arithmetic to the model: the router
scores every expert and a selection policy returns K expert ids and K
weights per token ("SGLang、NCCL 与 MoE EP：从职责边界到执行机制" §1.1 and the
TopKOutput of §3.6: topk_ids [T,K], topk_weights [T,K]).  Readings taken:

  * scores are the fp32 router logits, plus an optional per-expert fp32
    bias added with one fp32 addition;
  * the K selected experts are the K largest scores, in descending order;
    equal scores go to the lower expert id (NaN ranks below every number);
  * the weights are the softmax of the token's scores renormalised over the
    K selected experts, which equals the softmax over the K selected scores
    alone; it is evaluated in float64 and rounded once to fp32;
  * with ``bias_in_weights=False`` the bias only steers the selection and the
    weights use the unbiased logits of the selected experts.
"""
from __future__ import annotations

import math

import numpy as np


def router_scores(logits: np.ndarray, bias: np.ndarray | None) -> np.ndarray:
    """fp32 logits (+ fp32 bias): one correctly rounded fp32 add per entry."""
    s = np.asarray(logits, np.float32)
    if bias is None:
        return s.copy()
    return (s + np.asarray(bias, np.float32)[None, :]).astype(np.float32)


def router_topk(logits: np.ndarray, K: int, bias: np.ndarray | None = None,
                bias_in_weights: bool = True, tokens=None) -> tuple[np.ndarray, np.ndarray]:
    """topk_ids [n,K] int32 and topk_weights [n,K] fp32 for the given tokens
    (all by default), by a plain per-token ranking loop."""
    scores = router_scores(logits, bias)
    base = scores if bias_in_weights else np.asarray(logits, np.float32)
    T, E = scores.shape
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    ids = np.empty((len(tokens), K), np.int32)
    w = np.empty((len(tokens), K), np.float32)
    for n, t in enumerate(tokens):
        row = scores[t]

        def rank_key(e):
            v = float(row[e])
            return (1, 0.0, e) if math.isnan(v) else (0, -v, e)   # NaN after every number

        order = sorted(range(E), key=rank_key)[:K]
        v = [float(base[t, e]) for e in order]
        m = max(v)
        p = [math.exp(x - m) for x in v]
        s = math.fsum(p)
        ids[n] = order
        w[n] = [x / s for x in p]
    return ids, w
