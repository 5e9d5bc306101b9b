"""GPU parity of moe_router_topk against the oracle (oracle/router.py).

Bar: topk_ids bit-exact (both sides rank the same fp32 scores), topk_weights
within 1e-6 absolute (fp32 exp and a tree sum on the GPU vs a float64
softmax rounded once).  Full-size router inputs (prefill: 8192 x 256, top-8,
linear bias; skewed: 16384 x 64, top-6, Zipf bias) are compared on sampled
tokens, and on every token through properties that hold at any size."""
import numpy as np
import pytest
import torch

from gpu_util import announce, need_gpu
from oracle import router
from workloads import get_config, make_router_inputs

pytestmark = pytest.mark.gpu
W_TOL = 1e-6


@pytest.fixture(scope="module")
def ep():
    need_gpu()
    import combine_top_expert_amd as ep
    return ep


def run(ep, logits, K, bias=None, biw=True):
    T, E = logits.shape
    lg = torch.from_numpy(np.ascontiguousarray(logits)).cuda()
    b = None if bias is None else torch.from_numpy(np.ascontiguousarray(bias)).cuda()
    ids = torch.full((T, K), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, K), -7.0, dtype=torch.float32, device="cuda")
    ep.moe_router_topk(lg, K, ids, w, bias=b, bias_in_weights=biw)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def check(ids, w, logits, K, bias=None, biw=True, tokens=None):
    rid, rw = router.router_topk(logits, K, bias=bias, bias_in_weights=biw, tokens=tokens)
    gi = ids if tokens is None else ids[tokens]
    gw = w if tokens is None else w[tokens]
    assert np.array_equal(gi, rid)
    err = float(np.max(np.abs(gw.astype(np.float64) - rw))) if rw.size else 0.0
    print(f"[metric] router ids exact, max |dw| = {err:.2e}", flush=True)
    assert err <= W_TOL


@pytest.mark.parametrize("E,K", [(8, 1), (8, 8), (64, 6), (100, 7), (256, 8), (1000, 16), (1024, 64)])
@pytest.mark.parametrize("mode", ["plain", "bias", "bias_select_only", "ties"])
def test_router_small_all_tokens(ep, E, K, mode):
    announce("router", E, K, mode)
    rng = np.random.default_rng(E * 131 + K)
    x = rng.standard_normal((37, E)).astype(np.float32)
    bias = None
    if mode == "ties":
        x = (np.round(x * 2) / 2).astype(np.float32)
    if mode.startswith("bias"):
        bias = (0.5 * rng.standard_normal(E)).astype(np.float32)
    biw = mode != "bias_select_only"
    ids, w = run(ep, x, K, bias, biw)
    check(ids, w, x, K, bias, biw)


@pytest.mark.parametrize("E,K,T", [(256, 8, 16384), (200, 16, 16400), (128, 16, 1000), (64, 6, 1001)])
@pytest.mark.parametrize("mode", ["bias", "ties"])
def test_router_segmented_kernel(ep, E, K, T, mode):
    """Token counts that leave the last wave's segments partly empty, on the
    16-lane-segment kernel (E <= 128) and, at E = 200 and 256, on the
    wave-per-token kernel at large T: ids exact, weights to the bar."""
    announce("router seg", E, K, T, mode)
    rng = np.random.default_rng(E * 7 + K + T)
    x = rng.standard_normal((T, E)).astype(np.float32)
    if mode == "ties":
        x = (np.round(x * 2) / 2).astype(np.float32)
    bias = (0.5 * rng.standard_normal(E)).astype(np.float32) if mode == "bias" else None
    ids, w = run(ep, x, K, bias, True)
    check(ids, w, x, K, bias, True)


def test_router_special_values(ep):
    announce("router special values")
    x = np.array([[np.nan, -np.inf, 0.0, -0.0, 1.0, 1.0, -1.0, np.inf]], np.float32)
    x = np.repeat(x, 3, axis=0)
    ids, w = run(ep, x, 8)
    rid, _ = router.router_topk(x, 8)
    assert np.array_equal(ids, rid)               # inf, 1 (id 4), 1 (id 5), 0 (id 2), -0 (id 3), -1, -inf, nan
    assert list(ids[0]) == [7, 4, 5, 2, 3, 6, 1, 0]


@pytest.mark.parametrize("E,K", [(256, 16), (200, 8), (1024, 64)])
def test_router_special_values_wave_kernel(ep, E, K):
    """NaN, +-inf and +-0 among ordinary scores on the wave-per-token kernel
    (E > 128): NaN ranks below every number and goes to the lower id among
    NaNs, -0 ties +0, the lower id wins a tie; ids exact against the
    oracle."""
    announce("router special values, wave kernel", E, K)
    rng = np.random.default_rng(E + K)
    x = (np.round(rng.standard_normal((64, E)) * 2) / 2).astype(np.float32)
    specials = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0], np.float32)
    for t in range(64):
        pos = rng.choice(E, size=12, replace=False)
        x[t, pos] = specials[rng.integers(0, len(specials), size=12)]
    x[0, :] = np.nan                                # every score NaN: ids 0..K-1
    x[1, :] = 0.0
    x[1, ::2] = -0.0                                # every score zero
    ids, w = run(ep, x, K)
    rid, _ = router.router_topk(x, K)
    assert np.array_equal(ids, rid)
    assert list(ids[0]) == list(range(K))
    assert list(ids[1]) == list(range(K))


@pytest.mark.parametrize("name", ["prefill_fp8", "skewed_bf16"])
def test_router_full_size(ep, name):
    announce("router full", name)
    cfg = get_config(name)
    logits, bias = make_router_inputs(cfg)
    ids, w = run(ep, logits, cfg.K, bias)
    # every token: ids distinct, scores descending, nothing larger left out,
    # weights positive and summing to 1
    sc = (logits + bias[None, :]).astype(np.float32) if bias is not None else logits
    sel = np.take_along_axis(sc, ids.astype(np.int64), axis=1)
    assert np.all(np.diff(sel, axis=1) <= 0)
    masked = sc.copy()
    np.put_along_axis(masked, ids.astype(np.int64), -np.inf, axis=1)
    assert np.all(sel[:, -1] >= masked.max(axis=1))
    assert all(len(set(r)) == cfg.K for r in ids[:: max(1, cfg.T // 512)])
    assert np.all(w > 0) and np.allclose(w.sum(axis=1), 1.0, atol=1e-5)
    tokens = np.sort(np.random.default_rng(11).choice(cfg.T, 256, replace=False))
    check(ids, w, logits, cfg.K, bias, True, tokens)
