"""Pins of the backward oracle (oracle/backward.py) against references that
share none of its code:

* torch autograd of a dense float64 forward (every route run directly on x,
  no permutation, no layout) gives dx and d_w -- the hand-derived formulas
  must match the automatic derivative;
* central finite differences of SiLU(gate) * up in float64 pin
  silu_mul_backward;
* an explicit 0/1 permutation matrix pins permute_backward and the dispatch
  half of combine_backward;
* autograd's gradients of the dense forward's expert weights pin dW2, dW13.
Shapes include non-local experts (a share of L < E experts) and tokens with
no local route."""
import numpy as np
import pytest
import torch

from oracle import backward as B
from oracle import formats as F
from oracle import moe
from workloads import get_config, make_workload

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _dense_forward_backward(wl, dy, weight_grads=False):
    """float64 autograd of y[t] = sum_{k: local} w[t,k] * F_e(x[t]); with
    weight_grads also d/dW13[e] and d/dW2[e]."""
    cfg = wl.cfg
    ew = moe.ExpertWeights(cfg, wl.w)
    x = torch.tensor(moe.x_values(wl.x, cfg.act), dtype=torch.float64, requires_grad=True)
    w = torch.tensor(np.asarray(wl.weights, np.float64), requires_grad=True)
    W13 = [torch.tensor(ew.w13(e), requires_grad=weight_grads) for e in range(cfg.L)]
    W2 = [torch.tensor(ew.w2(e), requires_grad=weight_grads) for e in range(cfg.L)]
    T, K = wl.ids.shape
    y = torch.zeros(T, cfg.H, dtype=torch.float64)
    rows = []
    for t in range(T):
        for k in range(K):
            g = int(wl.ids[t, k])
            e = g - cfg.expert_begin
            if g < 0 or not (0 <= e < cfg.L):
                continue
            rows.append((t, k, e))
    for t, k, e in rows:
        gu = x[t] @ W13[e].T
        z = torch.nn.functional.silu(gu[:cfg.I]) * gu[cfg.I:]
        y[t] = y[t] + w[t, k] * (z @ W2[e].T)
    y.backward(torch.tensor(dy, dtype=torch.float64))
    if weight_grads:
        zero = lambda t, shape: (t.grad.numpy() if t.grad is not None else np.zeros(shape))
        return (x.grad.numpy(), w.grad.numpy(),
                np.stack([zero(W13[e], W13[e].shape) for e in range(cfg.L)]),
                np.stack([zero(W2[e], W2[e].shape) for e in range(cfg.L)]))
    return x.grad.numpy(), w.grad.numpy()


def _share_config():
    # 8 global experts, this GPU holds experts 2..5: routes to 0, 1, 6, 7 are
    # not local, and some tokens have no local route
    return get_config("toy_fp32").scaled(name="toy_fp32_share", L=4, expert_begin=2, T=48,
                                         routing="softmax", H=256, I=128)


@pytest.mark.parametrize("which", ["toy_fp32", "manyrow_fp32_small", "share"])
def test_layer_backward_matches_autograd(which):
    cfg = _share_config() if which == "share" else get_config(which)
    if which == "manyrow_fp32_small":
        cfg = cfg.scaled(name="manyrow_fp32_bwd", T=96)
    wl = make_workload(cfg)
    rng = np.random.default_rng(5)
    dy = rng.standard_normal((cfg.T, cfg.H)).astype(np.float32)
    res = B.layer_backward(wl, dy, moe.ExpertWeights(cfg, wl.w))
    dx_ref, dw_ref = _dense_forward_backward(wl, dy)
    # the oracle rounds G, Z, out and every gradient to fp32 once per step
    err_x = np.linalg.norm(res["dx"] - dx_ref) / np.linalg.norm(dx_ref)
    assert err_x < 2e-6, err_x
    local = np.zeros_like(dw_ref, bool)
    local[res["layout"]["slot_of"] >= 0] = True
    assert np.all(res["d_w"][~local] == 0)
    assert np.all(dw_ref[~local] == 0)
    err_w = np.linalg.norm(res["d_w"] - dw_ref) / np.linalg.norm(dw_ref)
    assert err_w < 2e-6, err_w
    if which == "share":
        no_local = ~(res["layout"]["slot_of"] >= 0).any(axis=1)
        assert no_local.any() and np.all(res["dx"][no_local] == 0)


@pytest.mark.parametrize("which", ["toy_fp32", "share"])
def test_weight_gradients_match_autograd(which):
    """dW2, dW13 of the oracle against autograd's gradients of the dense
    forward's weights (experts without rows: zeros on both sides)."""
    cfg = _share_config() if which == "share" else get_config(which)
    wl = make_workload(cfg)
    rng = np.random.default_rng(6)
    dy = rng.standard_normal((cfg.T, cfg.H)).astype(np.float32)
    res = B.layer_backward(wl, dy, moe.ExpertWeights(cfg, wl.w))
    _, _, dw13_ref, dw2_ref = _dense_forward_backward(wl, dy, weight_grads=True)
    for got, ref in ((res["dw2"], dw2_ref), (res["dw13"], dw13_ref)):
        assert got.shape == ref.shape
        err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert err < 2e-6, err
        for e in range(cfg.L):
            if not np.any(ref[e]):
                assert not np.any(got[e])


def test_wgrad_closed_form():
    rng = np.random.default_rng(1)
    b = rng.standard_normal((7, 5))
    a = rng.standard_normal((7, 3))
    c = B.wgrad(b, a, 5, 3)
    ref = np.array([[sum(b[r, n] * a[r, k] for r in range(7)) for k in range(3)] for n in range(5)])
    np.testing.assert_allclose(c, ref, rtol=1e-6)
    assert not np.any(B.wgrad(np.zeros((0, 5)), np.zeros((0, 3)), 5, 3))


def test_autograd_pin_catches_planted_mistakes():
    """The comparison above fails for a dropped term and for a sign error in
    the SiLU derivative (mistakes planted in a copy of the oracle's step)."""
    cfg = get_config("toy_fp32")
    wl = make_workload(cfg)
    rng = np.random.default_rng(5)
    dy = rng.standard_normal((cfg.T, cfg.H)).astype(np.float32)
    dx_ref, _ = _dense_forward_backward(wl, dy)
    good = B.silu_mul_backward

    def dropped(g, dz):            # d_gate without the (1 + gate (1 - s)) factor
        out = good(g, dz)
        I = dz.shape[1]
        s = 1.0 / (1.0 + np.exp(-g[:, :I]))
        out[:, :I] = (dz * g[:, I:] * s).astype(np.float32)
        return out

    def flipped(g, dz):            # wrong sign inside the factor
        I = dz.shape[1]
        s = 1.0 / (1.0 + np.exp(-g[:, :I]))
        out = good(g, dz)
        out[:, :I] = (dz * g[:, I:] * s * (1 - g[:, :I] * (1 - s))).astype(np.float32)
        return out

    for bad in (dropped, flipped):
        B.silu_mul_backward = bad
        try:
            res = B.layer_backward(wl, dy, moe.ExpertWeights(cfg, wl.w))
        finally:
            B.silu_mul_backward = good
        assert np.linalg.norm(res["dx"] - dx_ref) / np.linalg.norm(dx_ref) > 1e-3


def test_silu_mul_backward_finite_differences():
    rng = np.random.default_rng(3)
    I = 16
    g = (rng.standard_normal((5, 2 * I)) * 3).astype(np.float32)
    dz = rng.standard_normal((5, I)).astype(np.float32)

    def zf(gg):                    # Z(G) in float64
        gate, up = gg[:, :I], gg[:, I:]
        return gate / (1 + np.exp(-gate)) * up

    num = np.zeros_like(g, np.float64)
    h = 1e-6
    for i in range(g.shape[0]):
        for j in range(2 * I):
            gp = g.astype(np.float64).copy()
            gm = gp.copy()
            gp[i, j] += h
            gm[i, j] -= h
            num[i, j] = np.sum((zf(gp) - zf(gm)) * dz) / (2 * h)
    ana = B.silu_mul_backward(g, dz)
    assert np.max(np.abs(ana - num)) < 1e-4 * max(1.0, np.max(np.abs(num)))


def test_silu_mul_backward_special_values():
    """At gate = 0: SiLU = 0 and its derivative is 1/2; large |gate| saturates
    to the identity (derivative 1) or to ~0 without overflow."""
    g = np.array([[0.0, 60.0, -60.0, 2.0, 3.0, 5.0]], np.float32)   # I = 3: gates 0, 60, -60
    dz = np.ones((1, 3), np.float32)
    d = B.silu_mul_backward(g, dz)
    assert d[0, 0] == np.float32(0.5 * 2.0)         # d_gate = dz * up * 1/2
    assert abs(d[0, 1] - 3.0) < 1e-6                 # identity slope times up
    assert abs(d[0, 2]) < 1e-20 and np.isfinite(d).all()
    assert d[0, 3] == 0.0                            # d_up = dz * SiLU(0) = 0
    assert abs(d[0, 4] - 60.0) < 1e-4 and abs(d[0, 5]) < 1e-20


def test_permute_and_combine_backward_match_matrix_forms():
    cfg = _share_config()
    wl = make_workload(cfg)
    lay = moe.dispatch_layout(wl.ids, cfg.E, cfg.expert_begin, cfg.L, cfg.R)
    slot_of = lay["slot_of"]
    rows = moe.valid_rows(lay["counts"], lay["offsets"])
    rng = np.random.default_rng(9)
    H = 64
    d_rows = {int(q): rng.standard_normal(H).astype(np.float32) for q in rows}
    # explicit permutation matrix P[q, t] = 1 for each local route of t
    P = np.zeros((cfg.rows_cap, cfg.T))
    for t in range(cfg.T):
        for k in range(cfg.K):
            if slot_of[t, k] >= 0:
                P[slot_of[t, k], t] = 1
    D = np.zeros((cfg.rows_cap, H))
    for q, v in d_rows.items():
        D[q] = v
    dx = B.permute_backward(d_rows, slot_of, H, "f32")
    np.testing.assert_allclose(dx, P.T @ D, rtol=1e-6, atol=1e-6)
    # combine backward: d_out = W dy scattered through P; d_w[t,k] = <dy[t], out[q]>
    dy = rng.standard_normal((cfg.T, H)).astype(np.float32)
    out_rows = {int(q): rng.standard_normal(H).astype(np.float32) for q in rows}
    d_out, d_w = B.combine_backward(dy, out_rows, slot_of, wl.weights, "f32")
    for t in range(cfg.T):
        for k in range(cfg.K):
            q = slot_of[t, k]
            if q < 0:
                assert d_w[t, k] == 0
                continue
            np.testing.assert_array_equal(d_out[q], np.float32(wl.weights[t, k]) * dy[t])
            assert abs(d_w[t, k] - float(dy[t].astype(np.float64) @ out_rows[q])) < 1e-5
    assert set(d_out) == {int(q) for q in rows}


def test_to_format_rounds_bf16_once():
    v = np.array([1.0 + 2 ** -9, 1.0 + 3 * 2 ** -9], np.float32)
    np.testing.assert_array_equal(B.to_format(v, "bf16"), F.round_bf16(v))
    np.testing.assert_array_equal(B.to_format(v, "f32"), v)
