"""Pins of the decoder-layer oracle (CPU only)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import chunked

NAMES = ("g1", "Wq", "Wk", "Wv", "Wo", "g2", "W1", "W3", "W2")


def _rand(T=6, d=8, Hq=2, Hkv=1, dh=4, Fw=12, seed=0, std=0.3):
    rng = np.random.default_rng(seed)
    w = {
        "g1": 1 + 0.1 * rng.normal(size=d),
        "Wq": rng.normal(size=(Hq * dh, d)) * std,
        "Wk": rng.normal(size=(Hkv * dh, d)) * std,
        "Wv": rng.normal(size=(Hkv * dh, d)) * std,
        "Wo": rng.normal(size=(d, Hq * dh)) * std,
        "g2": 1 + 0.1 * rng.normal(size=d),
        "W1": rng.normal(size=(Fw, d)) * std,
        "W3": rng.normal(size=(Fw, d)) * std,
        "W2": rng.normal(size=(d, Fw)) * std,
    }
    x = rng.normal(size=(T, d))
    dy = rng.normal(size=(T, d))
    return x, dy, w


def _torch_layer(x, w, Hq, Hkv, dh, eps):
    """The same layer written with torch ops (rms_norm, silu, sdpa)."""
    T, d = x.shape
    h1 = F.rms_norm(x, (d,), weight=w["g1"], eps=eps)
    q = (h1 @ w["Wq"].T).reshape(T, Hq, dh).transpose(0, 1)[None]
    k = (h1 @ w["Wk"].T).reshape(T, Hkv, dh).transpose(0, 1)[None]
    v = (h1 @ w["Wv"].T).reshape(T, Hkv, dh).transpose(0, 1)[None]
    o = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=dh ** -0.5,
                                       enable_gqa=(Hq != Hkv))
    o = o[0].transpose(0, 1).reshape(T, Hq * dh)
    a = x + o @ w["Wo"].T
    n2 = F.rms_norm(a, (d,), weight=w["g2"], eps=eps)
    m = F.silu(n2 @ w["W1"].T) * (n2 @ w["W3"].T)
    return a + m @ w["W2"].T


@pytest.mark.parametrize("Hq,Hkv", [(2, 1), (4, 2), (2, 2)])
def test_against_torch_autograd(Hq, Hkv):
    T, d, dh, Fw, eps = 11, 16, 4, 24, 1e-6
    x, dy, w = _rand(T, d, Hq, Hkv, dh, Fw, seed=Hq + 3 * Hkv)
    xt = torch.tensor(x, requires_grad=True)
    wt = {k: torch.tensor(v, requires_grad=True) for k, v in w.items()}
    yt = _torch_layer(xt, wt, Hq, Hkv, dh, eps)
    yt.backward(torch.tensor(dy))
    dx, gr, y = oracle.layer_bwd(x, dy, w, Hq, Hkv, dh, eps)
    np.testing.assert_allclose(y, yt.detach().numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-10, atol=1e-12)
    for k in NAMES:
        np.testing.assert_allclose(gr[k], wt[k].grad.numpy(), rtol=1e-10, atol=1e-12,
                                   err_msg=k)


def test_finite_differences():
    T, d, Hq, Hkv, dh, Fw, eps = 6, 8, 2, 1, 4, 12, 1e-6
    x, dy, w = _rand(T, d, Hq, Hkv, dh, Fw, seed=1)
    dx, gr, _ = oracle.layer_bwd(x, dy, w, Hq, Hkv, dh, eps)
    h = 1e-6

    def f(xx, ww):
        return float((oracle.layer_fwd(xx, ww, Hq, Hkv, dh, eps)[0] * dy).sum())

    fd = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        fd[idx] = (f(xp, w) - f(xm, w)) / (2 * h)
    assert np.abs(fd - dx).max() <= 1e-7 * max(1.0, np.abs(dx).max())
    for k in NAMES:
        A = w[k]
        fd = np.zeros_like(A)
        for idx in np.ndindex(A.shape):
            wp = dict(w)
            wm = dict(w)
            wp[k] = A.copy()
            wm[k] = A.copy()
            wp[k][idx] += h
            wm[k][idx] -= h
            fd[idx] = (f(x, wp) - f(x, wm)) / (2 * h)
        assert np.abs(fd - gr[k]).max() <= 1e-7 * max(1.0, np.abs(gr[k]).max()), k


def test_zero_output_projections():
    # Wo = W2 = 0: y = x, so dx = dy; only dWo and dW2 are non-zero
    T, d, Hq, Hkv, dh, Fw, eps = 7, 8, 2, 1, 4, 12, 1e-6
    x, dy, w = _rand(T, d, Hq, Hkv, dh, Fw, seed=2)
    w["Wo"] = np.zeros_like(w["Wo"])
    w["W2"] = np.zeros_like(w["W2"])
    dx, gr, y = oracle.layer_bwd(x, dy, w, Hq, Hkv, dh, eps)
    np.testing.assert_array_equal(y, x)
    np.testing.assert_array_equal(dx, dy)
    for k in ("Wq", "Wk", "Wv", "W1", "W3", "g1", "g2"):
        assert np.abs(gr[k]).max() == 0.0, k
    # dWo = dy^T o and dW2 = dy^T m with o, m from an independent forward
    _, cache = oracle.layer_fwd(x, w, Hq, Hkv, dh, eps)
    np.testing.assert_allclose(gr["Wo"], dy.T @ cache["o"], atol=1e-13)
    np.testing.assert_allclose(gr["W2"], dy.T @ cache["m"], atol=1e-13)


def test_rmsnorm_scale_invariance():
    # eps = 0: RMSNorm(c x) = RMSNorm(x), so the gradient is orthogonal to x
    rng = np.random.default_rng(5)
    x = rng.normal(size=(9, 16))
    g = 1 + 0.1 * rng.normal(size=16)
    dy = rng.normal(size=(9, 16))
    dx, _ = oracle.rmsnorm_bwd(x, g, dy, 0.0)
    assert np.abs((dx * x).sum(axis=1)).max() < 1e-13


@pytest.mark.parametrize("D", [1, 2, 4, 7])
def test_chunked_equals_unchunked(D):
    T, d, Hq, Hkv, dh, Fw, eps = 7, 8, 4, 2, 4, 12, 1e-6
    x, dy, w = _rand(T, d, Hq, Hkv, dh, Fw, seed=10 + D)
    dx, gr, _ = oracle.layer_bwd(x, dy, w, Hq, Hkv, dh, eps)
    dx2, gr2 = chunked.layer_bwd(x, dy, w, Hq, Hkv, dh, eps, D)
    assert np.abs(dx - dx2).max() < 1e-12
    for k in NAMES:
        assert np.abs(gr[k] - gr2[k]).max() < 1e-12, k


# ---------------------------------------------------------------------------
# Packed independent sequences

def _torch_layer_masked(x, w, Hq, Hkv, dh, eps, mask):
    T, d = x.shape
    h1 = F.rms_norm(x, (d,), weight=w["g1"], eps=eps)
    q = (h1 @ w["Wq"].T).reshape(T, Hq, dh).transpose(0, 1)[None]
    k = (h1 @ w["Wk"].T).reshape(T, Hkv, dh).transpose(0, 1)[None]
    v = (h1 @ w["Wv"].T).reshape(T, Hkv, dh).transpose(0, 1)[None]
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=dh ** -0.5,
                                       enable_gqa=(Hq != Hkv))
    o = o[0].transpose(0, 1).reshape(T, Hq * dh)
    a = x + o @ w["Wo"].T
    n2 = F.rms_norm(a, (d,), weight=w["g2"], eps=eps)
    m = F.silu(n2 @ w["W1"].T) * (n2 @ w["W3"].T)
    return a + m @ w["W2"].T


def test_packed_against_torch_autograd_with_block_mask():
    T, d, Hq, Hkv, dh, Fw, eps = 13, 16, 4, 2, 4, 24, 1e-6
    cu = [0, 4, 5, 13]
    x, dy, w = _rand(T, d, Hq, Hkv, dh, Fw, seed=17)
    seq = np.repeat(np.arange(3), np.diff(cu))
    i, j = np.arange(T)[:, None], np.arange(T)[None, :]
    mask = torch.tensor((j <= i) & (seq[:, None] == seq[None, :]))
    xt = torch.tensor(x, requires_grad=True)
    wt = {k: torch.tensor(v, requires_grad=True) for k, v in w.items()}
    yt = _torch_layer_masked(xt, wt, Hq, Hkv, dh, eps, mask)
    yt.backward(torch.tensor(dy))
    dx, gr, y = oracle.layer_bwd(x, dy, w, Hq, Hkv, dh, eps, cu_seqlens=cu)
    np.testing.assert_allclose(y, yt.detach().numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-10, atol=1e-12)
    for k in NAMES:
        np.testing.assert_allclose(gr[k], wt[k].grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=k)


def test_packed_sequences_are_independent():
    # no upstream gradient on the second sequence: its dx is exactly zero and
    # every weight gradient is that of the first sequence on its own
    T, d, Hq, Hkv, dh, Fw, eps = 10, 8, 2, 1, 4, 12, 1e-6
    x, dy, w = _rand(T, d, Hq, Hkv, dh, Fw, seed=18)
    dy[6:] = 0.0
    dx, gr, _ = oracle.layer_bwd(x, dy, w, Hq, Hkv, dh, eps, cu_seqlens=[0, 6, 10])
    dx1, gr1, _ = oracle.layer_bwd(x[:6], dy[:6], w, Hq, Hkv, dh, eps)
    assert (dx[6:] == 0).all()
    np.testing.assert_allclose(dx[:6], dx1, rtol=1e-13, atol=1e-15)
    for k in NAMES:
        np.testing.assert_allclose(gr[k], gr1[k], rtol=1e-12, atol=1e-15, err_msg=k)


# ---------------------------------------------------------------------------
# Rotary position embedding of q and k

from helpers import ev, load_golden  # noqa: E402


def test_rope_hand_worked():
    g = load_golden("rope_hand.json")
    x = np.tile(ev(g["x"]), (2, 1))[:, None, :]          # [T=2, H=1, dh=4]
    pos = np.array(g["positions"], dtype=np.float64)
    out = oracle.rope(x, pos, g["theta"])[:, 0]
    np.testing.assert_allclose(out, np.array([ev(r) for r in g["out"]]), rtol=0, atol=1e-15)
    inv = oracle.rope(x, pos, g["theta"], inverse=True)[:, 0]
    np.testing.assert_allclose(inv, np.array([ev(r) for r in g["inverse_out"]]), rtol=0, atol=1e-15)


def test_rope_rotation_properties():
    rng = np.random.default_rng(21)
    T, H, dh, theta = 9, 3, 8, 10000.0
    q = rng.normal(size=(T, H, dh))
    k = rng.normal(size=(T, H, dh))
    pos = np.arange(T, dtype=np.float64)
    rq = oracle.rope(q, pos, theta)
    # position 0 is the identity; norms are kept; inverse undoes forward
    np.testing.assert_array_equal(rq[0], q[0])
    np.testing.assert_allclose(np.linalg.norm(rq, axis=-1), np.linalg.norm(q, axis=-1), rtol=1e-14)
    np.testing.assert_allclose(oracle.rope(rq, pos, theta, inverse=True), q, atol=1e-14)
    # scores depend on the position difference only: <R_i q, R_j k> = <R_{i+c} q, R_{j+c} k>
    for c in (1.0, 5.0, 1234.0):
        a = (oracle.rope(q, pos, theta)[:, None] * oracle.rope(k, pos, theta)[None]).sum(-1)
        b = (oracle.rope(q, pos + c, theta)[:, None] * oracle.rope(k, pos + c, theta)[None]).sum(-1)
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-11)


def test_rope_positions_restart_per_sequence():
    np.testing.assert_array_equal(oracle.rope_positions(7, [0, 3, 4, 7]),
                                  [0, 1, 2, 0, 0, 1, 2])
    np.testing.assert_array_equal(oracle.rope_positions(4), [0, 1, 2, 3])


def _torch_rope(x, theta):
    """Rotary embedding written as a complex product: the pair (x1_i, x2_i)
    is the complex number x1_i + j x2_i, multiplied by exp(j p f_i)."""
    T, H, dh = x.shape
    half = dh // 2
    f = theta ** (-2.0 * torch.arange(half, dtype=torch.float64) / dh)
    ang = torch.arange(T, dtype=torch.float64)[:, None] * f[None, :]
    z = torch.complex(x[..., :half], x[..., half:]) * torch.polar(torch.ones_like(ang), ang)[:, None, :]
    return torch.cat([z.real, z.imag], dim=-1)


def _torch_layer_rope(x, w, Hq, Hkv, dh, eps, theta):
    T, d = x.shape
    h1 = F.rms_norm(x, (d,), weight=w["g1"], eps=eps)
    q = (h1 @ w["Wq"].T).reshape(T, Hq, dh)
    k = (h1 @ w["Wk"].T).reshape(T, Hkv, dh)
    if "qn" in w:  # QK-norm: RMSNorm over each head vector
        q = F.rms_norm(q, (dh,), weight=w["qn"], eps=eps)
        k = F.rms_norm(k, (dh,), weight=w["kn"], eps=eps)
    if theta > 0:
        q, k = _torch_rope(q, theta), _torch_rope(k, theta)
    q = q.transpose(0, 1)[None]
    k = k.transpose(0, 1)[None]
    v = (h1 @ w["Wv"].T).reshape(T, Hkv, dh).transpose(0, 1)[None]
    o = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=dh ** -0.5,
                                       enable_gqa=(Hq != Hkv))
    o = o[0].transpose(0, 1).reshape(T, Hq * dh)
    a = x + o @ w["Wo"].T
    n2 = F.rms_norm(a, (d,), weight=w["g2"], eps=eps)
    m = F.silu(n2 @ w["W1"].T) * (n2 @ w["W3"].T)
    return a + m @ w["W2"].T


@pytest.mark.parametrize("theta", [10000.0, 2.0])
def test_rope_layer_against_torch_autograd(theta):
    T, d, Hq, Hkv, dh, Fw, eps = 12, 16, 4, 2, 8, 24, 1e-6
    x, dy, w = _rand(T, d, Hq, Hkv, dh, Fw, seed=31)
    xt = torch.tensor(x, requires_grad=True)
    wt = {k: torch.tensor(v, requires_grad=True) for k, v in w.items()}
    yt = _torch_layer_rope(xt, wt, Hq, Hkv, dh, eps, theta)
    yt.backward(torch.tensor(dy))
    dx, gr, y = oracle.layer_bwd(x, dy, w, Hq, Hkv, dh, eps, rope_theta=theta)
    np.testing.assert_allclose(y, yt.detach().numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-10, atol=1e-12)
    for k in NAMES:
        np.testing.assert_allclose(gr[k], wt[k].grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=k)
    # the rotation changes the result (a dropped rope would pass nothing above)
    y0, _ = oracle.layer_fwd(x, w, Hq, Hkv, dh, eps)
    assert np.abs(y0 - y).max() > 1e-3


def test_rope_layer_finite_differences():
    T, d, Hq, Hkv, dh, Fw, eps, theta = 6, 8, 2, 1, 4, 12, 1e-6, 3.0
    x, dy, w = _rand(T, d, Hq, Hkv, dh, Fw, seed=32)
    dx, gr, _ = oracle.layer_bwd(x, dy, w, Hq, Hkv, dh, eps, rope_theta=theta)
    h = 1e-6

    def f(xx, ww):
        return float((oracle.layer_fwd(xx, ww, Hq, Hkv, dh, eps, rope_theta=theta)[0] * dy).sum())

    fd = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        fd[idx] = (f(xp, w) - f(xm, w)) / (2 * h)
    assert np.abs(fd - dx).max() <= 1e-7 * max(1.0, np.abs(dx).max())
    for k in ("Wq", "Wk"):
        A = w[k]
        fd = np.zeros_like(A)
        for idx in np.ndindex(A.shape):
            wp, wm = dict(w), dict(w)
            wp[k], wm[k] = A.copy(), A.copy()
            wp[k][idx] += h
            wm[k][idx] -= h
            fd[idx] = (f(x, wp) - f(x, wm)) / (2 * h)
        assert np.abs(fd - gr[k]).max() <= 1e-7 * max(1.0, np.abs(gr[k]).max()), k


@pytest.mark.parametrize("D", [1, 3, 7])
def test_rope_chunked_equals_unchunked(D):
    T, d, Hq, Hkv, dh, Fw, eps = 7, 8, 4, 2, 4, 12, 1e-6
    x, dy, w = _rand(T, d, Hq, Hkv, dh, Fw, seed=40 + D)
    dx, gr, _ = oracle.layer_bwd(x, dy, w, Hq, Hkv, dh, eps, rope_theta=50.0)
    dx2, gr2 = chunked.layer_bwd(x, dy, w, Hq, Hkv, dh, eps, D, rope_theta=50.0)
    assert np.abs(dx - dx2).max() < 1e-12
    for k in NAMES:
        assert np.abs(gr[k] - gr2[k]).max() < 1e-12, k


def test_rope_packed_sequence_starts_at_position_zero():
    # the second packed sequence, on its own, is the same layer over a row
    # that starts at position 0
    T, d, Hq, Hkv, dh, Fw, eps, theta = 10, 8, 2, 1, 4, 12, 1e-6, 7.0
    x, dy, w = _rand(T, d, Hq, Hkv, dh, Fw, seed=33)
    dy[:4] = 0.0
    dx, gr, y = oracle.layer_bwd(x, dy, w, Hq, Hkv, dh, eps, cu_seqlens=[0, 4, 10], rope_theta=theta)
    dx2, gr2, y2 = oracle.layer_bwd(x[4:], dy[4:], w, Hq, Hkv, dh, eps, rope_theta=theta)
    np.testing.assert_allclose(y[4:], y2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dx[4:], dx2, rtol=1e-12, atol=1e-14)
    assert (dx[:4] == 0).all()
    for k in NAMES:
        np.testing.assert_allclose(gr[k], gr2[k], rtol=1e-12, atol=1e-14, err_msg=k)


# ---------------------------------------------------------------------------
# QK-norm: RMSNorm of every q and k head vector (gains qn, kn of width dh)

def _with_qk_norm(w, dh, seed):
    rng = np.random.default_rng(seed)
    w = dict(w)
    w["qn"] = 1 + 0.2 * rng.normal(size=dh)
    w["kn"] = 1 + 0.2 * rng.normal(size=dh)
    return w


@pytest.mark.parametrize("theta", [1e4, 0.0])
def test_qk_norm_against_torch_autograd(theta):
    T, d, Hq, Hkv, dh, Fw, eps = 12, 16, 4, 2, 8, 24, 1e-6
    x, dy, w = _rand(T, d, Hq, Hkv, dh, Fw, seed=51)
    w = _with_qk_norm(w, dh, 52)
    xt = torch.tensor(x, requires_grad=True)
    wt = {k: torch.tensor(v, requires_grad=True) for k, v in w.items()}
    yt = _torch_layer_rope(xt, wt, Hq, Hkv, dh, eps, theta)
    yt.backward(torch.tensor(dy))
    dx, gr, y = oracle.layer_bwd(x, dy, w, Hq, Hkv, dh, eps, rope_theta=theta)
    np.testing.assert_allclose(y, yt.detach().numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-10, atol=1e-12)
    for k in NAMES + ("qn", "kn"):
        np.testing.assert_allclose(gr[k], wt[k].grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=k)


def test_qk_norm_finite_differences():
    T, d, Hq, Hkv, dh, Fw, eps, theta = 6, 8, 2, 1, 4, 12, 1e-6, 5.0
    x, dy, w = _rand(T, d, Hq, Hkv, dh, Fw, seed=53)
    w = _with_qk_norm(w, dh, 54)
    dx, gr, _ = oracle.layer_bwd(x, dy, w, Hq, Hkv, dh, eps, rope_theta=theta)
    h = 1e-6

    def f(ww):
        return float((oracle.layer_fwd(x, ww, Hq, Hkv, dh, eps, rope_theta=theta)[0] * dy).sum())

    for k in ("qn", "kn", "Wq", "Wk"):
        A = w[k]
        fd = np.zeros_like(A)
        for idx in np.ndindex(A.shape):
            wp, wm = dict(w), dict(w)
            wp[k], wm[k] = A.copy(), A.copy()
            wp[k][idx] += h
            wm[k][idx] -= h
            fd[idx] = (f(wp) - f(wm)) / (2 * h)
        assert np.abs(fd - gr[k]).max() <= 1e-7 * max(1.0, np.abs(gr[k]).max()), k


def test_qk_norm_scale_invariance():
    # scaling Wq (or Wk) leaves every head vector's direction, hence the layer,
    # unchanged at eps = 0; so the gradient of Wq is orthogonal to Wq
    T, d, Hq, Hkv, dh, Fw = 7, 8, 2, 1, 4, 12
    x, dy, w = _rand(T, d, Hq, Hkv, dh, Fw, seed=55)
    w = _with_qk_norm(w, dh, 56)
    y0, _ = oracle.layer_fwd(x, w, Hq, Hkv, dh, 0.0, rope_theta=3.0)
    w2 = dict(w, Wq=3.0 * w["Wq"], Wk=0.5 * w["Wk"])
    y1, _ = oracle.layer_fwd(x, w2, Hq, Hkv, dh, 0.0, rope_theta=3.0)
    np.testing.assert_allclose(y0, y1, rtol=1e-12, atol=1e-13)
    _, gr, _ = oracle.layer_bwd(x, dy, w, Hq, Hkv, dh, 0.0, rope_theta=3.0)
    assert abs((gr["Wq"] * w["Wq"]).sum()) < 1e-12 * np.abs(gr["Wq"]).sum()
    assert abs((gr["Wk"] * w["Wk"]).sum()) < 1e-12 * np.abs(gr["Wk"]).sum()


@pytest.mark.parametrize("D", [1, 3, 7])
def test_qk_norm_chunked_equals_unchunked(D):
    T, d, Hq, Hkv, dh, Fw, eps = 7, 8, 4, 2, 4, 12, 1e-6
    x, dy, w = _rand(T, d, Hq, Hkv, dh, Fw, seed=60 + D)
    w = _with_qk_norm(w, dh, 61)
    dx, gr, _ = oracle.layer_bwd(x, dy, w, Hq, Hkv, dh, eps, rope_theta=50.0)
    dx2, gr2 = chunked.layer_bwd(x, dy, w, Hq, Hkv, dh, eps, D, rope_theta=50.0)
    assert np.abs(dx - dx2).max() < 1e-12
    for k in NAMES + ("qn", "kn"):
        assert np.abs(gr[k] - gr2[k]).max() < 1e-12, k
