"""Pins of the whole-model oracle (CPU only): a stack of decoder layers under
a final RMSNorm and the LM head with cross-entropy."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

NAMES = ("g1", "Wq", "Wk", "Wv", "Wo", "g2", "W1", "W3", "W2")


def _layer(rng, d, Hq, Hkv, dh, Fw, std=0.3):
    return {
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


def _rand(L=2, T=7, d=8, Hq=2, Hkv=1, dh=4, Fw=12, V=11, seed=0, ignore=(), weights=False):
    rng = np.random.default_rng(seed)
    layers = [_layer(rng, d, Hq, Hkv, dh, Fw) for _ in range(L)]
    x0 = rng.normal(size=(T, d))
    g_f = 1 + 0.1 * rng.normal(size=d)
    W = rng.normal(size=(V, d)) * 0.5
    y = rng.integers(0, V, size=T)
    for t in ignore:
        y[t] = -1
    w = rng.normal(size=T) if weights else None
    return x0, layers, g_f, W, y, w


def _torch_rope(x, theta):
    T, H, dh = x.shape
    half = dh // 2
    f = theta ** (-2.0 * torch.arange(half, dtype=torch.float64) / dh)
    ang = torch.arange(T, dtype=torch.float64)[:, None] * f[None, :]
    z = torch.complex(x[..., :half], x[..., half:]) * torch.polar(torch.ones_like(ang), ang)[:, None, :]
    return torch.cat([z.real, z.imag], dim=-1)


def _torch_model(x, layers, g_f, W, y, wts, Hq, Hkv, dh, eps, theta):
    """The model written with torch ops, loss by F.cross_entropy per token."""
    T, d = x.shape
    for w in layers:
        h1 = F.rms_norm(x, (d,), weight=w["g1"], eps=eps)
        q = (h1 @ w["Wq"].T).reshape(T, Hq, dh)
        k = (h1 @ w["Wk"].T).reshape(T, Hkv, dh)
        if theta > 0:
            q, k = _torch_rope(q, theta), _torch_rope(k, theta)
        v = (h1 @ w["Wv"].T).reshape(T, Hkv, dh)
        o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], k.transpose(0, 1)[None],
                                           v.transpose(0, 1)[None], is_causal=True,
                                           scale=dh ** -0.5, enable_gqa=(Hq != Hkv))
        a = x + o[0].transpose(0, 1).reshape(T, Hq * dh) @ w["Wo"].T
        n2 = F.rms_norm(a, (d,), weight=w["g2"], eps=eps)
        x = a + (F.silu(n2 @ w["W1"].T) * (n2 @ w["W3"].T)) @ w["W2"].T
    h = F.rms_norm(x, (d,), weight=g_f, eps=eps)
    yt = torch.tensor(y)
    valid = yt >= 0
    ce = F.cross_entropy(h @ W.T, yt.clamp(min=0), reduction="none")
    c = valid.double() * (1.0 if wts is None else torch.tensor(wts))
    return (c * ce).sum() / valid.sum()


@pytest.mark.parametrize("L,theta,weighted", [(1, 0.0, False), (2, 0.0, True), (3, 100.0, False)])
def test_against_torch_autograd(L, theta, weighted):
    Hq, Hkv, dh, eps = 4, 2, 4, 1e-6
    x0, layers, g_f, W, y, wts = _rand(L=L, T=9, d=16, Hq=Hq, Hkv=Hkv, dh=dh, Fw=20, V=13,
                                       seed=L, ignore=(0, 5), weights=weighted)
    xt = torch.tensor(x0, requires_grad=True)
    lt = [{k: torch.tensor(v, requires_grad=True) for k, v in w.items()} for w in layers]
    gt = torch.tensor(g_f, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    loss_t = _torch_model(xt, lt, gt, Wt, y, wts, Hq, Hkv, dh, eps, theta)
    loss_t.backward()
    loss, dx0, grads, dg_f, dW = oracle.model_bwd(x0, layers, g_f, W, y, wts, Hq=Hq, Hkv=Hkv,
                                                  dh=dh, eps=eps, rope_theta=theta)
    assert abs(loss - loss_t.item()) <= 1e-12 * abs(loss)
    np.testing.assert_allclose(dx0, xt.grad.numpy(), rtol=1e-9, atol=1e-13)
    np.testing.assert_allclose(dg_f, gt.grad.numpy(), rtol=1e-9, atol=1e-13)
    np.testing.assert_allclose(dW, Wt.grad.numpy(), rtol=1e-9, atol=1e-13)
    for l in range(L):
        for k in NAMES:
            np.testing.assert_allclose(grads[l][k], lt[l][k].grad.numpy(), rtol=1e-9, atol=1e-13,
                                       err_msg=f"layer {l} {k}")


def test_finite_differences():
    Hq, Hkv, dh, eps = 2, 1, 4, 1e-6
    x0, layers, g_f, W, y, _ = _rand(L=2, T=5, d=8, Hq=Hq, Hkv=Hkv, dh=dh, Fw=12, V=7, seed=9,
                                     ignore=(2,))
    kw = dict(Hq=Hq, Hkv=Hkv, dh=dh, eps=eps, rope_theta=10.0)
    loss, dx0, grads, dg_f, dW = oracle.model_bwd(x0, layers, g_f, W, y, **kw)
    h = 1e-6

    def f(x=x0, ls=layers, g=g_f, Wm=W):
        return oracle.model_bwd(x, ls, g, Wm, y, **kw)[0]

    def fd_of(A, call):
        out = np.zeros_like(A)
        for idx in np.ndindex(A.shape):
            Ap, Am = A.copy(), A.copy()
            Ap[idx] += h
            Am[idx] -= h
            out[idx] = (call(Ap) - call(Am)) / (2 * h)
        return out

    def close(fd, an):
        assert np.abs(fd - an).max() <= 1e-7 * max(1.0, np.abs(an).max())

    close(fd_of(x0, lambda A: f(x=A)), dx0)
    close(fd_of(g_f, lambda A: f(g=A)), dg_f)
    close(fd_of(W, lambda A: f(Wm=A)), dW)
    for l, k in ((0, "Wq"), (0, "g2"), (1, "Wk"), (1, "W2")):
        def call(A, l=l, k=k):
            ls = [dict(w) for w in layers]
            ls[l][k] = A
            return f(ls=ls)
        close(fd_of(layers[l][k], call), grads[l][k])


def test_identity_layers_reduce_to_norm_and_head():
    # Wo = W2 = 0 in every layer: each layer is the identity, so the model is
    # the final RMSNorm under the LM head; only dWo and dW2 of the layers move
    Hq, Hkv, dh, eps = 2, 1, 4, 1e-6
    x0, layers, g_f, W, y, _ = _rand(L=3, T=6, d=8, Hq=Hq, Hkv=Hkv, dh=dh, Fw=12, V=9, seed=4)
    for w in layers:
        w["Wo"] = np.zeros_like(w["Wo"])
        w["W2"] = np.zeros_like(w["W2"])
    loss, dx0, grads, dg_f, dW = oracle.model_bwd(x0, layers, g_f, W, y, Hq=Hq, Hkv=Hkv, dh=dh,
                                                  eps=eps)
    hn, _, _ = oracle.rmsnorm_fwd(x0, g_f, eps)
    L1, dH, dW1, _, _ = oracle.lmhead_ce(hn, W, y)
    dx1, dg1 = oracle.rmsnorm_bwd(x0, g_f, dH, eps)
    assert loss == L1
    np.testing.assert_allclose(dx0, dx1, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dg_f, dg1, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dW, dW1, rtol=1e-13, atol=1e-15)
    for g in grads:
        for k in ("Wq", "Wk", "Wv", "W1", "W3", "g1", "g2"):
            assert np.abs(g[k]).max() == 0.0, k


def test_packed_sequences_are_independent():
    # targets of the second sequence ignored: its dx0 rows are exactly zero,
    # and the first sequence's gradients equal those of the model on it alone
    # (the normaliser counts the same valid tokens)
    Hq, Hkv, dh, eps = 2, 1, 4, 1e-6
    x0, layers, g_f, W, y, _ = _rand(L=2, T=9, d=8, Hq=Hq, Hkv=Hkv, dh=dh, Fw=12, V=9, seed=5)
    y[5:] = -1
    kw = dict(Hq=Hq, Hkv=Hkv, dh=dh, eps=eps, rope_theta=20.0)
    loss, dx0, grads, dg_f, dW = oracle.model_bwd(x0, layers, g_f, W, y, cu_seqlens=[0, 5, 9], **kw)
    l1, dx1, g1, dgf1, dW1 = oracle.model_bwd(x0[:5], layers, g_f, W, y[:5], **kw)
    assert abs(loss - l1) < 1e-14
    assert (dx0[5:] == 0).all()
    np.testing.assert_allclose(dx0[:5], dx1, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(dW, dW1, rtol=1e-12, atol=1e-15)
    for l in range(2):
        for k in NAMES:
            np.testing.assert_allclose(grads[l][k], g1[l][k], rtol=1e-11, atol=1e-15)


def test_backward_at_given_inputs():
    # at the inputs of its own forward, the backward at given layer inputs is
    # the model backward; at perturbed inputs each layer's gradients are the
    # single-layer backward at that layer's given input
    Hq, Hkv, dh, eps = 2, 1, 4, 1e-6
    x0, layers, g_f, W, y, _ = _rand(L=3, T=6, d=8, Hq=Hq, Hkv=Hkv, dh=dh, Fw=12, V=9, seed=12)
    kw = dict(Hq=Hq, Hkv=Hkv, dh=dh, eps=eps, rope_theta=30.0)
    ref = oracle.model_bwd(x0, layers, g_f, W, y, **kw)
    xs = oracle.model_fwd(x0, layers, Hq, Hkv, dh, eps, None, 30.0)
    got = oracle.model_bwd_at(xs, layers, g_f, W, y, **kw)
    assert got[0] == ref[0]
    np.testing.assert_array_equal(got[1], ref[1])
    rng = np.random.default_rng(3)
    xs2 = [x + 1e-2 * rng.normal(size=x.shape) for x in xs]
    loss, dx0, grads, _, _ = oracle.model_bwd_at(xs2, layers, g_f, W, y, **kw)
    hn, _, _ = oracle.rmsnorm_fwd(xs2[3], g_f, eps)
    L3, dH, _, _, _ = oracle.lmhead_ce(hn, W, y)
    up, _ = oracle.rmsnorm_bwd(xs2[3], g_f, dH, eps)
    assert loss == L3
    for l in (2, 1, 0):
        up, g, _ = oracle.layer_bwd(xs2[l], up, layers[l], Hq, Hkv, dh, eps, rope_theta=30.0)
        for k in NAMES:
            np.testing.assert_array_equal(grads[l][k], g[k])
    np.testing.assert_array_equal(dx0, up)
