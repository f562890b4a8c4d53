"""One pre-norm decoder layer: forward and backward by the chain rule, fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources: StreamBP skill page, "Implementation" (the streaming layer backward:
a layer function run forward, then backward with the upstream gradient, the
weight gradients summed and the input gradient kept) and "Architecture
Overview" ("Layer-Wise Application").  The pages name no layer structure; the
plain reading of an 8B-class decoder layer is used (no bias, no rotary
embedding, gains multiply)::

    h1 = RMSNorm(x; g1)
    q, k, v = h1 Wq^T, h1 Wk^T, h1 Wv^T            (heads: Hq, Hkv of width dh)
    o  = CausalGQA(q, k, v), scale 1/sqrt(dh)
    a  = x + o Wo^T
    n2 = RMSNorm(a; g2)
    u, g = n2 W1^T, n2 W3^T
    m  = silu(u) * g
    y  = a + m W2^T

RMSNorm(x; g) = g * x / r with r = sqrt(mean(x^2) + eps).  Its backward, for
upstream dy and xhat = x / r::

    dx = (g * dy - xhat * mean(xhat * g * dy)) / r
    dg = sum_t dy * xhat

(from d xhat_k / d x_j = (delta_kj - xhat_k xhat_j / n) / r).

silu(u) = u sigma(u),   silu'(u) = sigma(u) (1 + u (1 - sigma(u))).
"""
from __future__ import annotations

import numpy as np

from .attention import attn_bwd, attn_bwd_packed, attn_fwd, attn_fwd_packed


def _as64(a):
    return np.asarray(a, dtype=np.float64)


def rmsnorm_fwd(x, g, eps):
    x = _as64(x)
    r = np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    xhat = x / r
    return _as64(g) * xhat, xhat, r


def rmsnorm_bwd(x, g, dy, eps):
    """Returns ``(dx, dg)``."""
    x, g, dy = _as64(x), _as64(g), _as64(dy)
    r = np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    xhat = x / r
    gdy = g * dy
    dx = (gdy - xhat * (xhat * gdy).mean(axis=-1, keepdims=True)) / r
    dg = (dy * xhat).sum(axis=0)
    return dx, dg


def _sigmoid(u):
    return 1.0 / (1.0 + np.exp(-u))


def layer_fwd(x, w, Hq, Hkv, dh, eps, cu_seqlens=None):
    """Forward of the layer; returns ``(y, cache)``.  ``cu_seqlens``: the
    tokens are packed independent sequences (attention stays inside each;
    every other step is token-wise)."""
    x = _as64(x)
    W = {k: _as64(v) for k, v in w.items()}
    T = x.shape[0]
    h1, _, _ = rmsnorm_fwd(x, W["g1"], eps)
    q = h1 @ W["Wq"].T
    k = h1 @ W["Wk"].T
    v = h1 @ W["Wv"].T
    scale = 1.0 / np.sqrt(dh)
    q4, k4, v4 = q.reshape(1, T, Hq, dh), k.reshape(1, T, Hkv, dh), v.reshape(1, T, Hkv, dh)
    if cu_seqlens is None:
        o4, lse = attn_fwd(q4, k4, v4, scale)
    else:
        o4, lse = attn_fwd_packed(q4, k4, v4, scale, cu_seqlens)
    o = o4.reshape(T, Hq * dh)
    a = x + o @ W["Wo"].T
    n2, _, _ = rmsnorm_fwd(a, W["g2"], eps)
    u = n2 @ W["W1"].T
    g = n2 @ W["W3"].T
    su = u * _sigmoid(u)
    m = su * g
    y = a + m @ W["W2"].T
    cache = dict(h1=h1, q=q, k=k, v=v, o=o, a=a, n2=n2, u=u, g=g, m=m, lse=lse)
    return y, cache


def layer_bwd(x, dy, w, Hq, Hkv, dh, eps, cu_seqlens=None):
    """Full (unchunked) backward.  Returns ``(dx, grads, y)``; ``grads`` maps
    every name of ``w`` (g1, Wq, Wk, Wv, Wo, g2, W1, W3, W2) to its gradient.
    ``cu_seqlens`` as in ``layer_fwd``."""
    x = _as64(x)
    dy = _as64(dy)
    W = {k: _as64(v) for k, v in w.items()}
    T = x.shape[0]
    y, c = layer_fwd(x, W, Hq, Hkv, dh, eps, cu_seqlens)
    gr = {}
    # MLP: y = a + m W2^T
    gr["W2"] = dy.T @ c["m"]
    dm = dy @ W["W2"]
    sig = _sigmoid(c["u"])
    su = c["u"] * sig
    dsilu = sig * (1.0 + c["u"] * (1.0 - sig))
    du = dm * c["g"] * dsilu
    dg = dm * su
    gr["W1"] = du.T @ c["n2"]
    gr["W3"] = dg.T @ c["n2"]
    dn2 = du @ W["W1"] + dg @ W["W3"]
    da_norm, gr["g2"] = rmsnorm_bwd(c["a"], W["g2"], dn2, eps)
    da = dy + da_norm
    # attention block: a = x + o Wo^T
    gr["Wo"] = da.T @ c["o"]
    do = da @ W["Wo"]
    scale = 1.0 / np.sqrt(dh)
    args = (c["q"].reshape(1, T, Hq, dh), c["k"].reshape(1, T, Hkv, dh),
            c["v"].reshape(1, T, Hkv, dh), do.reshape(1, T, Hq, dh), scale)
    if cu_seqlens is None:
        dq4, dk4, dv4, _, _ = attn_bwd(*args)
    else:
        dq4, dk4, dv4, _, _ = attn_bwd_packed(*args, cu_seqlens)
    dq = dq4.reshape(T, Hq * dh)
    dk = dk4.reshape(T, Hkv * dh)
    dv = dv4.reshape(T, Hkv * dh)
    gr["Wq"] = dq.T @ c["h1"]
    gr["Wk"] = dk.T @ c["h1"]
    gr["Wv"] = dv.T @ c["h1"]
    dh1 = dq @ W["Wq"] + dk @ W["Wk"] + dv @ W["Wv"]
    dx_norm, gr["g1"] = rmsnorm_bwd(x, W["g1"], dh1, eps)
    dx = da + dx_norm
    return dx, gr, y
