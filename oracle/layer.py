"""One pre-norm decoder layer: forward and backward by the chain rule, fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources: StreamBP skill page, "Implementation" (the streaming layer backward:
a layer function run forward, then backward with the upstream gradient, the
weight gradients summed and the input gradient kept) and "Architecture
Overview" ("Layer-Wise Application").  The pages name no layer structure; the
plain reading of an 8B-class decoder layer is used (no bias, gains multiply,
rotary position embedding optional)::

    h1 = RMSNorm(x; g1)
    q, k, v = h1 Wq^T, h1 Wk^T, h1 Wv^T            (heads: Hq, Hkv of width dh)
    q, k = HeadNorm(q; qn), HeadNorm(k; kn)         (only when w has "qn", "kn")
    q, k = Rope(q), Rope(k)                         (only when theta > 0)
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

Rotary position embedding (RoFormer, Su et al. 2021; not on the pages, which
name no position encoding): each head vector of width dh is split into halves
x = (x1, x2) of width dh/2, and for i < dh/2 the pair (x1_i, x2_i) is turned
by the angle p * theta^(-2i/dh), p the token's position:

    Rope(x)_i        = x1_i cos - x2_i sin
    Rope(x)_{i+dh/2} = x2_i cos + x1_i sin

A rotation's inverse is its transpose, so the backward turns the gradient by
the negative angle.  Positions count from 0 at the start of the row, and
from 0 at the start of each sequence when the row holds packed sequences.

QK-norm (optional, as in Qwen 3; not on the pages): HeadNorm is the RMSNorm
above applied to every head vector of width dh on its own, with one gain of
width dh shared by all heads of q (qn) and one shared by all heads of k (kn),
and the layer's eps.  Its backward is RMSNorm's, over (token, head) rows.
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


def rope_positions(T, cu_seqlens=None):
    """Position of every token: t, or t - cu[n] for the sequence n holding t."""
    pos = np.arange(T, dtype=np.float64)
    if cu_seqlens is not None:
        cu = list(cu_seqlens)
        for a, b in zip(cu, cu[1:]):
            pos[a:b] -= a
    return pos


def rope(x, pos, theta, inverse=False):
    """Rotary embedding of x [T, H, dh] at positions pos [T]; ``inverse``
    turns by the negative angle (the transpose of the forward rotation)."""
    x = _as64(x)
    dh = x.shape[-1]
    half = dh // 2
    inv_freq = float(theta) ** (-2.0 * np.arange(half) / dh)
    ang = _as64(pos)[:, None] * inv_freq[None, :]          # [T, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    if inverse:
        s = -s
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def _sigmoid(u):
    return 1.0 / (1.0 + np.exp(-u))


def layer_fwd(x, w, Hq, Hkv, dh, eps, cu_seqlens=None, rope_theta=0.0):
    """Forward of the layer; returns ``(y, cache)``.  ``cu_seqlens``: the
    tokens are packed independent sequences (attention stays inside each;
    every other step is token-wise).  ``rope_theta`` > 0 turns q and k by the
    rotary embedding of that base; 0 leaves them as projected."""
    x = _as64(x)
    W = {k: _as64(v) for k, v in w.items()}
    T = x.shape[0]
    h1, _, _ = rmsnorm_fwd(x, W["g1"], eps)
    q = h1 @ W["Wq"].T
    k = h1 @ W["Wk"].T
    v = h1 @ W["Wv"].T
    qk_norm = "qn" in W
    q_raw, k_raw = q, k
    if qk_norm:
        q = rmsnorm_fwd(q.reshape(T * Hq, dh), W["qn"], eps)[0].reshape(T, Hq * dh)
        k = rmsnorm_fwd(k.reshape(T * Hkv, dh), W["kn"], eps)[0].reshape(T, Hkv * dh)
    if rope_theta > 0:
        pos = rope_positions(T, cu_seqlens)
        q = rope(q.reshape(T, Hq, dh), pos, rope_theta).reshape(T, Hq * dh)
        k = rope(k.reshape(T, Hkv, dh), pos, rope_theta).reshape(T, Hkv * dh)
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
    cache = dict(h1=h1, q=q, k=k, v=v, o=o, a=a, n2=n2, u=u, g=g, m=m, lse=lse, q_raw=q_raw,
                 k_raw=k_raw)
    return y, cache


def layer_bwd(x, dy, w, Hq, Hkv, dh, eps, cu_seqlens=None, rope_theta=0.0):
    """Full (unchunked) backward.  Returns ``(dx, grads, y)``; ``grads`` maps
    every name of ``w`` (g1, Wq, Wk, Wv, Wo, g2, W1, W3, W2, and qn, kn with
    QK-norm) to its gradient.
    ``cu_seqlens`` and ``rope_theta`` as in ``layer_fwd``."""
    x = _as64(x)
    dy = _as64(dy)
    W = {k: _as64(v) for k, v in w.items()}
    T = x.shape[0]
    y, c = layer_fwd(x, W, Hq, Hkv, dh, eps, cu_seqlens, rope_theta)
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
    if rope_theta > 0:  # q, k were turned after the projection: turn back
        pos = rope_positions(T, cu_seqlens)
        dq = rope(dq.reshape(T, Hq, dh), pos, rope_theta, inverse=True).reshape(T, Hq * dh)
        dk = rope(dk.reshape(T, Hkv, dh), pos, rope_theta, inverse=True).reshape(T, Hkv * dh)
    if "qn" in W:  # back through the per-head norms
        dq, gr["qn"] = rmsnorm_bwd(c["q_raw"].reshape(T * Hq, dh), W["qn"], dq.reshape(T * Hq, dh), eps)
        dk, gr["kn"] = rmsnorm_bwd(c["k_raw"].reshape(T * Hkv, dh), W["kn"], dk.reshape(T * Hkv, dh), eps)
        dq = dq.reshape(T, Hq * dh)
        dk = dk.reshape(T, Hkv * dh)
    gr["Wq"] = dq.T @ c["h1"]
    gr["Wk"] = dk.T @ c["h1"]
    gr["Wv"] = dv.T @ c["h1"]
    dh1 = dq @ W["Wq"] + dk @ W["Wk"] + dv @ W["Wv"]
    dx_norm, gr["g1"] = rmsnorm_bwd(x, W["g1"], dh1, eps)
    dx = da + dx_norm
    return dx, gr, y
