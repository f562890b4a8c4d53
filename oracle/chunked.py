"""Chunked (StreamBP) evaluation of the same three functions, fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Used by one kind of
test only: chunked == unchunked (D-invariance), which shows that splitting
the chain rule along the sequence is algebraically exact, as the StreamBP
pages claim ("Exact Gradients" in the skill page's "Architecture Overview";
"linear decomposition of the chain rule along the sequence dimension" in the
arXiv abstract).  It is not the parity reference: the unchunked functions are.

Chunk table (skill page, "Implementation", the sequence decomposition): with
D chunks, ``size = T // D``; chunk i spans ``[i*size, (i+1)*size)`` and the
last one ends at T, so it takes the remainder.  D must satisfy 1 <= D <= T
(reading: D > T would make empty chunks).
"""
from __future__ import annotations

import numpy as np

from .layer import rmsnorm_fwd, rmsnorm_bwd, rope, rope_positions, _sigmoid


def chunk_table(T: int, D: int):
    if not (1 <= D <= T):
        raise ValueError("need 1 <= D <= T")
    size = T // D
    return [(i * size, (i + 1) * size if i < D - 1 else T) for i in range(D)]


def _as64(a):
    return np.asarray(a, dtype=np.float64)


def lmhead_ce(H, W, targets, weights, D, reduction="mean_valid"):
    """Per chunk: logits of the chunk only, softmax minus one-hot scaled by
    the global normaliser, dH rows of the chunk, dW accumulated."""
    H, W = _as64(H), _as64(W)
    T, d = H.shape
    y = np.asarray(targets).astype(np.int64)
    valid = y >= 0
    w = np.ones(T) if weights is None else _as64(weights)
    c = np.where(valid, w, 0.0)
    N = int(valid.sum()) if reduction == "mean_valid" else 1
    dH = np.zeros_like(H)
    dW = np.zeros_like(W)
    loss = 0.0
    if N == 0:
        return 0.0, dH, dW
    for s, e in chunk_table(T, D):
        Zc = H[s:e] @ W.T
        m = Zc.max(axis=1, keepdims=True)
        Ec = np.exp(Zc - m)
        Sc = Ec.sum(axis=1, keepdims=True)
        lse = (m + np.log(Sc))[:, 0]
        vc = valid[s:e]
        yc = np.where(vc, y[s:e], 0)
        r = np.arange(e - s)
        loss += float((c[s:e] * np.where(vc, lse - Zc[r, yc], 0.0)).sum())
        G = Ec / Sc
        G[r[vc], yc[vc]] -= 1.0
        G *= (c[s:e] / N)[:, None]
        G[~vc] = 0.0
        dH[s:e] = G @ W
        dW += G.T @ H[s:e]
    return loss / N, dH, dW


def attn_bwd(Q, K, V, dO, scale, D):
    """Query chunks in reverse order; chunk [s, e) reads keys [0, e) only and
    adds into dK, dV rows [0, e)."""
    Q, K, V, dO = _as64(Q), _as64(K), _as64(V), _as64(dO)
    B, T, Hq, dh = Q.shape
    Hkv = K.shape[2]
    G = Hq // Hkv
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for s, e in reversed(chunk_table(T, D)):
        ii = np.arange(s, e)[:, None]
        jj = np.arange(e)[None, :]
        for b in range(B):
            for h in range(Hq):
                kv = h // G
                q = Q[b, s:e, h]
                k = K[b, :e, kv]
                v = V[b, :e, kv]
                do = dO[b, s:e, h]
                S = scale * (q @ k.T)
                S[jj > ii] = -np.inf
                mx = S.max(axis=1, keepdims=True)
                P = np.exp(S - mx)
                P /= P.sum(axis=1, keepdims=True)
                o = P @ v
                dV[b, :e, kv] += P.T @ do
                dP = do @ v.T
                dS = P * (dP - (do * o).sum(axis=1, keepdims=True))
                dQ[b, s:e, h] = scale * (dS @ k)
                dK[b, :e, kv] += scale * (dS.T @ q)
    return dQ, dK, dV


def layer_bwd(x, dy, w, Hq, Hkv, dh, eps, D, rope_theta=0.0):
    """Streamed layer backward (``rope_theta`` as in ``layer.layer_fwd``).

    Pass F: h1 and the key/value projections for every token (the causal
    prefix every later query chunk needs).  Pass B, chunks in reverse order:
    recompute the chunk's forward, back-propagate the MLP, the second norm,
    the output projection and attention over the chunk's key prefix; dK/dV of
    chunk c are complete once chunk c is done (later chunks have already
    added theirs, earlier chunks never reach these keys), so the key/value
    projection gradients of chunk c are taken then.
    """
    x, dy = _as64(x), _as64(dy)
    W = {k: _as64(v) for k, v in w.items()}
    T, d = x.shape
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(dh)
    h1_all, _, _ = rmsnorm_fwd(x, W["g1"], eps)
    k_all = (h1_all @ W["Wk"].T).reshape(T, Hkv, dh)
    qk_norm = "qn" in W
    kraw_all = k_all
    if qk_norm:
        k_all = rmsnorm_fwd(k_all.reshape(T * Hkv, dh), W["kn"], eps)[0].reshape(T, Hkv, dh)
    pos = rope_positions(T)
    if rope_theta > 0:
        k_all = rope(k_all, pos, rope_theta)
    v_all = (h1_all @ W["Wv"].T).reshape(T, Hkv, dh)
    dk_all = np.zeros_like(k_all)
    dv_all = np.zeros_like(v_all)
    gr = {k: np.zeros_like(v) for k, v in W.items()}
    dx = np.zeros_like(x)
    for s, e in reversed(chunk_table(T, D)):
        xc = x[s:e]
        h1, _, _ = rmsnorm_fwd(xc, W["g1"], eps)
        q = (h1 @ W["Wq"].T).reshape(e - s, Hq, dh)
        q_raw = q
        if qk_norm:
            q = rmsnorm_fwd(q.reshape(-1, dh), W["qn"], eps)[0].reshape(e - s, Hq, dh)
        if rope_theta > 0:
            q = rope(q, pos[s:e], rope_theta)
        ii = np.arange(s, e)[:, None]
        jj = np.arange(e)[None, :]
        o = np.zeros((e - s, Hq, dh))
        Ps = {}
        for h in range(Hq):
            kv = h // G
            S = scale * (q[:, h] @ k_all[:e, kv].T)
            S[jj > ii] = -np.inf
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            Ps[h] = P
            o[:, h] = P @ v_all[:e, kv]
        o2 = o.reshape(e - s, Hq * dh)
        a = xc + o2 @ W["Wo"].T
        n2, _, _ = rmsnorm_fwd(a, W["g2"], eps)
        u = n2 @ W["W1"].T
        g = n2 @ W["W3"].T
        sig = _sigmoid(u)
        m = u * sig * g
        dyc = dy[s:e]
        gr["W2"] += dyc.T @ m
        dm = dyc @ W["W2"]
        du = dm * g * sig * (1.0 + u * (1.0 - sig))
        dg = dm * u * sig
        gr["W1"] += du.T @ n2
        gr["W3"] += dg.T @ n2
        dn2 = du @ W["W1"] + dg @ W["W3"]
        da_n, dg2 = rmsnorm_bwd(a, W["g2"], dn2, eps)
        gr["g2"] += dg2
        da = dyc + da_n
        gr["Wo"] += da.T @ o2
        do = (da @ W["Wo"]).reshape(e - s, Hq, dh)
        dq = np.zeros((e - s, Hq, dh))
        for h in range(Hq):
            kv = h // G
            P = Ps[h]
            dv_all[:e, kv] += P.T @ do[:, h]
            dP = do[:, h] @ v_all[:e, kv].T
            dS = P * (dP - (do[:, h] * o[:, h]).sum(axis=1, keepdims=True))
            dq[:, h] = scale * (dS @ k_all[:e, kv])
            dk_all[:e, kv] += scale * (dS.T @ q[:, h])
        dkc = dk_all[s:e]
        if rope_theta > 0:
            dq = rope(dq, pos[s:e], rope_theta, inverse=True)
            dkc = rope(dkc, pos[s:e], rope_theta, inverse=True)
        if qk_norm:
            dq, dqn = rmsnorm_bwd(q_raw.reshape(-1, dh), W["qn"], dq.reshape(-1, dh), eps)
            dkc, dkn = rmsnorm_bwd(kraw_all[s:e].reshape(-1, dh), W["kn"], dkc.reshape(-1, dh), eps)
            gr["qn"] += dqn
            gr["kn"] += dkn
        dq2 = dq.reshape(e - s, Hq * dh)
        dkc = dkc.reshape(e - s, Hkv * dh)
        dvc = dv_all[s:e].reshape(e - s, Hkv * dh)
        gr["Wq"] += dq2.T @ h1
        gr["Wk"] += dkc.T @ h1
        gr["Wv"] += dvc.T @ h1
        dh1 = dq2 @ W["Wq"] + dkc @ W["Wk"] + dvc @ W["Wv"]
        dx_n, dg1 = rmsnorm_bwd(xc, W["g1"], dh1, eps)
        gr["g1"] += dg1
        dx[s:e] = da + dx_n
    return dx, gr
