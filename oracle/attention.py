"""Causal grouped-query attention: forward and backward, unchunked, fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources: StreamBP skill page, "Architecture Overview" ("Causal Structure
Exploitation") and "Practical Guidance" ("Chunk Size Boundaries", "Causal
Masking"): a query sees only keys at or before its own position, and masks
must hold across chunk boundaries.  Grouped-query attention is the "GQA"
paper the mlsanity page lists under "Builds on"; the pages give no formula
for it, so the plain reading is used: query head h reads key/value head
floor(h / G) with G = Hq / Hkv (contiguous groups).

Definitions, per batch row b and query head h with kv = h // G, scale s::

    S   = s Q_h K_kv^T,  S_ij = -inf for j > i
    P   = softmax_rows(S),  O_h = P V_kv,  LSE_i = log sum_j exp(S_ij)
    dV_kv += P^T dO_h
    dP  = dO_h V_kv^T
    dS  = P * (dP - rowsum(dO_h * O_h))
    dQ_h  = s dS K_kv
    dK_kv += s dS^T Q_h

Layout: token-major, Q/dO/dQ [B, T, Hq, dh], K/V/dK/dV [B, T, Hkv, dh].

Packed sequences (``attn_bwd_packed``): several independent sequences laid
end to end in one row of T tokens, sequence n holding tokens
[cu[n], cu[n+1]).  "Practical Guidance" asks that attention masks hold
across chunk boundaries; the reading for packed data is that a query sees
only keys of its own sequence at or before it, so the packed result is,
sequence by sequence, the causal attention above on that sequence alone.
"""
from __future__ import annotations

import numpy as np


def _as64(a):
    return np.asarray(a, dtype=np.float64)


def _check(Q, K, V):
    B, T, Hq, dh = Q.shape
    Hkv = K.shape[2]
    if K.shape != (B, T, Hkv, dh) or V.shape != K.shape or Hq % Hkv != 0:
        raise ValueError("bad attention shapes")
    return B, T, Hq, Hkv, dh, Hq // Hkv


def _probs(q, k, scale):
    """Causal softmax rows of s q k^T for one head; returns (P, LSE)."""
    T = q.shape[0]
    S = scale * (q @ k.T)
    S[np.triu_indices(T, 1)] = -np.inf
    m = S.max(axis=1)
    E = np.exp(S - m[:, None])
    Z = E.sum(axis=1)
    return E / Z[:, None], m + np.log(Z)


def attn_fwd(Q, K, V, scale):
    """Returns ``(O [B,T,Hq,dh], LSE [B,T,Hq])``."""
    Q, K, V = _as64(Q), _as64(K), _as64(V)
    B, T, Hq, Hkv, dh, G = _check(Q, K, V)
    O = np.zeros_like(Q)
    LSE = np.zeros((B, T, Hq))
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            P, lse = _probs(Q[b, :, h], K[b, :, kv], scale)
            O[b, :, h] = P @ V[b, :, kv]
            LSE[b, :, h] = lse
    return O, LSE


def attn_bwd(Q, K, V, dO, scale):
    """Returns ``(dQ, dK, dV, O, LSE)`` of the causal GQA attention."""
    Q, K, V, dO = _as64(Q), _as64(K), _as64(V), _as64(dO)
    B, T, Hq, Hkv, dh, G = _check(Q, K, V)
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    O = np.zeros_like(Q)
    LSE = np.zeros((B, T, Hq))
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            q, k, v, do = Q[b, :, h], K[b, :, kv], V[b, :, kv], dO[b, :, h]
            P, lse = _probs(q, k, scale)
            o = P @ v
            O[b, :, h] = o
            LSE[b, :, h] = lse
            dV[b, :, kv] += P.T @ do
            dP = do @ v.T
            delta = (do * o).sum(axis=1)
            dS = P * (dP - delta[:, None])
            dQ[b, :, h] = scale * (dS @ k)
            dK[b, :, kv] += scale * (dS.T @ q)
    return dQ, dK, dV, O, LSE


def attn_bwd_sampled(Q, K, V, dO, scale, b, h_list, q_rows, k_rows):
    """Exact gradients at sampled positions, for full-size spot checks.

    For batch row ``b``, every query head in ``h_list`` gives ``dQ[b, i, h]``
    for each i in ``q_rows``; every kv head those heads belong to gives
    ``dK[b, j, kv]`` and ``dV[b, j, kv]`` for each j in ``k_rows``, summed
    over *all* G query heads of the group.  Work is O(T^2 dh) per head (the
    log-sum-exp of every query row is needed for a key's gradient), memory
    O(T) per row: no [T, T] matrix is formed.

    Returns ``(dQ_s {h: [len(q_rows), dh]}, dK_s {kv: ...}, dV_s {kv: ...})``.
    """
    Q, K, V, dO = (np.asarray(a) for a in (Q, K, V, dO))
    _, T, Hq, Hkv, dh, G = _check(Q, K, V)
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_rows = np.asarray(k_rows, dtype=np.int64)
    kv_heads = sorted({h // G for h in h_list})
    dQ_s, dK_s, dV_s = {}, {}, {}
    for kv in kv_heads:
        k = _as64(K[b, :, kv])
        v = _as64(V[b, :, kv])
        dKs = np.zeros((len(k_rows), dh))
        dVs = np.zeros((len(k_rows), dh))
        for h in range(kv * G, (kv + 1) * G):
            q = _as64(Q[b, :, h])
            do = _as64(dO[b, :, h])
            # log-sum-exp and output of every query row, block by block
            lse = np.empty(T)
            delta = np.empty(T)
            blk = 512
            for r0 in range(0, T, blk):
                r1 = min(T, r0 + blk)
                S = scale * (q[r0:r1] @ k[:r1].T)
                ii = np.arange(r0, r1)[:, None]
                jj = np.arange(r1)[None, :]
                S[jj > ii] = -np.inf
                m = S.max(axis=1)
                E = np.exp(S - m[:, None])
                Zs = E.sum(axis=1)
                lse[r0:r1] = m + np.log(Zs)
                o = (E / Zs[:, None]) @ v[:r1]
                delta[r0:r1] = (do[r0:r1] * o).sum(axis=1)
            if h in h_list:
                rows = []
                for i in q_rows:
                    s_i = scale * (k[: i + 1] @ q[i])
                    p = np.exp(s_i - lse[i])
                    dp = v[: i + 1] @ do[i]
                    ds = p * (dp - delta[i])
                    rows.append(scale * (ds @ k[: i + 1]))
                dQ_s[h] = np.array(rows)
            for n, j in enumerate(k_rows):
                # key j is seen by queries i >= j
                s_j = scale * (q[j:] @ k[j])
                p = np.exp(s_j - lse[j:])
                dVs[n] += p @ do[j:]
                dp = do[j:] @ v[j]
                ds = p * (dp - delta[j:])
                dKs[n] += scale * (ds @ q[j:])
        dK_s[kv] = dKs
        dV_s[kv] = dVs
    return dQ_s, dK_s, dV_s


def _packed_cu(cu_seqlens, B, T):
    cu = [int(c) for c in cu_seqlens]
    if B != 1 or cu[0] != 0 or cu[-1] != T or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("packed attention needs B = 1 and 0 = cu[0] <= ... <= cu[-1] = T")
    return cu


def attn_fwd_packed(Q, K, V, scale, cu_seqlens):
    """Forward of ``attn_bwd_packed``: ``(O, LSE)``, each sequence alone."""
    Q, K, V = _as64(Q), _as64(K), _as64(V)
    B, T, Hq, Hkv, dh, G = _check(Q, K, V)
    cu = _packed_cu(cu_seqlens, B, T)
    O = np.zeros_like(Q)
    LSE = np.zeros((B, T, Hq))
    for a, b in zip(cu, cu[1:]):
        if b > a:
            O[:, a:b], LSE[:, a:b] = attn_fwd(Q[:, a:b], K[:, a:b], V[:, a:b], scale)
    return O, LSE


def attn_bwd_packed(Q, K, V, dO, scale, cu_seqlens):
    """Causal GQA attention over packed sequences (one batch row).

    ``cu_seqlens`` holds the sequence boundaries 0 = cu[0] <= ... <= cu[n] = T;
    query i sees key j iff both lie in the same sequence and j <= i.  Each
    sequence is an independent causal attention, so the result is
    ``attn_bwd`` of every slice [cu[n], cu[n+1]) placed back in the row.
    Returns ``(dQ, dK, dV, O, LSE)`` like ``attn_bwd``.
    """
    Q, K, V, dO = _as64(Q), _as64(K), _as64(V), _as64(dO)
    B, T, Hq, Hkv, dh, G = _check(Q, K, V)
    cu = _packed_cu(cu_seqlens, B, T)
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    O = np.zeros_like(Q)
    LSE = np.zeros((B, T, Hq))
    for a, b in zip(cu, cu[1:]):
        if b == a:
            continue
        sl = slice(a, b)
        r = attn_bwd(Q[:, sl], K[:, sl], V[:, sl], dO[:, sl], scale)
        dQ[:, sl], dK[:, sl], dV[:, sl], O[:, sl], LSE[:, sl] = r
    return dQ, dK, dV, O, LSE
