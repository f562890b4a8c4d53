"""Pins of the causal GQA attention oracle (CPU only)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import chunked
from helpers import ev, load_golden


def _rand(B=2, T=9, Hq=4, Hkv=2, dh=4, seed=0):
    rng = np.random.default_rng(seed)
    Q = rng.normal(size=(B, T, Hq, dh))
    K = rng.normal(size=(B, T, Hkv, dh))
    V = rng.normal(size=(B, T, Hkv, dh))
    dO = rng.normal(size=(B, T, Hq, dh))
    return Q, K, V, dO


def test_hand_worked_golden():
    g = load_golden("attention_hand.json")
    sh = (1, 2, 1, 1)
    Q, K, V, dO = (ev(g[k]).reshape(sh) for k in ("Q", "K", "V", "dO"))
    dQ, dK, dV, O, LSE = oracle.attn_bwd(Q, K, V, dO, ev(g["scale"]))
    np.testing.assert_allclose(O.ravel(), ev(g["O"]), atol=1e-14)
    np.testing.assert_allclose(LSE.ravel(), ev(g["LSE"]), atol=1e-14)
    np.testing.assert_allclose(dQ.ravel(), ev(g["dQ"]), atol=1e-14)
    np.testing.assert_allclose(dK.ravel(), ev(g["dK"]), atol=1e-14)
    np.testing.assert_allclose(dV.ravel(), ev(g["dV"]), atol=1e-14)


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (4, 1), (3, 3)])
def test_against_torch_sdpa(Hq, Hkv):
    Q, K, V, dO = _rand(B=2, T=17, Hq=Hq, Hkv=Hkv, dh=8, seed=Hq * 10 + Hkv)
    s = 0.37
    # torch wants [B, H, T, dh]
    tq, tk, tv = (torch.tensor(a.transpose(0, 2, 1, 3), requires_grad=True) for a in (Q, K, V))
    out = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=s,
                                         enable_gqa=(Hq != Hkv))
    out.backward(torch.tensor(dO.transpose(0, 2, 1, 3)))
    dQ, dK, dV, O, _ = oracle.attn_bwd(Q, K, V, dO, s)
    tr = lambda t: t.detach().numpy().transpose(0, 2, 1, 3)
    np.testing.assert_allclose(O, tr(out), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dQ, tr(tq.grad), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dK, tr(tk.grad), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dV, tr(tv.grad), rtol=1e-11, atol=1e-12)


def test_finite_differences():
    # f = <dO, O>, so df/dX is the oracle's gradient
    Q, K, V, dO = _rand(B=2, T=9, Hq=4, Hkv=2, dh=4, seed=4)
    s = 0.5
    dQ, dK, dV, _, _ = oracle.attn_bwd(Q, K, V, dO, s)
    h = 1e-6

    def f(q, k, v):
        return float((oracle.attn_fwd(q, k, v, s)[0] * dO).sum())

    for which, A, G in ((0, Q, dQ), (1, K, dK), (2, V, dV)):
        fd = np.zeros_like(A)
        for idx in np.ndindex(A.shape):
            Ap, Am = A.copy(), A.copy()
            Ap[idx] += h
            Am[idx] -= h
            ap = [Q, K, V]
            am = [Q, K, V]
            ap[which], am[which] = Ap, Am
            fd[idx] = (f(*ap) - f(*am)) / (2 * h)
        assert np.abs(fd - G).max() <= 1e-7 * max(1.0, np.abs(G).max())


def test_key_gradient_sums_to_zero():
    # rows of dS sum to zero, so sum_j dK_j = s * dS^T Q summed over j is 0
    Q, K, V, dO = _rand(B=1, T=21, seed=9)
    _, dK, _, _, _ = oracle.attn_bwd(Q, K, V, dO, 0.3)
    assert np.abs(dK.sum(axis=1)).max() < 1e-12


def test_single_token():
    Q, K, V, dO = _rand(B=2, T=1, Hq=4, Hkv=2, seed=2)
    dQ, dK, dV, O, _ = oracle.attn_bwd(Q, K, V, dO, 0.5)
    # dS = P (dP - delta) vanishes up to the rounding of two equal dot products
    assert np.abs(dQ).max() < 1e-15 and np.abs(dK).max() < 1e-15
    G = 2
    ref = dO.reshape(2, 1, 2, G, 4).sum(axis=3)
    np.testing.assert_allclose(dV, ref, atol=1e-15)
    np.testing.assert_allclose(O, np.repeat(V, G, axis=2), atol=1e-15)


def test_zero_queries_uniform_weights():
    # Q = 0: weights uniform over the causal prefix
    B, T, Hq, Hkv, dh = 1, 7, 2, 1, 3
    _, K, V, dO = _rand(B, T, Hq, Hkv, dh, seed=6)
    Q = np.zeros((B, T, Hq, dh))
    _, _, dV, O, _ = oracle.attn_bwd(Q, K, V, dO, 1.0)
    for i in range(T):
        np.testing.assert_allclose(O[0, i, 0], V[0, : i + 1, 0].mean(axis=0), atol=1e-14)
    ref = np.zeros((T, dh))
    for j in range(T):
        for i in range(j, T):
            ref[j] += dO[0, i].sum(axis=0) / (i + 1)
    np.testing.assert_allclose(dV[0, :, 0], ref, atol=1e-14)


def test_gqa_equals_mha_with_repeated_heads():
    Q, K, V, dO = _rand(B=1, T=8, Hq=6, Hkv=2, dh=4, seed=12)
    G = 3
    Kr, Vr = np.repeat(K, G, axis=2), np.repeat(V, G, axis=2)
    a = oracle.attn_bwd(Q, K, V, dO, 0.4)
    b = oracle.attn_bwd(Q, Kr, Vr, dO, 0.4)
    np.testing.assert_allclose(a[0], b[0], atol=1e-14)
    np.testing.assert_allclose(a[1], b[1].reshape(1, 8, 2, G, 4).sum(3), atol=1e-13)
    np.testing.assert_allclose(a[2], b[2].reshape(1, 8, 2, G, 4).sum(3), atol=1e-13)


@pytest.mark.parametrize("D", [1, 2, 3, 9])
def test_chunked_equals_unchunked(D):
    Q, K, V, dO = _rand(B=2, T=9, seed=D)
    a = oracle.attn_bwd(Q, K, V, dO, 0.45)
    b = chunked.attn_bwd(Q, K, V, dO, 0.45, D)
    for x, y in zip(a[:3], b):
        assert np.abs(x - y).max() < 1e-12


def test_sampled_matches_full():
    Q, K, V, dO = _rand(B=2, T=40, Hq=4, Hkv=2, dh=5, seed=13)
    dQ, dK, dV, _, _ = oracle.attn_bwd(Q, K, V, dO, 0.3)
    qr, kr = [0, 5, 39], [0, 17, 39]
    dQs, dKs, dVs = oracle.attn_bwd_sampled(Q, K, V, dO, 0.3, 1, [1, 2], qr, kr)
    for h in (1, 2):
        np.testing.assert_allclose(dQs[h], dQ[1, qr, h], atol=1e-13)
    for kv in (0, 1):
        np.testing.assert_allclose(dKs[kv], dK[1, kr, kv], atol=1e-13)
        np.testing.assert_allclose(dVs[kv], dV[1, kr, kv], atol=1e-13)


# ---------------------------------------------------------------------------
# Packed independent sequences (block-diagonal causal mask)

def _packed_mask(cu, T):
    seq = np.zeros(T, dtype=np.int64)
    for n, (a, b) in enumerate(zip(cu, cu[1:])):
        seq[a:b] = n
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    return (j <= i) & (seq[:, None] == seq[None, :])


@pytest.mark.parametrize("cu,Hq,Hkv", [([0, 5, 6, 13, 19], 4, 2), ([0, 19], 2, 2),
                                        ([0, 1, 2, 3, 10, 19], 3, 1), ([0, 4, 4, 19], 4, 4)])
def test_packed_against_torch_sdpa_with_block_mask(cu, Hq, Hkv):
    Q, K, V, dO = _rand(B=1, T=19, Hq=Hq, Hkv=Hkv, dh=8, seed=len(cu) + Hq)
    s = 0.41
    mask = torch.tensor(_packed_mask(cu, 19))
    tq, tk, tv = (torch.tensor(a.transpose(0, 2, 1, 3), requires_grad=True) for a in (Q, K, V))
    out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=s,
                                         enable_gqa=(Hq != Hkv))
    out.backward(torch.tensor(dO.transpose(0, 2, 1, 3)))
    dQ, dK, dV, O, _ = oracle.attn_bwd_packed(Q, K, V, dO, s, cu)
    tr = lambda t: t.detach().numpy().transpose(0, 2, 1, 3)
    np.testing.assert_allclose(O, tr(out), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dQ, tr(tq.grad), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dK, tr(tk.grad), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dV, tr(tv.grad), rtol=1e-11, atol=1e-12)


def test_packed_finite_differences():
    cu = [0, 3, 4, 9]
    Q, K, V, dO = _rand(B=1, T=9, Hq=2, Hkv=1, dh=3, seed=41)
    s = 0.6
    dQ, dK, dV, _, _ = oracle.attn_bwd_packed(Q, K, V, dO, s, cu)
    mask = _packed_mask(cu, 9)

    def f(q, k, v):
        # <dO, O> with the block-diagonal causal mask written out directly
        tot = 0.0
        for h in range(2):
            S = s * (q[0, :, h] @ k[0, :, 0].T)
            S = np.where(mask, S, -np.inf)
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            tot += float(((P @ v[0, :, 0]) * dO[0, :, h]).sum())
        return tot

    h = 1e-6
    for which, A, G in ((0, Q, dQ), (1, K, dK), (2, V, dV)):
        fd = np.zeros_like(A)
        for idx in np.ndindex(A.shape):
            ap, am = [Q, K, V], [Q, K, V]
            Ap, Am = A.copy(), A.copy()
            Ap[idx] += h
            Am[idx] -= h
            ap[which], am[which] = Ap, Am
            fd[idx] = (f(*ap) - f(*am)) / (2 * h)
        assert np.abs(fd - G).max() <= 1e-7 * max(1.0, np.abs(G).max())


def test_packed_one_sequence_is_causal_and_cross_sequence_independent():
    Q, K, V, dO = _rand(B=1, T=12, seed=42)
    a = oracle.attn_bwd_packed(Q, K, V, dO, 0.5, [0, 12])
    b = oracle.attn_bwd(Q, K, V, dO, 0.5)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    # changing the second sequence leaves the first one's gradients alone
    cu = [0, 5, 12]
    r1 = oracle.attn_bwd_packed(Q, K, V, dO, 0.5, cu)
    K2 = K.copy()
    K2[:, 5:] += 1.0
    r2 = oracle.attn_bwd_packed(Q, K2, V, dO, 0.5, cu)
    for x, y in zip(r1[:3], r2[:3]):
        np.testing.assert_array_equal(x[:, :5], y[:, :5])
