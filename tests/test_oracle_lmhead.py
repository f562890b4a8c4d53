"""Pins of the LM-head + cross-entropy oracle (CPU only).

Each test checks the oracle against something other than itself: hand-worked
closed forms, central finite differences of its own loss, torch's independent
fp64 cross-entropy autograd, invariants and special cases fixed by the
mathematics, and the chunked evaluation (D-invariance).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import chunked
from helpers import ev, load_golden


def _rand(T=7, d=5, V=11, seed=0, masked=True, weighted=True):
    rng = np.random.default_rng(seed)
    H = rng.normal(size=(T, d))
    W = rng.normal(size=(V, d)) * 0.7
    y = rng.integers(0, V, size=T)
    if masked:
        y[[1, 4]] = -1
    w = rng.normal(size=T) if weighted else None
    return H, W, y, w


@pytest.mark.parametrize("case", [c["name"] for c in load_golden("lmhead_ce_hand.json")["cases"]])
def test_hand_worked_golden(case):
    g = load_golden("lmhead_ce_hand.json")
    c = [c for c in g["cases"] if c["name"] == case][0]
    H, W = ev(g["H"]), ev(g["W"])
    w = None if c["weights"] is None else np.array(c["weights"])
    L, dH, dW, tl, _ = oracle.lmhead_ce(H, W, np.array(c["targets"]), w, c["reduction"])
    assert abs(L - ev(c["loss"])) < 1e-14
    np.testing.assert_allclose(tl, ev(c["token_loss"]), atol=1e-14)
    np.testing.assert_allclose(dH, ev(c["dH"]), atol=1e-14)
    np.testing.assert_allclose(dW, ev(c["dW"]), atol=1e-14)


@pytest.mark.parametrize("masked,weighted,reduction", [
    (False, False, "mean_valid"), (True, False, "mean_valid"),
    (True, True, "mean_valid"), (True, True, "sum")])
def test_finite_differences(masked, weighted, reduction):
    H, W, y, w = _rand(masked=masked, weighted=weighted)
    L, dH, dW, _, _ = oracle.lmhead_ce(H, W, y, w, reduction)
    h = 1e-6

    def loss(Hx, Wx):
        return oracle.lmhead_ce(Hx, Wx, y, w, reduction)[0]

    for A, G, which in ((H, dH, 0), (W, dW, 1)):
        fd = np.zeros_like(A)
        for idx in np.ndindex(A.shape):
            Ap, Am = A.copy(), A.copy()
            Ap[idx] += h
            Am[idx] -= h
            args_p = (Ap, W) if which == 0 else (H, Ap)
            args_m = (Am, W) if which == 0 else (H, Am)
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.abs(fd - G).max() <= 1e-7 * max(1.0, np.abs(G).max())


@pytest.mark.parametrize("weighted", [False, True])
def test_against_torch_autograd(weighted):
    H, W, y, w = _rand(T=23, d=9, V=31, seed=3, weighted=weighted)
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    yt = torch.tensor(y)
    logits = Ht @ Wt.T
    per_tok = F.cross_entropy(logits, yt.clamp_min(0), reduction="none")
    valid = (yt >= 0).to(torch.float64)
    wt = torch.ones(len(y), dtype=torch.float64) if w is None else torch.tensor(w)
    N = valid.sum()
    Lt = (per_tok * valid * wt).sum() / N
    Lt.backward()
    L, dH, dW, tl, lse = oracle.lmhead_ce(H, W, y, w)
    assert abs(L - Lt.item()) < 1e-12
    np.testing.assert_allclose(dH, Ht.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(dW, Wt.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(tl, (per_tok * valid).detach().numpy(), atol=1e-12)
    ref_lse = torch.logsumexp(logits, 1).detach().numpy()
    v = y >= 0
    np.testing.assert_allclose(lse[v], ref_lse[v], rtol=1e-13)
    assert np.isnan(lse[~v]).all()


def test_invariants():
    H, W, y, w = _rand(T=17, d=6, V=13, seed=5)
    _, dH, dW, _, _ = oracle.lmhead_ce(H, W, y, w)
    # rows of (softmax - onehot) sum to zero, so the vocab sum of dW vanishes
    assert np.abs(dW.sum(axis=0)).max() < 1e-14
    # ignored tokens contribute nothing to dH
    assert (dH[y < 0] == 0.0).all()


def test_zero_weight_matrix_closed_form():
    # W = 0: every softmax is uniform, L = ln V (mean of unweighted CE),
    # dH = dZ W = 0, dW = sum_t (c_t/N)(1/V - e_{y_t}) h_t^T.
    T, d, V = 9, 4, 6
    rng = np.random.default_rng(11)
    H = rng.normal(size=(T, d))
    W = np.zeros((V, d))
    y = rng.integers(0, V, size=T)
    L, dH, dW, _, _ = oracle.lmhead_ce(H, W, y)
    assert abs(L - math.log(V)) < 1e-14
    assert (dH == 0).all()
    ref = np.zeros((V, d))
    for t in range(T):
        for v in range(V):
            ref[v] += (1.0 / T) * ((1.0 / V) - (1.0 if v == y[t] else 0.0)) * H[t]
    np.testing.assert_allclose(dW, ref, atol=1e-15)


def test_all_ignored_gives_zeros():
    H, W, y, w = _rand()
    y[:] = -1
    L, dH, dW, tl, lse = oracle.lmhead_ce(H, W, y, w)
    assert L == 0.0 and (dH == 0).all() and (dW == 0).all() and (tl == 0).all()


def test_row_blocking_matches_unblocked():
    H, W, y, w = _rand(T=37, d=6, V=19, seed=7)
    a = oracle.lmhead_ce(H, W, y, w)
    b = oracle.lmhead_ce(H, W, y, w, row_block=5)
    assert abs(a[0] - b[0]) < 1e-13
    for x, z in zip(a[1:4], b[1:4]):
        assert np.abs(x - z).max() < 1e-13


def test_sampled_rows_match_full():
    H, W, y, w = _rand(T=29, d=6, V=19, seed=8)
    _, dH, _, tl, lse = oracle.lmhead_ce(H, W, y, w)
    rows = np.array([0, 1, 4, 13, 28])
    N = int((y >= 0).sum())
    dHr, tlr, lser = oracle.lmhead_ce_rows(H, W, y, w, rows, N)
    np.testing.assert_allclose(dHr, dH[rows], atol=1e-15)
    np.testing.assert_allclose(tlr, tl[rows], atol=1e-15)
    np.testing.assert_array_equal(np.isnan(lser), np.isnan(lse[rows]))


@pytest.mark.parametrize("reduction", ["mean_valid", "sum"])
@pytest.mark.parametrize("row_block", [1, 4, 1024])
def test_sampled_dW_rows_match_full(reduction, row_block):
    # selected vocab rows of dW, every row's lse over blocks of rows, against
    # the full gradient; rows 0 and V-1 and one that is the target of many
    # tokens (its one-hot term is summed over all of them)
    H, W, y, w = _rand(T=41, d=6, V=23, seed=21)
    y[::3] = 7
    vrows = np.array([0, 7, 11, 22, 7])
    L, _, dW, tl, _ = oracle.lmhead_ce(H, W, y, w, reduction)
    dWr, Lr, Sr = oracle.lmhead_dW_rows(H, W, y, w, vrows, reduction, row_block=row_block)
    np.testing.assert_allclose(dWr, dW[vrows], rtol=0, atol=1e-14)
    assert abs(Lr - L) < 1e-12
    N = int((y >= 0).sum()) if reduction == "mean_valid" else 1
    assert abs(Sr - float((np.abs(np.where(y >= 0, w, 0.0)) * tl).sum()) / N) < 1e-12


def test_sampled_dW_rows_zero_weights_and_all_ignored():
    H, W, y, w = _rand(T=20, d=5, V=9, seed=22)
    w[:10] = 0.0
    _, _, dW, _, _ = oracle.lmhead_ce(H, W, y, w)
    dWr, _, _ = oracle.lmhead_dW_rows(H, W, y, w, np.arange(9), row_block=3)
    np.testing.assert_allclose(dWr, dW, rtol=0, atol=1e-14)
    y[:] = -1
    dWr, Lr, Sr = oracle.lmhead_dW_rows(H, W, y, w, np.arange(9))
    assert Lr == 0.0 and Sr == 0.0 and (dWr == 0).all()


@pytest.mark.parametrize("T,D", [(13, 1), (13, 2), (13, 3), (13, 13), (64, 5)])
def test_chunked_equals_unchunked(T, D):
    H, W, y, w = _rand(T=T, d=6, V=17, seed=T + D)
    L, dH, dW, _, _ = oracle.lmhead_ce(H, W, y, w)
    L2, dH2, dW2 = chunked.lmhead_ce(H, W, y, w, D)
    assert abs(L - L2) < 1e-12
    assert np.abs(dH - dH2).max() < 1e-12
    assert np.abs(dW - dW2).max() < 1e-12


def test_chunk_table_rule():
    # size = T // D, the last chunk takes the remainder
    assert chunked.chunk_table(10, 3) == [(0, 3), (3, 6), (6, 10)]
    assert chunked.chunk_table(5, 5) == [(i, i + 1) for i in range(5)]
    assert chunked.chunk_table(7, 1) == [(0, 7)]
    for bad in ((5, 0), (5, 6)):
        with pytest.raises(ValueError):
            chunked.chunk_table(*bad)


# ---------------------------------------------------------------------------
# Forward-only per-token log-probability (GRPO / DPO front end)

@pytest.mark.parametrize("case", [c["name"] for c in load_golden("lmhead_logprob_hand.json")["cases"]])
def test_logprob_hand_worked_golden(case):
    g = load_golden("lmhead_logprob_hand.json")
    c = [c for c in g["cases"] if c["name"] == case][0]
    lp, lse = oracle.lmhead_logprob(ev(g["H"]), ev(g["W"]), np.array(c["targets"]))
    np.testing.assert_allclose(lp, ev(c["logprob"]), atol=1e-15)
    np.testing.assert_allclose(lse, ev(c["lse"]), atol=1e-15)


def test_logprob_normalises_over_the_vocabulary():
    # every row's probabilities exp(logprob) over all V possible targets sum
    # to one, and each is at most one
    T, d, V = 5, 4, 9
    rng = np.random.default_rng(21)
    H = rng.normal(size=(T, d)) * 2.0
    W = rng.normal(size=(V, d))
    Hrep = np.repeat(H, V, axis=0)
    y = np.tile(np.arange(V), T)
    lp, lse = oracle.lmhead_logprob(Hrep, W, y)
    assert (lp <= 0).all()
    np.testing.assert_allclose(np.exp(lp).reshape(T, V).sum(axis=1), 1.0, atol=1e-14)
    # lse does not depend on the target
    assert np.ptp(lse.reshape(T, V), axis=1).max() < 1e-13


def test_logprob_zero_weight_matrix_is_uniform():
    T, d, V = 6, 3, 7
    rng = np.random.default_rng(22)
    y = rng.integers(0, V, size=T)
    y[2] = -1
    lp, lse = oracle.lmhead_logprob(rng.normal(size=(T, d)), np.zeros((V, d)), y)
    v = y >= 0
    np.testing.assert_allclose(lp[v], -math.log(V), atol=1e-15)
    np.testing.assert_allclose(lse[v], math.log(V), atol=1e-15)
    assert lp[2] == 0.0 and lse[2] == 0.0


def test_logprob_against_torch_log_softmax():
    H, W, y, _ = _rand(T=23, d=6, V=31, seed=23)
    lp, lse = oracle.lmhead_logprob(H, W, y)
    Z = torch.from_numpy(H) @ torch.from_numpy(W).T
    ls = F.log_softmax(Z, dim=1)
    v = y >= 0
    ref = ls[torch.arange(len(y)), torch.from_numpy(np.where(v, y, 0))].numpy()
    np.testing.assert_allclose(lp[v], ref[v], atol=1e-13)
    np.testing.assert_allclose(lse[v], torch.logsumexp(Z, dim=1).numpy()[v], atol=1e-13)
    assert (lp[~v] == 0).all() and (lse[~v] == 0).all()


def test_logprob_shift_of_all_logits():
    # a constant added to every logit of a row leaves the log-probability
    # unchanged and moves lse by the constant: with a column of ones in H,
    # adding k to that column of W adds k to every logit
    H, W, y, _ = _rand(T=11, d=5, V=13, seed=24)
    H[:, 0] = 1.0
    W2 = W.copy()
    W2[:, 0] += 3.25
    lp, lse = oracle.lmhead_logprob(H, W, y)
    lp2, lse2 = oracle.lmhead_logprob(H, W2, y)
    v = y >= 0
    np.testing.assert_allclose(lp2, lp, atol=1e-13)
    np.testing.assert_allclose(lse2[v], lse[v] + 3.25, atol=1e-13)


def test_logprob_is_minus_token_cross_entropy():
    # the pinned cross-entropy oracle's per-token loss is -logprob
    H, W, y, w = _rand(T=19, d=6, V=17, seed=25)
    lp, lse = oracle.lmhead_logprob(H, W, y)
    _, _, _, tl, lse_ce = oracle.lmhead_ce(H, W, y, w)
    np.testing.assert_allclose(lp, -tl, atol=1e-14)
    v = y >= 0
    np.testing.assert_allclose(lse[v], lse_ce[v], atol=1e-14)


def test_logprob_rows_and_blocking():
    H, W, y, _ = _rand(T=29, d=6, V=19, seed=26)
    lp, lse = oracle.lmhead_logprob(H, W, y)
    lpb, lseb = oracle.lmhead_logprob(H, W, y, row_block=4)
    assert np.abs(lp - lpb).max() < 1e-13 and np.abs(lse - lseb).max() < 1e-13
    rows = np.array([0, 1, 4, 13, 28])
    lpr, lser = oracle.lmhead_logprob_rows(H, W, y, rows)
    np.testing.assert_allclose(lpr, lp[rows], atol=1e-15)
    np.testing.assert_allclose(lser, lse[rows], atol=1e-15)
