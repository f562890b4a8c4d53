"""LM head + softmax cross-entropy: loss and exact gradients, unchunked, fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources (StreamBP skill page, "StreamBP: Memory-Efficient Backpropagation"):

* "Implementation", the logits-gradient routine: per-token cross-entropy of
  the logits, then softmax of the logits with one subtracted at the target
  column.  That routine divides each chunk by its own length; that contradicts
  the "Exact Gradients" item of "Architecture Overview" and the mean loss of
  the train step on the same page, so the normaliser here is global (reading:
  divide by N, the number of non-ignored tokens, or by 1 for a plain sum).
* "Implementation", the linear-layer chunk gradient: grad_weight from the
  activations and the upstream gradient, grad_input from the upstream gradient
  and the weight.  Weights are stored [out, in] (y = x W^T), so here
  dW = dZ^T H and dH = dZ W.
* "Practical Guidance", "Loss Objectives": SFT, GRPO and DPO all feed this
  step; the per-token weight c_t carries a GRPO advantage or a DPO sequence
  weight (reading: weights multiply, the normaliser stays the token count).

Definitions, for tokens t with hidden row h_t, target y_t and weight w_t::

    Z      = H W^T                                   [T, V]
    lse_t  = log sum_v exp(Z_tv)
    l_t    = lse_t - Z_{t, y_t}                      (per-token CE)
    c_t    = w_t * [y_t >= 0]                        (y_t < 0: ignored)
    N      = #{t : y_t >= 0}  (mean_valid)   or 1  (sum)
    L      = (1/N) sum_t c_t l_t
    dZ_t   = (c_t / N) (softmax(Z_t) - e_{y_t})
    dH     = dZ W ,   dW = dZ^T H

N = 0 (every token ignored) gives L = 0, dH = 0, dW = 0 (reading; a plain
mean would be 0/0).

Forward-only per-token log-probability (``lmhead_logprob``).  The "Loss
Objectives" item of "Practical Guidance" names GRPO and DPO beside SFT; both
weight each token by a quantity formed from the log-probability the model
assigns to that token (a policy ratio, a sequence log-likelihood), which is
read here as the plain log-softmax of the logits at the target::

    logprob_t = Z_{t, y_t} - lse_t  = -l_t          (y_t >= 0)
    logprob_t = lse_t = 0                           (y_t < 0, by convention)
"""
from __future__ import annotations

import numpy as np
import torch


def _as64(a):
    return np.asarray(a, dtype=np.float64)


def _coeffs(targets, weights, reduction):
    y = np.asarray(targets).astype(np.int64)
    valid = y >= 0
    if weights is None:
        w = np.ones(y.shape[0], dtype=np.float64)
    else:
        w = _as64(weights)
    c = np.where(valid, w, 0.0)
    if reduction == "mean_valid":
        N = int(valid.sum())
    elif reduction == "sum":
        N = 1
    else:
        raise ValueError(reduction)
    return y, valid, c, N


def _logsumexp_rows(Z):
    m = Z.max(axis=1)
    return m + np.log(np.exp(Z - m[:, None]).sum(axis=1))


def lmhead_ce(H, W, targets, weights=None, reduction="mean_valid", row_block=None):
    """Loss and gradients of the weighted, masked mean cross-entropy.

    Returns ``(loss, dH, dW, token_loss, lse)``; ``token_loss[t]`` is the
    unweighted per-token CE l_t (0 for ignored tokens) and ``lse[t]`` the
    log-sum-exp of row t (NaN for ignored tokens).

    ``row_block`` only bounds host memory for large T: it evaluates the same
    full-row definition over fixed blocks of rows (independent of any chunk
    count), each softmax row complete, with dW one fp64 sum over all rows.
    """
    H = _as64(H)
    W = _as64(W)
    T, d = H.shape
    V = W.shape[0]
    y, valid, c, N = _coeffs(targets, weights, reduction)
    dH = np.zeros((T, d))
    dW = np.zeros((V, d))
    token_loss = np.zeros(T)
    lse_all = np.full(T, np.nan)
    if N == 0:
        return 0.0, dH, dW, token_loss, lse_all
    rb = T if row_block is None else int(row_block)
    total = 0.0
    for r0 in range(0, T, rb):
        r1 = min(T, r0 + rb)
        rows = np.arange(r0, r1)
        Z = H[r0:r1] @ W.T
        lse = _logsumexp_rows(Z)
        v = valid[r0:r1]
        yr = np.where(v, y[r0:r1], 0)
        z_y = Z[np.arange(r1 - r0), yr]
        ell = np.where(v, lse - z_y, 0.0)
        token_loss[r0:r1] = ell
        lse_all[r0:r1] = np.where(v, lse, np.nan)
        total += float((c[r0:r1] * ell).sum())
        P = np.exp(Z - lse[:, None])
        P[np.arange(r1 - r0)[v], yr[v]] -= 1.0
        dZ = (c[r0:r1] / N)[:, None] * P
        dZ[~v] = 0.0
        dH[rows] = dZ @ W
        dW += dZ.T @ H[r0:r1]
    return total / N, dH, dW, token_loss, lse_all


def lmhead_ce_rows(H, W, targets, weights, rows, N, reduction="mean_valid"):
    """Per-row outputs for a sample of rows, for full-size spot checks.

    Row t's logits gradient needs only Z_t = h_t W^T and the global
    normaliser N, so dH[t], l_t and lse_t can be evaluated one row at a time.
    ``N`` is the valid-token count of the whole input (ignored for 'sum').
    Returns ``(dH_rows, token_loss_rows, lse_rows)``.
    """
    W = _as64(W)
    rows = np.asarray(rows, dtype=np.int64)
    Hr = _as64(np.asarray(H)[rows])
    y = np.asarray(targets).astype(np.int64)[rows]
    w = np.ones(rows.shape[0]) if weights is None else _as64(np.asarray(weights)[rows])
    valid = y >= 0
    c = np.where(valid, w, 0.0)
    n = 1 if reduction == "sum" else N
    Z = Hr @ W.T
    lse = _logsumexp_rows(Z)
    yr = np.where(valid, y, 0)
    ell = np.where(valid, lse - Z[np.arange(len(rows)), yr], 0.0)
    P = np.exp(Z - lse[:, None])
    P[np.arange(len(rows))[valid], yr[valid]] -= 1.0
    if n == 0:
        dZ = np.zeros_like(P)
    else:
        dZ = (c / n)[:, None] * P
    dZ[~valid] = 0.0
    return dZ @ W, ell, np.where(valid, lse, np.nan)


def lmhead_dW_rows(H, W, targets, weights, vrows, reduction="mean_valid", row_block=1024):
    """Selected rows of dW at any T, for full-size spot checks.

    dW[v] = sum_t dZ_tv h_t with dZ_tv = (c_t/N)(exp(Z_tv - lse_t) - [y_t = v]).
    Column v of dZ needs lse_t of every token, and lse_t needs the whole
    logits row t, so every valid row's logits are formed over fixed blocks of
    ``row_block`` rows (a host-memory bound only, independent of any chunk
    count; each softmax row complete), but only the columns ``vrows`` of dZ
    are kept.  Rows with c_t = 0 (ignored, or weight 0) add nothing and are
    skipped.  Returns ``(dW_rows [len(vrows), d], loss, scale)`` with
    ``scale = (1/N) sum_t |c_t| l_t``, the size of the loss before signed
    weights cancel.
    """
    H = np.asarray(H)
    W = _as64(W)
    vrows = np.asarray(vrows, dtype=np.int64)
    d = W.shape[1]
    y, valid, c, N = _coeffs(targets, weights, reduction)
    out = np.zeros((vrows.shape[0], d))
    if N == 0:
        return out, 0.0, 0.0
    live = np.nonzero(c != 0.0)[0]
    total = 0.0
    total_abs = 0.0
    rb = int(row_block)
    for b0 in range(0, live.shape[0], rb):
        rows = live[b0:b0 + rb]
        Hb = _as64(H[rows])
        Z = Hb @ W.T
        # the same log-sum-exp as _logsumexp_rows, through torch's threaded
        # fp64 routine (the pass over T x V logits dominates at full size)
        lse = torch.logsumexp(torch.from_numpy(Z), dim=1).numpy()
        yb = y[rows]
        ell = lse - Z[np.arange(rows.shape[0]), yb]
        total += float((c[rows] * ell).sum())
        total_abs += float((np.abs(c[rows]) * ell).sum())
        Ps = np.exp(Z[:, vrows] - lse[:, None])            # softmax columns vrows
        del Z
        Ps -= (yb[:, None] == vrows[None, :])              # one-hot at the target
        out += (Ps * (c[rows] / N)[:, None]).T @ Hb
    return out, total / N, total_abs / N


def lmhead_logprob(H, W, targets, row_block=None):
    """Per-token target log-probability and log-sum-exp, unchunked, fp64.

    Returns ``(logprob, lse)``, both [T]: ``logprob[t] = Z_{t,y_t} - lse_t``
    and ``lse[t] = log sum_v exp(Z_tv)`` for ``y_t >= 0``; both 0 for ignored
    tokens.  ``row_block`` bounds host memory only (fixed blocks of complete
    rows, as in ``lmhead_ce``).
    """
    H = _as64(H)
    W = _as64(W)
    T = H.shape[0]
    y = np.asarray(targets).astype(np.int64)
    valid = y >= 0
    logprob = np.zeros(T)
    lse_out = np.zeros(T)
    rb = T if row_block is None else int(row_block)
    for r0 in range(0, T, rb):
        r1 = min(T, r0 + rb)
        Z = H[r0:r1] @ W.T
        lse = _logsumexp_rows(Z)
        v = valid[r0:r1]
        yr = np.where(v, y[r0:r1], 0)
        z_y = Z[np.arange(r1 - r0), yr]
        logprob[r0:r1] = np.where(v, z_y - lse, 0.0)
        lse_out[r0:r1] = np.where(v, lse, 0.0)
    return logprob, lse_out


def lmhead_logprob_rows(H, W, targets, rows):
    """``lmhead_logprob`` restricted to a sample of rows (each row needs only
    its own logits), for full-size spot checks.  Returns ``(logprob, lse)``
    for the given rows."""
    rows = np.asarray(rows, dtype=np.int64)
    return lmhead_logprob(np.asarray(H)[rows], W, np.asarray(targets)[rows])
