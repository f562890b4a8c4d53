"""Degenerate shapes on the GPU against the oracle: a single token, a
one-word vocabulary (loss and every gradient exactly zero), and one-token
layer, forward and model calls with rotary embedding and QK-norm."""
import math

import numpy as np
import pytest
import torch

import memory_efficient_exact_amd as sbp
import oracle
import synthetic
from helpers import normwise

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = 2e-2


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_one_word_vocabulary_gives_exact_zeros(dtype):
    # softmax over one class is exactly 1: loss 0, dZ = 0, dH = 0, dW = 0
    inp = synthetic.lmhead_inputs(5, 64, 1, dtype, seed=41, w_std=0.1)
    loss, dH, dW, tl = sbp.lmhead_ce(inp.H.to(DEV), inp.W.to(DEV), inp.targets.to(DEV), D=2,
                                     token_loss=True)
    torch.cuda.synchronize()
    assert loss.item() == 0.0
    assert (dH == 0).all() and (dW == 0).all() and (tl == 0).all()
    L, rH, rW, _, _ = oracle.lmhead_ce(synthetic.to_f64(inp.H), synthetic.to_f64(inp.W),
                                       inp.targets.numpy())
    assert L == 0.0 and not rH.any() and not rW.any()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_token_lm_head(dtype):
    inp = synthetic.lmhead_inputs(1, 64, 300, dtype, seed=42, w_std=0.1)
    loss, dH, dW, _ = sbp.lmhead_ce(inp.H.to(DEV), inp.W.to(DEV), inp.targets.to(DEV), D=1)
    lp, _ = sbp.lmhead_logprob(inp.H.to(DEV), inp.W.to(DEV), inp.targets.to(DEV), D=1)
    torch.cuda.synchronize()
    L, rH, rW, _, _ = oracle.lmhead_ce(synthetic.to_f64(inp.H), synthetic.to_f64(inp.W),
                                       inp.targets.numpy())
    tol = 1e-4 if dtype == "f32" else TOL
    assert abs(loss.item() - L) <= tol * abs(L)
    assert normwise(dH.float().cpu().numpy(), rH) <= tol
    assert normwise(dW.cpu().numpy(), rW) <= tol
    assert abs(lp.item() + L) <= tol * abs(L)


def test_single_token_layer_with_rotation_and_qk_norm():
    L = synthetic.layer_inputs(1, 128, 4, 2, 64, 256, "bf16", seed=43, w_std=0.05, gain_std=0.1,
                               qk_norm=True)
    w = {k: v.to(DEV) for k, v in L.w.items()}
    dx, gr = sbp.layer_bwd(L.x.to(DEV), L.dy.to(DEV), w, L.Hq, L.Hkv, L.dh, L.eps, D=1,
                           rope_theta=1e4)
    y = sbp.layer_fwd(L.x.to(DEV), w, L.Hq, L.Hkv, L.dh, L.eps, D=1, rope_theta=1e4)
    torch.cuda.synchronize()
    f = synthetic.to_f64
    rdx, rgr, ry = oracle.layer_bwd(f(L.x), f(L.dy), {k: f(v) for k, v in L.w.items()}, L.Hq,
                                    L.Hkv, L.dh, L.eps, rope_theta=1e4)
    assert normwise(dx.float().cpu().numpy(), rdx) <= TOL
    assert normwise(y.float().cpu().numpy(), ry) <= TOL
    # one token attends only to itself: P = 1, so dS = P (dP - Delta) vanishes
    # and q, k (hence Wq, Wk, qn, kn) get no gradient, up to rounding on both
    # sides; every other gradient is compared as usual
    scale = np.abs(rgr["Wv"]).max()
    for k in rgr:
        g = gr[k].cpu().numpy()
        if k in ("Wq", "Wk", "qn", "kn"):
            assert np.abs(rgr[k]).max() <= 1e-12 * scale, k
            assert np.abs(g).max() <= 1e-3 * scale, k
        else:
            assert normwise(g, rgr[k]) <= TOL, k


def test_single_token_model():
    M = synthetic.model_inputs(1, 128, 2, 1, 64, 256, 300, 1, "bf16", seed=44, w_std=0.05,
                               gain_std=0.1, rope_theta=1e4, lm_w_std=0.1)
    layers = [{k: v.to(DEV) for k, v in w.items()} for w in M.layers]
    xs = sbp.model_fwd(M.x0.to(DEV), layers, M.Hq, M.Hkv, M.dh, M.eps, 1, None, M.rope_theta)
    loss, dx0, grads, dgf, dW, _ = sbp.model_bwd(xs, layers, M.g_final.to(DEV), M.W.to(DEV),
                                                 M.targets.to(DEV), Hq=M.Hq, Hkv=M.Hkv, dh=M.dh,
                                                 eps=M.eps, D_lm=1, D_layer=1,
                                                 rope_theta=M.rope_theta)
    torch.cuda.synchronize()
    f = synthetic.to_f64
    rl, rdx, rgr, rdg, rdW = oracle.model_bwd(f(M.x0), [{k: f(v) for k, v in w.items()}
                                                         for w in M.layers], f(M.g_final), f(M.W),
                                              M.targets.numpy(), Hq=M.Hq, Hkv=M.Hkv, dh=M.dh,
                                              eps=M.eps, rope_theta=M.rope_theta)
    assert abs(loss.item() - rl) <= TOL * abs(rl)
    assert normwise(dx0.float().cpu().numpy(), rdx) <= TOL
    assert normwise(dW.cpu().numpy(), rdW) <= TOL
    assert normwise(dgf.cpu().numpy(), rdg) <= TOL
    for k in ("Wv", "Wo", "W1", "W2", "W3", "g2"):
        assert normwise(grads[0][k].cpu().numpy(), rgr[0][k]) <= TOL, k


@pytest.mark.parametrize("d", [128, 64])
def test_target_id_beyond_vocabulary_is_loud_not_out_of_bounds(d):
    # a target id >= V is a caller error; without debug mode every read stays
    # in bounds and the error shows as NaN: the loss, dH, dW and that token's
    # loss (d = 128: fused row statistics; d = 64: the fp32 logits pass)
    inp = synthetic.lmhead_inputs(256, d, 512, "bf16", seed=44, w_std=0.05)
    inp.targets[17] = 512
    inp.targets[200] = 1 << 30
    H, W, tg = inp.H.to(DEV), inp.W.to(DEV), inp.targets.to(DEV)
    loss, dH, dW, tl = sbp.lmhead_ce(H, W, tg, D=3, token_loss=True)
    lp, ls = sbp.lmhead_logprob(H, W, tg, D=3, lse=True)
    torch.cuda.synchronize()
    assert math.isnan(loss.item())
    assert torch.isnan(dH.float()).all() and torch.isnan(dW).all()
    assert torch.isnan(tl[17]) and torch.isnan(tl[200])
    # the forward log-prob marks exactly the bad tokens
    bad = torch.zeros(256, dtype=torch.bool)
    bad[[17, 200]] = True
    assert torch.isnan(lp.cpu()[bad]).all() and torch.isnan(ls.cpu()[bad]).all()
    assert torch.isfinite(lp.cpu()[~bad]).all() and torch.isfinite(ls.cpu()[~bad]).all()
    tgt = inp.targets.clone()
    tgt[bad] = -1
    rlp, rls = oracle.lmhead_logprob(synthetic.to_f64(inp.H), synthetic.to_f64(inp.W), tgt.numpy())
    assert normwise(lp.cpu().numpy()[~bad.numpy()], rlp[~bad.numpy()]) <= TOL
