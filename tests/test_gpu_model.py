"""GPU parity of the whole-model streamed backward (sbp_layer_fwd per layer,
then sbp_model_bwd) against the fp64 oracle's model backward on the same
inputs (bf16 with fp32 accumulation): normwise max|gpu - ref| / max|ref| <=
2e-2 on dx0, the final gain, the LM head and every layer gradient; the loss
relative to max(|L|, (1/N) sum |c_t| l_t).  fp32 mode: 1e-4 normwise."""
import numpy as np
import pytest
import torch

import memory_efficient_exact_amd as sbp
import oracle
import synthetic
from helpers import normwise

pytestmark = pytest.mark.gpu
TOL = 2e-2
NAMES = ("g1", "Wq", "Wk", "Wv", "Wo", "g2", "W1", "W3", "W2")


def _gpu(M, D_lm, D_layer, cu=None, accumulate=False, state=None, targets=None):
    dev = torch.device("cuda:0")
    layers = [{k: v.to(dev) for k, v in w.items()} for w in M.layers]
    c = None if cu is None else torch.tensor(cu, dtype=torch.int32, device=dev)
    xs = sbp.model_fwd(M.x0.to(dev), layers, M.Hq, M.Hkv, M.dh, M.eps, D_layer, c, M.rope_theta)
    y = (M.targets if targets is None else targets).to(dev)
    wts = None if M.weights is None else M.weights.to(dev)
    kw = {}
    if state is not None:
        kw = dict(grads=state[2], dg_final=state[3], dW_lm=state[4])
    out = sbp.model_bwd(xs, layers, M.g_final.to(dev), M.W.to(dev), y, wts, Hq=M.Hq, Hkv=M.Hkv,
                        dh=M.dh, eps=M.eps, D_lm=D_lm, D_layer=D_layer, cu_seqlens=c,
                        rope_theta=M.rope_theta, accumulate=accumulate, token_loss=True, **kw)
    torch.cuda.synchronize()
    _gpu.xs = xs
    return out


def _oracle(M, cu=None, T=None, targets=None):
    T = M.x0.shape[0] if T is None else T
    f = synthetic.to_f64
    y = (M.targets if targets is None else targets)[:T].numpy()
    wts = None if M.weights is None else f(M.weights[:T])
    return oracle.model_bwd(f(M.x0[:T]), [{k: f(v) for k, v in w.items()} for w in M.layers],
                            f(M.g_final), f(M.W), y, wts, Hq=M.Hq, Hkv=M.Hkv, dh=M.dh, eps=M.eps,
                            cu_seqlens=cu, rope_theta=M.rope_theta)


def _loss_scale(M, T=None, targets=None):
    """(1/N) sum_t |c_t| l_t from the oracle's own per-token losses."""
    T = M.x0.shape[0] if T is None else T
    f = synthetic.to_f64
    xs = oracle.model_fwd(f(M.x0[:T]), [{k: f(v) for k, v in w.items()} for w in M.layers],
                          M.Hq, M.Hkv, M.dh, M.eps, None, M.rope_theta)
    h, _, _ = oracle.rmsnorm_fwd(xs[-1], f(M.g_final), M.eps)
    y = (M.targets if targets is None else targets)[:T].numpy()
    _, _, _, tl, _ = oracle.lmhead_ce(h, f(M.W), y)
    c = np.abs(f(M.weights[:T])) if M.weights is not None else 1.0
    return float((c * tl).sum() / max(1, (y >= 0).sum()))


def _check(out, ref, scale, rows=None):
    loss, dx0, grads, dgf, dW, _ = out
    rl, rdx, rgr, rdgf, rdW = ref
    dx = dx0.float().cpu().numpy()
    if rows is not None:
        dx = dx[:rows]
    errs = {"loss": abs(loss.item() - rl) / max(abs(rl), scale), "dx0": normwise(dx, rdx),
            "dg_final": normwise(dgf.cpu().numpy(), rdgf), "dW_lm": normwise(dW.cpu().numpy(), rdW)}
    for l, g in enumerate(grads):
        for k in NAMES:
            errs[f"{l}.{k}"] = normwise(g[k].cpu().numpy(), rgr[l][k])
    print("errors:", {k: round(v, 5) for k, v in sorted(errs.items())}, flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL}
    assert not bad, errs
    return errs


@pytest.mark.parametrize("L,T,D_lm,D_layer,theta,cu,weighted", [
    (2, 300, 3, 2, 1e4, None, False),                       # ragged chunks, rotary
    (1, 257, 1, 3, 0.0, None, True),                         # weighted, no rotary
    (3, 384, 4, 4, 5e5, [0, 100, 101, 384], False),          # packed sequences
    (0, 200, 2, 3, 0.0, None, False),                        # no layers: norm + head
])
def test_parity(L, T, D_lm, D_layer, theta, cu, weighted):
    M = synthetic.model_inputs(T, 256, 4, 2, 64, 512, 1000, L, "bf16", seed=7 * T + L,
                               w_std=0.05, gain_std=0.1, rope_theta=theta, ignore_frac=0.1,
                               weighted=weighted, lm_w_std=0.1)
    out = _gpu(M, D_lm, D_layer, cu)
    ref = _oracle(M, cu)
    _check(out, ref, _loss_scale(M) if cu is None else abs(ref[0]))


def test_qk_norm_parity():
    M = synthetic.model_inputs(300, 256, 4, 2, 64, 512, 1000, 2, "bf16", seed=31, w_std=0.05,
                               gain_std=0.1, rope_theta=1e6, ignore_frac=0.1, lm_w_std=0.1,
                               qk_norm=True)
    out = _gpu(M, 3, 2)
    ref = _oracle(M)
    _check(out, ref, _loss_scale(M))
    for l, g in enumerate(out[2]):
        for k in ("qn", "kn"):
            assert normwise(g[k].cpu().numpy(), ref[2][l][k]) <= TOL, (l, k)


@pytest.mark.parametrize("L,T,D_lm,D_layer,theta,cu,qk", [
    (2, 300, 3, 2, 1e4, None, False),                       # ragged chunks, rotary
    (2, 257, 1, 257, 0.0, None, True),                       # one token per layer chunk, QK-norm
    (1, 200, 2, 3, 5e5, [0, 70, 71, 200], False),            # packed sequences
    (0, 96, 96, 2, 0.0, None, False),                        # no layers: norm + head
])
def test_parity_fp32(L, T, D_lm, D_layer, theta, cu, qk):
    """fp32 mode (every tensor and product fp32): the backward at the layer
    inputs the fp32 chunked forward gives, against the oracle's backward at
    those inputs (exact upcast), within 1e-4 normwise."""
    M = synthetic.model_inputs(T, 128, 4, 2, 64, 256, 500, L, "f32", seed=11 * T + L,
                               w_std=0.05, gain_std=0.1, rope_theta=theta, ignore_frac=0.1,
                               lm_w_std=0.1, qk_norm=qk)
    out = _gpu(M, D_lm, D_layer, cu)
    xs = [synthetic.to_f64(x.cpu()) for x in _gpu.xs]
    f = synthetic.to_f64
    ref = oracle.model_bwd_at(xs, [{k: f(v) for k, v in w.items()} for w in M.layers],
                              f(M.g_final), f(M.W), M.targets.numpy(), Hq=M.Hq, Hkv=M.Hkv,
                              dh=M.dh, eps=M.eps, cu_seqlens=cu, rope_theta=M.rope_theta)
    loss, dx0, grads, dgf, dW, _ = out
    errs = {"loss": abs(loss.item() - ref[0]) / abs(ref[0]), "dx0": normwise(dx0.cpu().numpy(), ref[1]),
            "dg_final": normwise(dgf.cpu().numpy(), ref[3]), "dW_lm": normwise(dW.cpu().numpy(), ref[4])}
    for l, g in enumerate(grads):
        for k in g:
            errs[f"{l}.{k}"] = normwise(g[k].cpu().numpy(), ref[2][l][k])
    print("errors:", {k: f"{v:.2e}" for k, v in sorted(errs.items())}, flush=True)
    bad = {k: v for k, v in errs.items() if not v <= 1e-4}
    assert not bad, errs


def test_accumulate_adds_into_every_gradient():
    M = synthetic.model_inputs(256, 128, 2, 1, 64, 256, 500, 2, "bf16", seed=5, w_std=0.05,
                               gain_std=0.1, rope_theta=1e4, lm_w_std=0.1)
    first = _gpu(M, 2, 2)
    saved = ([{k: v.clone() for k, v in g.items()} for g in first[2]], first[3].clone(),
             first[4].clone())
    second = _gpu(M, 4, 1, accumulate=True, state=first)
    for g2, g0 in zip(second[2], saved[0]):
        for k in NAMES:
            assert normwise(g2[k].cpu().numpy(), 2 * g0[k].cpu().numpy()) < 1e-2, k
    assert normwise(second[3].cpu().numpy(), 2 * saved[1].cpu().numpy()) < 1e-2
    assert normwise(second[4].cpu().numpy(), 2 * saved[2].cpu().numpy()) < 1e-2


def test_full_size_prefix():
    """The whole-model workload's shapes (4 layers of d=4096, 32/8 heads of
    128, F=14336, rotary base 5e5, LM head V=128256, T=16384) with every
    target past the first P tokens ignored.  The call's contract is the
    backward at the layer inputs it is given (here the chunked forward's bf16
    outputs): the oracle's backward at those same inputs, exactly upcast, is
    the reference.  By causality the gradients are those of the P-token
    prefix with the same N = P valid tokens; dx0 past P must be exactly zero.
    (From x0 instead, the oracle's fp64 forward and the bf16 forward drift
    apart by ~1% over four layers at this width, which is the forward's
    rounding, not the backward's.)"""
    cfg = synthetic.WORKLOADS[8]
    M = synthetic.workload_inputs(8)
    P = 64
    y = M.targets.clone()
    y[P:] = -1
    out = _gpu(M, cfg["D_lm"], cfg["D"], targets=y)
    xs = [synthetic.to_f64(x[:P].cpu()) for x in _gpu.xs]
    assert (out[1][P:] == 0).all()
    f = synthetic.to_f64
    ref = oracle.model_bwd_at(xs, [{k: f(v) for k, v in w.items()} for w in M.layers],
                              f(M.g_final), f(M.W), y[:P].numpy(), Hq=M.Hq, Hkv=M.Hkv, dh=M.dh,
                              eps=M.eps, rope_theta=M.rope_theta)
    _check(out, ref, abs(ref[0]), rows=P)


def test_full_size_forward_drift_is_bounded():
    """The same inputs end to end: the chunked bf16 forward and the backward
    against the oracle's fp64 forward and backward from x0.  This is not the
    parity test (that is the backward at the given inputs, above); it bounds
    how far the bf16 forward's rounding moves the gradients over four layers.
    Measured on MI355X: at most 2.7% normwise (on the layer gains and dK
    projections); 5e-2 is held as a regression bound."""
    cfg = synthetic.WORKLOADS[8]
    M = synthetic.workload_inputs(8)
    P = 64
    y = M.targets.clone()
    y[P:] = -1
    out = _gpu(M, cfg["D_lm"], cfg["D"], targets=y)
    ref = _oracle(M, T=P, targets=y)
    loss, dx0, grads, dgf, dW, _ = out
    errs = [normwise(dx0[:P].float().cpu().numpy(), ref[1]), normwise(dW.cpu().numpy(), ref[4])]
    errs += [normwise(g[k].cpu().numpy(), ref[2][l][k]) for l, g in enumerate(grads) for k in NAMES]
    assert max(errs) <= 5e-2, max(errs)
