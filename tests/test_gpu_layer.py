"""GPU parity of sbp_layer_bwd against the fp64 oracle (bf16, fp32
accumulation): normwise max|gpu - ref| / max|ref| <= 2e-2 on dx and on every
weight and gain gradient."""
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


def _gpu(L, D, grads=None, accumulate=False, dy=None):
    dev = torch.device("cuda:0")
    w = {k: v.to(dev) for k, v in L.w.items()}
    dyd = (L.dy if dy is None else dy).to(dev)
    dx, gr = sbp.layer_bwd(L.x.to(dev), dyd, w, L.Hq, L.Hkv, L.dh, L.eps, D=D, grads=grads,
                           accumulate=accumulate)
    torch.cuda.synchronize()
    return dx, gr


def _oracle(L, T=None, dy=None):
    T = L.x.shape[0] if T is None else T
    dyv = L.dy if dy is None else dy
    w = {k: synthetic.to_f64(v) for k, v in L.w.items()}
    return oracle.layer_bwd(synthetic.to_f64(L.x[:T]), synthetic.to_f64(dyv[:T]), w, L.Hq, L.Hkv,
                            L.dh, L.eps)


def _check(dx, gr, rdx, rgr, tol=TOL):
    errs = {"dx": normwise(dx.float().cpu().numpy(), rdx)}
    for k in NAMES:
        errs[k] = normwise(gr[k].cpu().numpy(), rgr[k])
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, errs
    return errs


@pytest.mark.parametrize("T,d,Hq,Hkv,dh,F,D", [
    (300, 256, 4, 2, 64, 512, 3),     # ragged chunks, GQA
    (512, 512, 8, 2, 128, 1024, 4),   # dh 128
    (257, 128, 2, 1, 64, 256, 1),     # one chunk, MQA
    (64, 64, 2, 2, 64, 128, 64),      # D = T
    (1000, 256, 4, 4, 128, 768, 7),   # MHA, several key tiles per chunk
])
def test_parity(T, d, Hq, Hkv, dh, F, D):
    L = synthetic.layer_inputs(T, d, Hq, Hkv, dh, F, "bf16", seed=T + d + D, w_std=0.05,
                               gain_std=0.1)
    dx, gr = _gpu(L, D)
    rdx, rgr, _ = _oracle(L)
    _check(dx, gr, rdx, rgr)


def test_accumulate_adds_into_grads():
    L = synthetic.layer_inputs(256, 128, 2, 1, 64, 256, "bf16", seed=3, w_std=0.05, gain_std=0.1)
    dx1, g1 = _gpu(L, 2)
    g0 = {k: v.clone() for k, v in g1.items()}
    dx2, g2 = _gpu(L, 4, grads=g1, accumulate=True)
    for k in NAMES:
        assert normwise(g2[k].cpu().numpy(), 2 * g0[k].cpu().numpy()) < 1e-2, k
    assert normwise(dx2.float().cpu().numpy(), dx1.float().cpu().numpy()) < 1e-2


def test_gpu_D_invariance():
    L = synthetic.layer_inputs(1024, 256, 4, 2, 128, 512, "bf16", seed=9, w_std=0.05, gain_std=0.1)
    base = _gpu(L, 1)
    for D in (2, 8):
        dx, gr = _gpu(L, D)
        assert normwise(dx.float().cpu().numpy(), base[0].float().cpu().numpy()) < 1e-2
        for k in NAMES:
            assert normwise(gr[k].cpu().numpy(), base[1][k].cpu().numpy()) < 1e-2, k


def test_zero_output_projections_give_identity():
    # Wo = W2 = 0: y = x, so dx = dy exactly and only dWo, dW2 are non-zero
    L = synthetic.layer_inputs(300, 128, 2, 1, 64, 256, "bf16", seed=4, w_std=0.05, gain_std=0.1)
    L.w["Wo"] = torch.zeros_like(L.w["Wo"])
    L.w["W2"] = torch.zeros_like(L.w["W2"])
    dx, gr = _gpu(L, 3)
    assert torch.equal(dx.cpu(), L.dy)
    for k in ("Wq", "Wk", "Wv", "W1", "W3", "g1", "g2"):
        assert (gr[k] == 0).all(), k
    rdx, rgr, _ = _oracle(L)
    assert normwise(gr["Wo"].cpu().numpy(), rgr["Wo"]) <= TOL
    assert normwise(gr["W2"].cpu().numpy(), rgr["W2"]) <= TOL


def test_full_size_T65536_prefix():
    """The decoder-layer workload at its full size (T=65536, d=4096, 32/8
    heads of 128, F=14336, D=16), with the upstream gradient zero beyond the
    first P tokens.  Causality makes every gradient equal to that of the
    P-token prefix alone (later tokens neither feed the prefix forward nor,
    with zero upstream, carry any gradient), so the fp64 oracle on P tokens is
    the exact reference; dx beyond P must be exactly zero."""
    cfg = synthetic.WORKLOADS[3]
    L = synthetic.workload_inputs(3)
    P = 128
    dy = L.dy.clone()
    dy[P:] = 0
    dx, gr = _gpu(L, cfg["D"], dy=dy)
    assert (dx[P:] == 0).all()
    rdx, rgr, _ = _oracle(L, T=P, dy=dy)
    _check(dx[:P], gr, rdx, rgr)


def test_full_width_dense_upstream_T4096():
    """The decoder-layer workload's full width (d=4096, 32/8 heads of 128,
    F=14336) at T=4096 with D=16 and a dense N(0,1) upstream gradient on
    every token: all 16 chunks add live gradients into dK/dV and every fp32
    weight and gain gradient, compared element by element with the fp64
    oracle on the whole sequence."""
    L = synthetic.layer_inputs(4096, 4096, 32, 8, 128, 14336, "bf16", seed=4096, w_std=0.02,
                               gain_std=0.1)
    dx, gr = _gpu(L, 16)
    rdx, rgr, _ = _oracle(L)
    _check(dx, gr, rdx, rgr)


# ---- packed independent sequences (sbp_layer_bwd_packed) -----------------
def _gpu_packed(L, D, cu, grads=None, accumulate=False):
    dev = torch.device("cuda:0")
    w = {k: v.to(dev) for k, v in L.w.items()}
    c = torch.tensor(cu, dtype=torch.int32, device=dev)
    dx, gr = sbp.layer_bwd(L.x.to(dev), L.dy.to(dev), w, L.Hq, L.Hkv, L.dh, L.eps, D=D,
                           grads=grads, accumulate=accumulate, cu_seqlens=c)
    torch.cuda.synchronize()
    return dx, gr


def _oracle_packed(L, cu):
    w = {k: synthetic.to_f64(v) for k, v in L.w.items()}
    return oracle.layer_bwd(synthetic.to_f64(L.x), synthetic.to_f64(L.dy), w, L.Hq, L.Hkv, L.dh,
                            L.eps, cu_seqlens=cu)


@pytest.mark.parametrize("T,d,Hq,Hkv,dh,F,D,cu", [
    (300, 256, 4, 2, 64, 512, 3, [0, 41, 42, 170, 300]),      # cuts inside tiles and chunks
    (512, 512, 8, 2, 128, 1024, 4, [0, 128, 256, 384, 512]),  # tile-aligned sequences
    (640, 256, 4, 1, 128, 512, 5, [0, 1, 1, 333, 639, 640]),  # empty and one-token sequences
])
def test_packed_parity(T, d, Hq, Hkv, dh, F, D, cu):
    L = synthetic.layer_inputs(T, d, Hq, Hkv, dh, F, "bf16", seed=2 * T + d + D, w_std=0.05,
                               gain_std=0.1)
    dx, gr = _gpu_packed(L, D, cu)
    rdx, rgr, _ = _oracle_packed(L, cu)
    _check(dx, gr, rdx, rgr)


def test_packed_one_sequence_equals_layer_call():
    L = synthetic.layer_inputs(384, 256, 4, 2, 64, 512, "bf16", seed=12, w_std=0.05, gain_std=0.1)
    dx, gr = _gpu(L, 3)
    dxp, grp = _gpu_packed(L, 3, [0, 384])
    assert torch.equal(dx, dxp)
    for k in NAMES:
        assert torch.equal(gr[k], grp[k]), k


# ---- rotary embedding of q and k (rope_theta > 0) -------------------------
def _gpu_rope(L, D, theta, cu=None, dy=None):
    dev = torch.device("cuda:0")
    w = {k: v.to(dev) for k, v in L.w.items()}
    c = None if cu is None else torch.tensor(cu, dtype=torch.int32, device=dev)
    dyd = (L.dy if dy is None else dy).to(dev)
    dx, gr = sbp.layer_bwd(L.x.to(dev), dyd, w, L.Hq, L.Hkv, L.dh, L.eps, D=D, cu_seqlens=c,
                           rope_theta=theta)
    torch.cuda.synchronize()
    return dx, gr


def _oracle_rope(L, theta, cu=None, T=None, dy=None):
    T = L.x.shape[0] if T is None else T
    dyv = L.dy if dy is None else dy
    w = {k: synthetic.to_f64(v) for k, v in L.w.items()}
    return oracle.layer_bwd(synthetic.to_f64(L.x[:T]), synthetic.to_f64(dyv[:T]), w, L.Hq, L.Hkv,
                            L.dh, L.eps, cu_seqlens=cu, rope_theta=theta)


@pytest.mark.parametrize("T,d,Hq,Hkv,dh,F,D,theta,cu", [
    (300, 256, 4, 2, 64, 512, 3, 10000.0, None),                      # ragged chunks, dh 64
    (512, 512, 8, 2, 128, 1024, 4, 1e6, None),                        # dh 128, large base
    (1000, 256, 4, 1, 128, 512, 7, 500.0, None),                      # MQA, fast rotation
    (640, 256, 4, 2, 128, 512, 5, 10000.0, [0, 1, 1, 333, 639, 640]),  # packed: positions restart
])
def test_rope_parity(T, d, Hq, Hkv, dh, F, D, theta, cu):
    L = synthetic.layer_inputs(T, d, Hq, Hkv, dh, F, "bf16", seed=3 * T + d + D, w_std=0.05,
                               gain_std=0.1)
    dx, gr = _gpu_rope(L, D, theta, cu)
    rdx, rgr, _ = _oracle_rope(L, theta, cu)
    _check(dx, gr, rdx, rgr)


def test_rope_long_row():
    """T = 4096 with a base of 1e4: the fastest pair turns by ~4095 rad at the
    last position, where the table's angle reduction matters."""
    L = synthetic.layer_inputs(4096, 256, 4, 2, 128, 512, "bf16", seed=77, w_std=0.05,
                               gain_std=0.1)
    dx, gr = _gpu_rope(L, 4, 1e4)
    rdx, rgr, _ = _oracle_rope(L, 1e4)
    _check(dx, gr, rdx, rgr)


def test_rope_full_size_T65536_prefix():
    """Workload-3 shapes with rotary embedding (base 1e6), upstream gradient
    zero beyond the first P tokens: the P-token prefix backward is exact."""
    cfg = synthetic.WORKLOADS[3]
    L = synthetic.workload_inputs(3)
    P = 128
    dy = L.dy.clone()
    dy[P:] = 0
    dx, gr = _gpu_rope(L, cfg["D"], 1e6, dy=dy)
    assert (dx[P:] == 0).all()
    rdx, rgr, _ = _oracle_rope(L, 1e6, T=P, dy=dy)
    _check(dx[:P], gr, rdx, rgr)


# ---- QK-norm: per-head RMSNorm of q and k (gains qn, kn) -----------------
@pytest.mark.parametrize("T,d,Hq,Hkv,dh,F,D,theta,cu", [
    (300, 256, 4, 2, 64, 512, 3, 1e4, None),                          # dh 64, rotary
    (512, 512, 8, 2, 128, 1024, 4, 0.0, None),                        # no rotation
    (640, 256, 4, 2, 128, 512, 5, 1e6, [0, 1, 1, 333, 639, 640]),      # packed
])
def test_qk_norm_parity(T, d, Hq, Hkv, dh, F, D, theta, cu):
    L = synthetic.layer_inputs(T, d, Hq, Hkv, dh, F, "bf16", seed=11 * T + d + D, w_std=0.05,
                               gain_std=0.1, qk_norm=True)
    dx, gr = _gpu_rope(L, D, theta, cu)
    rdx, rgr, _ = _oracle_rope(L, theta, cu)
    _check(dx, gr, rdx, rgr)
    for k in ("qn", "kn"):
        assert normwise(gr[k].cpu().numpy(), rgr[k]) <= TOL, k


def test_qk_norm_full_size_T65536_prefix():
    """Workload-3 shapes with QK-norm and rotary embedding (base 1e6), upstream
    gradient zero beyond the first P tokens: the P-token prefix is exact."""
    cfg = synthetic.WORKLOADS[3]
    L = synthetic.layer_inputs(cfg["T"], cfg["d"], cfg["Hq"], cfg["Hkv"], cfg["dh"], cfg["F"],
                               "bf16", seed=1003, gain_std=0.1, qk_norm=True)
    P = 128
    dy = L.dy.clone()
    dy[P:] = 0
    dx, gr = _gpu_rope(L, cfg["D"], 1e6, dy=dy)
    assert (dx[P:] == 0).all()
    rdx, rgr, _ = _oracle_rope(L, 1e6, T=P, dy=dy)
    _check(dx[:P], gr, rdx, rgr)
    for k in ("qn", "kn"):
        assert normwise(gr[k].cpu().numpy(), rgr[k]) <= TOL, k


# ---- fp32 mode: every tensor and product fp32, normwise <= 1e-4 -----------
TOL_F32 = 1e-4


@pytest.mark.parametrize("T,d,Hq,Hkv,dh,F,D,theta,qk,cu", [
    (300, 256, 4, 2, 64, 512, 3, 0.0, False, None),                    # ragged chunks, GQA
    (257, 128, 2, 1, 128, 256, 1, 0.0, False, None),                   # one chunk, MQA, dh 128
    (64, 64, 2, 2, 64, 128, 64, 0.0, False, None),                     # D = T
    (400, 256, 4, 2, 128, 512, 4, 1e4, True, None),                    # rotary + QK-norm
    (640, 256, 4, 2, 64, 512, 5, 1e4, False, [0, 1, 1, 333, 639, 640]),  # packed, rotary
])
def test_parity_fp32(T, d, Hq, Hkv, dh, F, D, theta, qk, cu):
    L = synthetic.layer_inputs(T, d, Hq, Hkv, dh, F, "f32", seed=5 * T + d + D, w_std=0.05,
                               gain_std=0.1, qk_norm=qk)
    dx, gr = _gpu_rope(L, D, theta, cu)
    assert dx.dtype == torch.float32
    rdx, rgr, _ = _oracle_rope(L, theta, cu)
    _check(dx, gr, rdx, rgr, tol=TOL_F32)
    if qk:
        for k in ("qn", "kn"):
            assert normwise(gr[k].cpu().numpy(), rgr[k]) <= TOL_F32, k


def test_fp32_accumulate_and_forward():
    L = synthetic.layer_inputs(200, 128, 2, 1, 64, 256, "f32", seed=21, w_std=0.05, gain_std=0.1)
    dx1, g1 = _gpu(L, 2)
    g0 = {k: v.clone() for k, v in g1.items()}
    _, g2 = _gpu(L, 3, grads=g1, accumulate=True)
    for k in NAMES:
        assert normwise(g2[k].cpu().numpy(), 2 * g0[k].cpu().numpy()) < 1e-5, k
    dev = torch.device("cuda:0")
    w = {k: v.to(dev) for k, v in L.w.items()}
    y = sbp.layer_fwd(L.x.to(dev), w, L.Hq, L.Hkv, L.dh, L.eps, D=3, rope_theta=1e4)
    torch.cuda.synchronize()
    _, _, ry = oracle.layer_bwd(synthetic.to_f64(L.x), synthetic.to_f64(L.dy),
                                {k: synthetic.to_f64(v) for k, v in L.w.items()}, L.Hq, L.Hkv,
                                L.dh, L.eps, rope_theta=1e4)
    assert y.dtype == torch.float32
    assert normwise(y.cpu().numpy(), ry) <= TOL_F32
