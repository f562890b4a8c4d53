"""Large-magnitude inputs on the GPU against the fp64 oracle.

The workloads' inputs give logits of std ~1.3 and attention scores of std ~1,
so the numeric shortcuts of the kernels only see their easy range there:

* the LM head keeps the chunk's logits as fp16 values relative to the max of
  their 64-column group, and its GEMM epilogue forms per-group (max, sum-exp)
  partials that later kernels merge; here the logits spread over tens to
  hundreds, with rows whose softmax is one-hot at the target and rows whose
  softmax peaks away from it, on the fused (d % 128 == 0) and the fp32-logits
  paths, with ragged row and column tiles;
* attention's online softmax moves its running max only when a key tile
  exceeds it by more than 8 (base 2); here Q and K have std 3 (scores of std
  ~9) and one head dimension carries a ramp over key positions, so nearly
  every later key tile raises the max by more than that.

Same bars as the other parity tests: normwise <= 2e-2 (bf16), <= 1e-4 (fp32).
"""
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
TOL = {"bf16": 2e-2, "f32": 1e-4}


def _peaked_lmhead(T, d, V, dtype, seed, h_std, w_std):
    inp = synthetic.lmhead_inputs(T, d, V, dtype, seed=seed, h_std=h_std, w_std=w_std,
                                  ignore_frac=0.05)
    y = inp.targets
    # rows 3, 10, 17, ...: h = a W[y] (softmax one-hot at the target);
    # rows 5, 12, 19, ...: h = a W[v] with v != y (peaked away from it);
    # the peak logit a |W_v|^2 is then about 150
    a = 150.0 / (w_std * w_std * d)
    for r in range(3, T, 7):
        if y[r] >= 0:
            inp.H[r] = (a * inp.W[int(y[r])].float()).to(inp.H.dtype)
    for r in range(5, T, 7):
        if y[r] >= 0:
            inp.H[r] = (a * inp.W[(int(y[r]) + 1) % V].float()).to(inp.H.dtype)
    return inp


@pytest.mark.parametrize("dtype,T,d,V,D,h_std,w_std", [
    ("bf16", 1000, 1024, 5000, 3, 1.0, 0.2),   # fused statistics; logit std ~6
    ("bf16", 777, 1024, 4133, 2, 8.0, 0.02),   # large hidden states; ragged tiles
    ("bf16", 600, 1032, 3000, 3, 1.0, 0.2),    # d % 128 != 0: fp32 logits pass
    ("f32", 400, 256, 2000, 3, 1.0, 0.5),      # fp32 mode
])
def test_lmhead_large_logits(dtype, T, d, V, D, h_std, w_std):
    inp = _peaked_lmhead(T, d, V, dtype, 500 + T, h_std, w_std)
    H, W, tg = inp.H.to(DEV), inp.W.to(DEV), inp.targets.to(DEV)
    loss, dH, dW, tl = sbp.lmhead_ce(H, W, tg, D=D, token_loss=True)
    lp, ls = sbp.lmhead_logprob(H, W, tg, D=D, lse=True)
    torch.cuda.synchronize()
    L, rH, rW, rtl, rlse = oracle.lmhead_ce(synthetic.to_f64(inp.H), synthetic.to_f64(inp.W),
                                            inp.targets.numpy())
    rlp, rls = oracle.lmhead_logprob(synthetic.to_f64(inp.H), synthetic.to_f64(inp.W),
                                     inp.targets.numpy())
    tol = TOL[dtype]
    # the logits really are spread over tens (and the peaked rows over hundreds)
    assert np.nanmax(rlse) > 50.0
    assert abs(loss.item() - L) <= tol * abs(L)
    errs = {"dH": normwise(dH.float().cpu().numpy(), rH),
            "dW": normwise(dW.cpu().numpy(), rW),
            "tl": normwise(tl.cpu().numpy(), rtl),
            "logprob": normwise(lp.cpu().numpy(), rlp),
            "lse": normwise(ls.cpu().numpy(), rls)}
    assert all(e <= tol for e in errs.values()), errs


def _ramped_attn(B, T, Hq, Hkv, dh, seed, std=3.0, slope=0.25, qconst=4.0):
    inp = synthetic.attn_inputs(B, T, Hq, Hkv, dh, "bf16", seed=seed, std=std)
    # score term s * qconst * slope * j grows along the key position j
    ramp = (slope * torch.arange(T, dtype=torch.float32)).to(torch.bfloat16)
    inp.K[:, :, :, 0] = ramp[None, :, None]
    inp.Q[:, :, :, 0] = qconst
    return inp


@pytest.mark.parametrize("B,T,Hq,Hkv,dh,D", [
    (1, 700, 4, 2, 128, 3),
    (2, 517, 4, 1, 64, 2),
    (1, 1100, 2, 2, 64, 1),
])
def test_attention_large_scores_rising_max(B, T, Hq, Hkv, dh, D):
    inp = _ramped_attn(B, T, Hq, Hkv, dh, seed=T + dh)
    s = 1.0 / math.sqrt(dh)
    q = synthetic.to_f64(inp.Q)
    k = synthetic.to_f64(inp.K)
    # scores of std ~9 on top of a ramp that climbs more than 8 log2 units
    # (5.5 natural) per 64-key tile
    assert s * 4.0 * 0.25 * 64 > 8 * math.log(2)
    assert np.std(s * np.einsum("d,jd->j", q[0, -1, 0, 1:], k[0, :, 0, 1:])) > 5.0
    dQ, dK, dV = sbp.attn_bwd(inp.Q.to(DEV), inp.K.to(DEV), inp.V.to(DEV), inp.dO.to(DEV), D=D)
    torch.cuda.synchronize()
    rQ, rK, rV, _, _ = oracle.attn_bwd(q, k, synthetic.to_f64(inp.V), synthetic.to_f64(inp.dO), s)
    errs = (normwise(dQ.float().cpu().numpy(), rQ), normwise(dK.cpu().numpy(), rK),
            normwise(dV.cpu().numpy(), rV))
    assert all(e <= TOL["bf16"] for e in errs), errs


def test_attention_large_scores_packed():
    # the same inputs as packed sequences: the ramp restarts nowhere, but
    # every sequence's first tile sets its own running max
    T = 900
    inp = _ramped_attn(1, T, 4, 2, 128, seed=77)
    cu = [0, 130, 131, 500, 900]
    s = 1.0 / math.sqrt(128)
    c = torch.tensor(cu, dtype=torch.int32, device=DEV)
    dQ, dK, dV = sbp.attn_bwd(inp.Q.to(DEV), inp.K.to(DEV), inp.V.to(DEV), inp.dO.to(DEV), D=4,
                              cu_seqlens=c)
    torch.cuda.synchronize()
    f = synthetic.to_f64
    rQ, rK, rV = oracle.attn_bwd_packed(f(inp.Q), f(inp.K), f(inp.V), f(inp.dO), s, cu)[:3]
    errs = (normwise(dQ.float().cpu().numpy(), rQ), normwise(dK.cpu().numpy(), rK),
            normwise(dV.cpu().numpy(), rV))
    assert all(e <= TOL["bf16"] for e in errs), errs
