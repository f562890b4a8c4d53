"""GPU parity of sbp_lmhead_ce_fwd_bwd against the fp64 oracle.

Normwise error max|gpu - ref| / max|ref| per output; fp32 mode <= 1e-4,
bf16 mode <= 2e-2 (fp32 accumulation).  The loss is compared against
max(|L|, (1/N) sum_t |c_t| l_t) because signed weights can cancel L.
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

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _run(inp, D, reduction="mean_valid", accumulate=False, dW=None, dw_group=1):
    dev = torch.device("cuda:0")
    H, W, tg = inp.H.to(dev), inp.W.to(dev), inp.targets.to(dev)
    w = None if inp.weights is None else inp.weights.to(dev)
    loss, dH, dWo, tl = sbp.lmhead_ce(H, W, tg, w, D=D, reduction=reduction,
                                      accumulate=accumulate, dW=dW, token_loss=True,
                                      dw_group=dw_group)
    torch.cuda.synchronize()
    return loss, dH, dWo, tl


def _check(inp, D, dtype, reduction="mean_valid"):
    loss, dH, dW, tl = _run(inp, D, reduction)
    L, rH, rW, rtl, _ = oracle.lmhead_ce(synthetic.to_f64(inp.H), synthetic.to_f64(inp.W),
                                         inp.targets.numpy(), synthetic.to_f64(inp.weights),
                                         reduction)
    tol = TOL[dtype]
    y = inp.targets.numpy()
    valid = y >= 0
    N = max(1, int(valid.sum())) if reduction == "mean_valid" else 1
    c = np.where(valid, 1.0 if inp.weights is None else inp.weights.numpy().astype(np.float64), 0.0)
    den = max(abs(L), float(np.abs(c * rtl).sum()) / N, 1e-30)
    e_loss = abs(loss.item() - L) / den
    e_dH = normwise(dH.float().cpu().numpy(), rH)
    e_dW = normwise(dW.cpu().numpy(), rW)
    e_tl = normwise(tl.cpu().numpy(), rtl)
    assert e_loss <= tol, (e_loss, loss.item(), L)
    assert e_dH <= tol, e_dH
    assert e_dW <= tol, e_dW
    assert e_tl <= tol, e_tl
    # ignored tokens give exactly zero dH rows
    if (~valid).any():
        assert (dH[torch.from_numpy(~valid).cuda()] == 0).all()
    return dict(loss=e_loss, dH=e_dH, dW=e_dW, tl=e_tl)


# ---- the small fp32 workload at its exact size, D swept ------------------
@pytest.mark.parametrize("D", [4, 1, 2, 3, 256])
def test_fp32_workload0_D_sweep(D):
    inp = synthetic.workload_inputs(0)
    _check(inp, D, "f32")


# ---- ragged shapes spanning several tiles --------------------------------
@pytest.mark.parametrize("dtype,T,d,V,D", [
    ("f32", 333, 68, 1000, 3),
    ("f32", 1000, 128, 777, 7),
    ("bf16", 1000, 256, 5000, 3),
    ("bf16", 517, 136, 2063, 1),
    ("bf16", 2048, 512, 8192, 8),
    ("bf16", 300, 64, 130, 300),   # D = T: one token per chunk
])
def test_ragged_parity(dtype, T, d, V, D):
    inp = synthetic.lmhead_inputs(T, d, V, dtype, seed=T + d + V + D,
                                  w_std=0.02 if dtype == "bf16" else None, ignore_frac=0.1)
    _check(inp, D, dtype)


def test_weighted_masked_packed_skips_chunks():
    # the weighted-token workload's structure at a small size: 8 packed
    # sequences, first quarter of each masked, per-sequence N(0,1) weights;
    # D = 32 makes every fourth chunk fully masked (skipped on the device)
    inp = synthetic.lmhead_inputs(8 * 128, 128, 3000, "bf16", seed=5, w_std=0.02, n_seq=8,
                                  masked_frac=0.25, weighted=True)
    _check(inp, 32, "bf16")


def test_weight_gradient_groups_first_group_inactive():
    # T_c = 1024 makes the weight gradient one GEMM per 4 chunks (4 groups);
    # every token of the first group is ignored, so the second group's GEMM
    # must overwrite the stale dW passed in, and the groups after it add;
    # one chunk inside the third group is ignored as well (zero slot).
    inp = synthetic.lmhead_inputs(16384, 64, 512, "bf16", seed=11, w_std=0.02)
    inp.targets[:4096] = -1
    inp.targets[9216:10240] = -1
    L, rH, rW, _, _ = oracle.lmhead_ce(synthetic.to_f64(inp.H), synthetic.to_f64(inp.W),
                                       inp.targets.numpy())
    dW0 = torch.full((512, 64), 7.0, device="cuda:0")
    loss, dH, dW, _ = _run(inp, 16, dW=dW0, dw_group=4)
    assert abs(loss.item() - L) / abs(L) <= TOL["bf16"]
    assert normwise(dH.float().cpu().numpy(), rH) <= TOL["bf16"]
    assert normwise(dW.cpu().numpy(), rW) <= TOL["bf16"]
    assert (dH[:4096] == 0).all()


@pytest.mark.parametrize("d", [256, 136])
def test_weight_gradient_group_chosen_by_the_workspace(d):
    # groups of 1, 2 and 4 chunks (T_c = 1024) and a workspace larger than
    # any group needs: the same gradients (d = 256: the chunk's logits sit in
    # the dZ group buffer and become dZ in place; d = 136: fp32 logits)
    inp = synthetic.lmhead_inputs(4096, d, 3000, "bf16", seed=13, w_std=0.05, ignore_frac=0.1)
    L, rH, rW, _, _ = oracle.lmhead_ce(synthetic.to_f64(inp.H), synthetic.to_f64(inp.W),
                                       inp.targets.numpy())
    outs = [_run(inp, 4, dw_group=g) for g in (1, 2, 4)]
    dev = torch.device("cuda:0")
    big = torch.empty(sbp.lmhead_ce_workspace_size(4096, d, 3000, 4, torch.bfloat16, 4) + 12345,
                      dtype=torch.uint8, device=dev)
    outs.append(sbp.lmhead_ce(inp.H.to(dev), inp.W.to(dev), inp.targets.to(dev), D=4,
                              workspace=big, token_loss=True))
    torch.cuda.synchronize()
    for loss, dH, dW, _ in outs:
        assert abs(loss.item() - L) / abs(L) <= TOL["bf16"]
        assert normwise(dH.float().cpu().numpy(), rH) <= TOL["bf16"]
        assert normwise(dW.cpu().numpy(), rW) <= TOL["bf16"]
    # the group changes only the summation order of dW
    for o in outs[1:]:
        assert normwise(o[2].cpu().numpy(), outs[0][2].cpu().numpy()) <= 1e-5
        assert torch.equal(o[1], outs[0][1])


def test_sum_reduction():
    inp = synthetic.lmhead_inputs(400, 64, 900, "f32", seed=9, weighted=True, ignore_frac=0.2)
    _check(inp, 5, "f32", reduction="sum")


def test_all_tokens_ignored():
    inp = synthetic.lmhead_inputs(256, 64, 512, "bf16", seed=3, w_std=0.02)
    inp.targets[:] = -1
    dW0 = torch.full((512, 64), 7.0, device="cuda:0")
    loss, dH, dW, tl = _run(inp, 4, dW=dW0.clone())
    assert loss.item() == 0.0 and (dH == 0).all() and (dW == 0).all() and (tl == 0).all()
    loss, dH, dW, tl = _run(inp, 4, accumulate=True, dW=dW0.clone())
    assert (dW == 7.0).all()


def test_accumulate_adds_into_dW():
    inp = synthetic.lmhead_inputs(512, 128, 1024, "f32", seed=4)
    _, _, dW1, _ = _run(inp, 4)
    _, _, dW2, _ = _run(inp, 2, accumulate=True, dW=dW1.clone())
    assert normwise(dW2.cpu().numpy(), 2 * dW1.cpu().numpy()) < 1e-5


def test_gpu_D_invariance_bf16():
    inp = synthetic.lmhead_inputs(4096, 512, 4096, "bf16", seed=8, w_std=0.02)
    outs = [_run(inp, D) for D in (1, 2, 16)]
    base = outs[0]
    for o in outs[1:]:
        assert abs(o[0].item() - base[0].item()) <= 1e-5 * abs(base[0].item())
        assert normwise(o[1].float().cpu().numpy(), base[1].float().cpu().numpy()) < 1e-2
        assert normwise(o[2].cpu().numpy(), base[2].cpu().numpy()) < 1e-4


# ---- full-size workloads: sampled rows + size-free identities ------------
def _vocab_sample(V, y, rng, n_rand=16):
    """dW rows to compare: the first and last rows, rows on both sides of
    256-row tile edges (one early, one at the last full tile), the rows that
    are the target of the most tokens, and random rows."""
    last_tile = (V // 256) * 256
    edges = [0, 1, 255, 256, 8191, 8192, last_tile - 1, min(last_tile, V - 1), V - 1]
    counts = np.bincount(y[y >= 0], minlength=V)
    heavy = np.argsort(counts, kind="stable")[-4:]
    return np.unique(np.concatenate([edges, heavy, rng.integers(0, V, n_rand)]))


def _check_dW_rows(inp, dW, vrows, tol=2e-2):
    ref, _, _ = oracle.lmhead_dW_rows(synthetic.to_f64(inp.H), synthetic.to_f64(inp.W),
                                      inp.targets.numpy(), synthetic.to_f64(inp.weights), vrows)
    got = dW[torch.from_numpy(vrows).cuda()].double().cpu().numpy()
    e = normwise(got, ref)
    assert e <= tol, e
    return e


def _full_size(index, rows, vrows=None, inp=None):
    cfg = synthetic.WORKLOADS[index]
    inp = synthetic.workload_inputs(index) if inp is None else inp
    # the launch configuration the benchmark times: groups of ~4096 tokens
    loss, dH, dW, tl = _run(inp, cfg["D"], dw_group=sbp.lmhead_ce_max_group(cfg["T"], cfg["D"]))
    y = inp.targets.numpy()
    N = int((y >= 0).sum())
    rows = np.asarray(rows)
    rH, rtl, _ = oracle.lmhead_ce_rows(synthetic.to_f64(inp.H), synthetic.to_f64(inp.W), y,
                                       synthetic.to_f64(inp.weights), rows, N)
    e_dH = normwise(dH[torch.from_numpy(rows).cuda()].float().cpu().numpy(), rH)
    e_tl = normwise(tl[torch.from_numpy(rows).cuda()].cpu().numpy(), rtl)
    assert e_dH <= 2e-2, e_dH
    assert e_tl <= 2e-2, e_tl
    # sum_v (softmax - onehot) = 0 for every token, so the vocab sum of dW is 0
    col = dW.double().sum(0).abs().max().item()
    assert col <= 1e-3 * dW.abs().max().item() * math.sqrt(dW.shape[0]), col
    # <dW, W> = sum_tv dZ_tv Z_tv = <dH, H>
    a = (dW.double() * inp.W.to("cuda:0").double()).sum().item()
    b = (dH.double() * inp.H.to("cuda:0").double()).sum().item()
    assert abs(a - b) <= 2e-2 * max(abs(a), abs(b)), (a, b)
    # loss from the per-token losses (rows checked above) and the weights
    c = np.where(y >= 0, 1.0 if inp.weights is None else inp.weights.numpy(), 0.0)
    L = float((c * tl.double().cpu().numpy()).sum()) / N
    assert abs(loss.item() - L) <= 1e-4 * max(abs(L), 1e-3)
    if vrows is not None:
        # dW rows element by element: every token's lse enters each column
        _check_dW_rows(inp, dW, vrows)
    return inp


def test_full_size_bf16_T32768_V128256():
    rng = np.random.default_rng(0)
    rows = np.concatenate([[0, 1, 2047, 2048, 32767], rng.integers(0, 32768, 27)])
    inp = synthetic.workload_inputs(1)
    # two vocab rows made the target of many tokens, spread over all chunks
    # (their one-hot terms are summed across every dW group)
    y = inp.targets
    y[rng.integers(0, 32768, 600)] = 77777
    y[rng.integers(0, 32768, 60)] = 128255
    vrows = _vocab_sample(128256, y.numpy(), rng)
    _full_size(1, rows, vrows, inp=inp)


@pytest.mark.parametrize("D,n_seq", [(8, 2), (32, 8)])
def test_dW_rows_weighted_masked_V152064_d3584(D, n_seq):
    # the weighted workload's vocabulary and width at T = 16384: packed
    # sequences, first quarter of each masked (whole chunks skipped on the
    # device, dW groups mixing skipped and live chunks), one N(0,1) weight
    # per sequence; dW rows element by element and dH on sampled rows
    T = 16384
    inp = synthetic.lmhead_inputs(T, 3584, 152064, "bf16", seed=1004 + D, w_std=0.02,
                                  n_seq=n_seq, masked_frac=0.25, weighted=True)
    loss, dH, dW, tl = _run(inp, D)
    rng = np.random.default_rng(D)
    y = inp.targets.numpy()
    vrows = _vocab_sample(152064, y, rng)
    ref_rows, L, scale = oracle.lmhead_dW_rows(synthetic.to_f64(inp.H), synthetic.to_f64(inp.W),
                                               y, synthetic.to_f64(inp.weights), vrows)
    got = dW[torch.from_numpy(vrows).cuda()].double().cpu().numpy()
    assert normwise(got, ref_rows) <= 2e-2, normwise(got, ref_rows)
    N = int((y >= 0).sum())
    rows = np.concatenate([[0, T // n_seq // 4 - 1, T // n_seq // 4, T - 1], rng.integers(0, T, 28)])
    rH, rtl, _ = oracle.lmhead_ce_rows(synthetic.to_f64(inp.H), synthetic.to_f64(inp.W), y,
                                       synthetic.to_f64(inp.weights), rows, N)
    assert normwise(dH[torch.from_numpy(rows).cuda()].float().cpu().numpy(), rH) <= 2e-2
    assert abs(loss.item() - L) <= 2e-2 * max(abs(L), scale), (loss.item(), L, scale)
    assert (dH[torch.from_numpy(y < 0).cuda()] == 0).all()


def test_full_size_weighted_T131072_V152064():
    rng = np.random.default_rng(1)
    rows = np.concatenate([[0, 4095, 4096, 16383, 16384 + 4096, 131071],
                           rng.integers(0, 131072, 26)])
    _full_size(4, rows)


# ---- forward-only per-token log-probability (sbp_lmhead_logprob_fwd) -----
def _lp_run(inp, D):
    dev = torch.device("cuda:0")
    lp, ls = sbp.lmhead_logprob(inp.H.to(dev), inp.W.to(dev), inp.targets.to(dev), D=D, lse=True)
    torch.cuda.synchronize()
    return lp.cpu().numpy(), ls.cpu().numpy()


def _lp_check(inp, D, dtype):
    lp, ls = _lp_run(inp, D)
    rlp, rls = oracle.lmhead_logprob(synthetic.to_f64(inp.H), synthetic.to_f64(inp.W),
                                     inp.targets.numpy())
    e_lp, e_ls = normwise(lp, rlp), normwise(ls, rls)
    assert e_lp <= TOL[dtype], e_lp
    assert e_ls <= TOL[dtype], e_ls
    ign = inp.targets.numpy() < 0
    assert (lp[ign] == 0).all() and (ls[ign] == 0).all()
    return e_lp, e_ls


@pytest.mark.parametrize("dtype,T,d,V,D", [
    ("bf16", 1000, 256, 5000, 3),    # fused epilogue; ragged row and column tiles
    ("bf16", 2048, 512, 8192, 8),    # whole tiles only
    ("bf16", 517, 136, 2063, 1),     # d % 128 != 0: fp32 logits pass
    ("bf16", 300, 128, 130, 300),    # D = T, V < one tile
    ("f32", 333, 68, 1000, 3),
    ("f32", 256, 64, 512, 4),
])
def test_logprob_parity(dtype, T, d, V, D):
    inp = synthetic.lmhead_inputs(T, d, V, dtype, seed=7 * T + d + V + D,
                                  w_std=0.05 if dtype == "bf16" else None, ignore_frac=0.1)
    _lp_check(inp, D, dtype)


def test_logprob_target_in_last_partial_column_block():
    # every target in the last, partial 64-column quarter of the last tile
    inp = synthetic.lmhead_inputs(640, 256, 1000, "bf16", seed=31, w_std=0.05)
    inp.targets[:] = torch.randint(960, 1000, (640,), generator=torch.Generator().manual_seed(3),
                                   dtype=torch.int32)
    _lp_check(inp, 2, "bf16")


def test_logprob_masked_chunks_and_D_invariance():
    # packed sequences with masked prompts: D = 32 skips every fourth chunk
    inp = synthetic.lmhead_inputs(8 * 128, 128, 3000, "bf16", seed=32, w_std=0.05, n_seq=8,
                                  masked_frac=0.25)
    lp32, ls32 = _lp_run(inp, 32)
    _lp_check(inp, 32, "bf16")
    lp1, ls1 = _lp_run(inp, 1)
    # chunking changes only the GEMM's tile edges (and so the order in which
    # a row's statistics are merged), not the result beyond fp32 rounding
    assert normwise(lp32, lp1) <= 1e-5 and normwise(ls32, ls1) <= 1e-5


def test_logprob_is_minus_token_loss():
    inp = synthetic.lmhead_inputs(1024, 256, 4000, "bf16", seed=33, w_std=0.05, ignore_frac=0.1)
    lp, _ = _lp_run(inp, 4)
    _, _, _, tl = _run(inp, 4)
    assert normwise(-lp, tl.cpu().numpy()) <= 1e-6


def test_logprob_all_ignored():
    inp = synthetic.lmhead_inputs(256, 128, 512, "bf16", seed=34, w_std=0.05)
    inp.targets[:] = -1
    lp, ls = _lp_run(inp, 4)
    assert (lp == 0).all() and (ls == 0).all()


def test_logprob_full_size_T131072_V152064():
    # the forward log-prob workload at its full size and chunking, sampled rows
    cfg = synthetic.WORKLOADS[5]
    inp = synthetic.workload_inputs(5)
    lp, ls = _lp_run(inp, cfg["D"])
    y = inp.targets.numpy()
    rng = np.random.default_rng(5)
    rows = np.concatenate([[0, 4095, 4096, 16383, 16384 + 4096, 131071],
                           rng.integers(0, 131072, 26)])
    rlp, rls = oracle.lmhead_logprob_rows(synthetic.to_f64(inp.H), synthetic.to_f64(inp.W), y,
                                          rows)
    assert normwise(lp[rows], rlp) <= 2e-2
    assert normwise(ls[rows], rls) <= 2e-2
    valid = y >= 0
    # a probability is at most one; ignored rows are zeros
    assert lp[valid].max() <= 1e-4
    assert (lp[~valid] == 0).all() and (ls[~valid] == 0).all()
