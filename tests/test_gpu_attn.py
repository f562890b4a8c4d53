"""GPU parity of sbp_attn_bwd_chunked against the fp64 oracle (bf16 inputs,
fp32 accumulation): normwise max|gpu - ref| / max|ref| <= 2e-2 on dQ, dK, dV."""
import math

import numpy as np
import pytest
import torch

import memory_efficient_exact_amd as sbp
import oracle
import synthetic
from helpers import normwise

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _gpu(inp, D, **kw):
    dev = torch.device("cuda:0")
    out = sbp.attn_bwd(inp.Q.to(dev), inp.K.to(dev), inp.V.to(dev), inp.dO.to(dev), D=D, **kw)
    torch.cuda.synchronize()
    return out


def _ref(inp, scale):
    return oracle.attn_bwd(synthetic.to_f64(inp.Q), synthetic.to_f64(inp.K),
                           synthetic.to_f64(inp.V), synthetic.to_f64(inp.dO), scale)


@pytest.mark.parametrize("B,T,Hq,Hkv,dh,D", [
    (1, 300, 4, 2, 64, 3),      # ragged T, ragged chunks
    (2, 257, 4, 1, 128, 1),     # B > 1, one chunk, MQA
    (1, 512, 8, 2, 128, 4),     # tile-aligned chunks
    (1, 64, 2, 2, 64, 64),      # D = T: one query per chunk
    (1, 1000, 4, 4, 128, 7),    # MHA, several key tiles per chunk
    (1, 1, 2, 1, 64, 1),        # a single token
    (1, 700, 6, 3, 128, 2),     # Hkv = 3 (kv heads do not divide the 8 XCDs)
    (1, 520, 16, 2, 64, 2),     # G = 8 query heads per kv head
    (1, 400, 16, 16, 64, 3),    # Hkv = 16 > 8 XCDs
])
def test_parity(B, T, Hq, Hkv, dh, D):
    inp = synthetic.attn_inputs(B, T, Hq, Hkv, dh, "bf16", seed=T + Hq + dh + D)
    s = 1.0 / math.sqrt(dh)
    dQ, dK, dV = _gpu(inp, D)
    rQ, rK, rV, _, _ = _ref(inp, s)
    eq = normwise(dQ.float().cpu().numpy(), rQ)
    ek = normwise(dK.cpu().numpy(), rK)
    ev = normwise(dV.cpu().numpy(), rV)
    assert eq <= TOL and ek <= TOL and ev <= TOL, (eq, ek, ev)


def test_given_forward_statistics():
    # O and LSE supplied by the caller (from the oracle's forward): no recompute
    B, T, Hq, Hkv, dh, D = 1, 384, 4, 2, 128, 3
    inp = synthetic.attn_inputs(B, T, Hq, Hkv, dh, "bf16", seed=11)
    s = 1.0 / math.sqrt(dh)
    rQ, rK, rV, rO, rL = _ref(inp, s)
    dev = torch.device("cuda:0")
    O = torch.from_numpy(rO).to(torch.bfloat16).to(dev)
    L = torch.from_numpy(rL).to(torch.float32).to(dev).contiguous()
    dQ, dK, dV = _gpu(inp, D, O=O, lse=L)
    assert normwise(dQ.float().cpu().numpy(), rQ) <= TOL
    assert normwise(dK.cpu().numpy(), rK) <= TOL
    assert normwise(dV.cpu().numpy(), rV) <= TOL


def test_accumulate_adds_into_dK_dV():
    inp = synthetic.attn_inputs(1, 256, 4, 2, 64, "bf16", seed=5)
    dQ1, dK1, dV1 = _gpu(inp, 2)
    dQ2, dK2, dV2 = _gpu(inp, 4, dK=dK1.clone(), dV=dV1.clone(), accumulate=True)
    assert normwise(dK2.cpu().numpy(), 2 * dK1.cpu().numpy()) < 1e-2
    assert normwise(dV2.cpu().numpy(), 2 * dV1.cpu().numpy()) < 1e-2


def test_gpu_D_invariance():
    inp = synthetic.attn_inputs(1, 1024, 8, 2, 128, "bf16", seed=7)
    outs = [_gpu(inp, D) for D in (1, 2, 8)]
    for o in outs[1:]:
        for x, y in zip(o, outs[0]):
            assert normwise(x.float().cpu().numpy(), y.float().cpu().numpy()) < 1e-2


def test_full_size_T16384_sampled():
    """The causal GQA workload at its full size (B=1, T=16384, 32/8 heads of
    128, D=8), checked against exact per-row oracle values on sampled heads,
    queries and keys, plus sum_j dK_j = 0 on every kv head."""
    cfg = synthetic.WORKLOADS[2]
    inp = synthetic.workload_inputs(2)
    s = 1.0 / math.sqrt(cfg["dh"])
    dQ, dK, dV = _gpu(inp, cfg["D"])
    T = cfg["T"]
    rng = np.random.default_rng(2)
    q_rows = np.concatenate([[0, 1, 2047, 2048, T - 1], rng.integers(0, T, 11)])
    k_rows = np.concatenate([[0, 2047, 2048, 14335, T - 1], rng.integers(0, T, 11)])
    heads = [0, 13]  # kv groups 0 and 3
    dQs, dKs, dVs = oracle.attn_bwd_sampled(synthetic.to_f64(inp.Q),
                                            synthetic.to_f64(inp.K), synthetic.to_f64(inp.V),
                                            synthetic.to_f64(inp.dO), s, 0, heads, q_rows, k_rows)
    dQc, dKc, dVc = dQ.float().cpu().numpy(), dK.cpu().numpy(), dV.cpu().numpy()
    for h, ref in dQs.items():
        assert normwise(dQc[0, q_rows, h], ref) <= TOL, h
    for kv, ref in dKs.items():
        assert normwise(dKc[0, k_rows, kv], ref) <= TOL, kv
        assert normwise(dVc[0, k_rows, kv], dVs[kv]) <= TOL, kv
    colsum = np.abs(dK.double().sum(1).cpu().numpy()).max()
    assert colsum <= 1e-2 * np.abs(dKc).max() * math.sqrt(T), colsum


# ---- packed independent sequences (sbp_attn_bwd_packed) -------------------
def _cu(T, cuts):
    return [0] + list(cuts) + [T]


def _gpu_packed(inp, D, cu, **kw):
    c = torch.tensor(cu, dtype=torch.int32, device="cuda:0")
    return _gpu(inp, D, cu_seqlens=c, **kw)


def _ref_packed(inp, scale, cu):
    return oracle.attn_bwd_packed(synthetic.to_f64(inp.Q), synthetic.to_f64(inp.K),
                                  synthetic.to_f64(inp.V), synthetic.to_f64(inp.dO), scale, cu)


def _random_cuts(T, n, seed):
    rng = np.random.default_rng(seed)
    return sorted(rng.choice(np.arange(1, T), size=n, replace=False).tolist())


@pytest.mark.parametrize("T,Hq,Hkv,dh,D,cuts", [
    (300, 4, 2, 64, 3, [37, 38, 150, 151]),      # length-1 sequences; cuts inside tiles and chunks
    (700, 8, 2, 128, 4, _random_cuts(700, 6, 1)),
    (512, 4, 1, 64, 1, [128, 256, 384]),         # tile-aligned sequences, MQA
    (200, 4, 4, 128, 3, [50, 50, 199]),          # an empty sequence; a last sequence of 1
    (300, 2, 2, 64, 300, [100, 101]),            # D = T
    (1000, 4, 2, 128, 7, []),                    # one sequence
    (1500, 4, 2, 128, 5, _random_cuts(1500, 3, 2)),
])
def test_packed_parity(T, Hq, Hkv, dh, D, cuts):
    inp = synthetic.attn_inputs(1, T, Hq, Hkv, dh, "bf16", seed=3 * T + Hq + dh + D)
    s = 1.0 / math.sqrt(dh)
    cu = _cu(T, cuts)
    dQ, dK, dV = _gpu_packed(inp, D, cu)
    rQ, rK, rV, _, _ = _ref_packed(inp, s, cu)
    eq = normwise(dQ.float().cpu().numpy(), rQ)
    ek = normwise(dK.cpu().numpy(), rK)
    ev = normwise(dV.cpu().numpy(), rV)
    assert eq <= TOL and ek <= TOL and ev <= TOL, (eq, ek, ev)
    # every sequence on its own, so that a leak into a short sequence shows
    # (a sequence of one token has dK = 0 exactly: its floor is a hundredth
    # of the whole tensor's scale)
    gk = dK.cpu().numpy()
    floor = 1e-2 * np.abs(rK).max()
    for a, b in zip(cu, cu[1:]):
        if b > a:
            err = np.abs(gk[:, a:b] - rK[:, a:b]).max()
            assert err <= TOL * max(np.abs(rK[:, a:b]).max(), floor), (a, b, err)


def test_packed_one_sequence_equals_causal_call():
    inp = synthetic.attn_inputs(1, 777, 4, 2, 128, "bf16", seed=21)
    a = _gpu(inp, 3)
    b = _gpu_packed(inp, 3, [0, 777])
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_packed_given_forward_statistics_and_accumulate():
    T, Hq, Hkv, dh, D = 640, 4, 2, 64, 4
    cu = _cu(T, [90, 91, 333])
    inp = synthetic.attn_inputs(1, T, Hq, Hkv, dh, "bf16", seed=22)
    s = 1.0 / math.sqrt(dh)
    rQ, rK, rV, rO, rL = _ref_packed(inp, s, cu)
    dev = torch.device("cuda:0")
    O = torch.from_numpy(rO).to(torch.bfloat16).to(dev)
    L = torch.from_numpy(rL).to(torch.float32).to(dev).contiguous()
    dQ, dK, dV = _gpu_packed(inp, D, cu, O=O, lse=L)
    assert normwise(dQ.float().cpu().numpy(), rQ) <= TOL
    assert normwise(dK.cpu().numpy(), rK) <= TOL
    assert normwise(dV.cpu().numpy(), rV) <= TOL
    _, dK2, dV2 = _gpu_packed(inp, 2, cu, dK=dK.clone(), dV=dV.clone(), accumulate=True)
    assert normwise(dK2.cpu().numpy(), 2 * rK) <= TOL
    assert normwise(dV2.cpu().numpy(), 2 * rV) <= TOL


def test_packed_full_size_T16384_sampled_sequences():
    # the attention workload's shape with 8 packed sequences of random
    # lengths, at its chunking; three sequences checked against the oracle
    cfg = synthetic.WORKLOADS[2]
    T, D = cfg["T"], cfg["D"]
    inp = synthetic.workload_inputs(2)
    cu = _cu(T, _random_cuts(T, 7, 3))
    dQ, dK, dV = _gpu_packed(inp, D, cu)
    s = 1.0 / math.sqrt(cfg["dh"])
    for n in (0, 3, 7):
        a, b = cu[n], cu[n + 1]
        sub = synthetic.AttnInputs(inp.Q[:, a:b], inp.K[:, a:b], inp.V[:, a:b], inp.dO[:, a:b])
        rQ, rK, rV, _, _ = _ref_packed(sub, s, [0, b - a])
        assert normwise(dQ[:, a:b].float().cpu().numpy(), rQ) <= TOL, n
        assert normwise(dK[:, a:b].cpu().numpy(), rK) <= TOL, n
        assert normwise(dV[:, a:b].cpu().numpy(), rV) <= TOL, n


# ---- fp32 mode: every product in fp32, normwise <= 1e-4 -------------------
TOL_F32 = 1e-4


@pytest.mark.parametrize("B,T,Hq,Hkv,dh,D", [
    (1, 300, 4, 2, 64, 3),      # ragged T and chunks, GQA
    (2, 257, 4, 1, 128, 1),     # B > 1, one chunk, MQA
    (1, 96, 2, 2, 64, 96),      # D = T
    (1, 1000, 4, 4, 128, 7),    # MHA, several key tiles per chunk
])
def test_parity_fp32(B, T, Hq, Hkv, dh, D):
    inp = synthetic.attn_inputs(B, T, Hq, Hkv, dh, "f32", seed=3 * T + Hq + dh + D)
    s = 1.0 / math.sqrt(dh)
    dQ, dK, dV = _gpu(inp, D)
    assert dQ.dtype == torch.float32
    rQ, rK, rV, _, _ = _ref(inp, s)
    errs = (normwise(dQ.cpu().numpy(), rQ), normwise(dK.cpu().numpy(), rK),
            normwise(dV.cpu().numpy(), rV))
    assert all(e <= TOL_F32 for e in errs), errs


def test_fp32_single_token():
    # one token attends only to itself: P = 1, so dS = P (dP - Delta) is 0 in
    # exact arithmetic and dQ = dK = 0 (the reference is exactly zero, so a
    # normwise ratio is undefined); in fp32, dP and Delta are sums in
    # different orders and leave a residue of the order of fp32 rounding of
    # the terms dO . V; dV = dO summed over the group
    inp = synthetic.attn_inputs(1, 1, 2, 1, 128, "f32", seed=5)
    dQ, dK, dV = _gpu(inp, 1)
    rQ, rK, rV, _, _ = _ref(inp, 1.0 / math.sqrt(128))
    assert not rQ.any() and not rK.any()
    s = 1.0 / math.sqrt(128)
    f = synthetic.to_f64
    term = np.abs(f(inp.dO)).max() * np.abs(f(inp.V)).max() * 128
    assert np.abs(dQ.cpu().numpy()).max() <= 1e-6 * s * term * np.abs(f(inp.K)).max() * 128
    assert np.abs(dK.cpu().numpy()).max() <= 1e-6 * s * term * np.abs(f(inp.Q)).max() * 128 * 2
    assert normwise(dV.cpu().numpy(), rV) <= TOL_F32


def test_fp32_given_forward_statistics_and_packed():
    B, T, Hq, Hkv, dh = 1, 400, 4, 2, 64
    inp = synthetic.attn_inputs(B, T, Hq, Hkv, dh, "f32", seed=12)
    s = 1.0 / math.sqrt(dh)
    rQ, rK, rV, rO, rL = _ref(inp, s)
    dev = torch.device("cuda:0")
    O = torch.from_numpy(rO).to(torch.float32).to(dev)
    L = torch.from_numpy(rL).to(torch.float32).to(dev).contiguous()
    dQ, dK, dV = _gpu(inp, 3, O=O, lse=L)
    for g, r in ((dQ, rQ), (dK, rK), (dV, rV)):
        assert normwise(g.cpu().numpy(), r) <= TOL_F32
    cu = [0, 70, 71, 250, 400]
    c = torch.tensor(cu, dtype=torch.int32, device=dev)
    dQ, dK, dV = _gpu(inp, 4, cu_seqlens=c)
    f = synthetic.to_f64
    pQ, pK, pV = oracle.attn_bwd_packed(f(inp.Q), f(inp.K), f(inp.V), f(inp.dO), s, cu)[:3]
    for g, r in ((dQ, pQ), (dK, pK), (dV, pV)):
        assert normwise(g.cpu().numpy(), r) <= TOL_F32
