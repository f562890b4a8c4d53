"""The allocation-free attention entry point (sbp_attn_bwd_chunked_noalloc,
scratch in a static device array) against sbp_attn_bwd_chunked (scratch in a
caller workspace): both through the C ABI, on two calls in a row, the second
smaller, so the second runs on the scratch the first left behind."""
import math

import pytest
import torch

import memory_efficient_exact_amd as sbp
from memory_efficient_exact_amd import _lib
import oracle
import synthetic
from helpers import normwise

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _noalloc(inp, D, dK=None, dV=None, accumulate=False):
    Q, K, V, dO = (x.to(DEV) for x in (inp.Q, inp.K, inp.V, inp.dO))
    B, T, Hq, dh = Q.shape
    Hkv = K.shape[2]
    dQ = torch.empty_like(Q)
    dK = torch.empty(B, T, Hkv, dh, dtype=torch.float32, device=DEV) if dK is None else dK
    dV = torch.empty(B, T, Hkv, dh, dtype=torch.float32, device=DEV) if dV is None else dV
    st = sbp.load().sbp_attn_bwd_chunked_noalloc(
        _ptr(Q), _ptr(K), _ptr(V), _ptr(dO), None, None, B, T, Hq, Hkv, dh,
        1.0 / math.sqrt(dh), D, _lib.SBP_BF16, int(accumulate), _ptr(dQ), _ptr(dK), _ptr(dV),
        torch.cuda.current_stream(DEV).cuda_stream)
    _lib.check(st)
    torch.cuda.synchronize()
    return dQ, dK, dV


def _with_workspace(inp, D):
    out = sbp.attn_bwd(inp.Q.to(DEV), inp.K.to(DEV), inp.V.to(DEV), inp.dO.to(DEV), D=D)
    torch.cuda.synchronize()
    return out


def _same(a, b, ref):
    for x, y, r in zip(a, b, ref):
        # the same kernels on the same inputs: identical results, and both
        # within the bf16 bar of the fp64 oracle
        assert torch.equal(x, y)
        assert normwise(x.float().cpu().numpy(), r) <= 2e-2


def test_noalloc_matches_workspace_entry_point_twice_shrinking():
    shapes = [(1, 1000, 8, 2, 128, 3), (2, 300, 4, 2, 64, 2)]
    for B, T, Hq, Hkv, dh, D in shapes:
        print(f"noalloc case B={B} T={T} Hq={Hq} Hkv={Hkv} dh={dh} D={D}", flush=True)
        inp = synthetic.attn_inputs(B, T, Hq, Hkv, dh, "bf16", seed=T + dh)
        ref = oracle.attn_bwd(synthetic.to_f64(inp.Q), synthetic.to_f64(inp.K),
                              synthetic.to_f64(inp.V), synthetic.to_f64(inp.dO),
                              1.0 / math.sqrt(dh))[:3]
        _same(_noalloc(inp, D), _with_workspace(inp, D), ref)


def test_noalloc_accumulates_like_the_workspace_entry_point():
    inp = synthetic.attn_inputs(1, 256, 4, 2, 64, "bf16", seed=5)
    _, dK1, dV1 = _with_workspace(inp, 2)
    _, dK2, dV2 = _noalloc(inp, 4, dK=dK1.clone(), dV=dV1.clone(), accumulate=True)
    assert normwise(dK2.cpu().numpy(), 2 * dK1.cpu().numpy()) < 1e-2
    assert normwise(dV2.cpu().numpy(), 2 * dV1.cpu().numpy()) < 1e-2


def test_noalloc_rejects_scratch_beyond_its_size_before_any_launch():
    # B * Hq * chunk length past 16 MiB of statistics: an error, nothing run
    small = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    st = sbp.load().sbp_attn_bwd_chunked_noalloc(
        _ptr(small), _ptr(small), _ptr(small), _ptr(small), None, None, 1, 65536, 64, 8, 128,
        0.088, 1, _lib.SBP_BF16, 0, _ptr(small), _ptr(small), _ptr(small),
        torch.cuda.current_stream(DEV).cuda_stream)
    assert st == _lib.SBP_ERR_UNSUPPORTED
    assert b"static" in sbp.load().sbp_last_error()
