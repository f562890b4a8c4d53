"""GPU parity of sbp_layer_fwd (chunked decoder-layer forward) against the
fp64 oracle's layer forward: normwise max|gpu - ref| / max|ref| <= 2e-2 on y
(bf16 in and out, fp32 accumulation)."""
import numpy as np
import pytest
import torch

import memory_efficient_exact_amd as sbp
import oracle
import synthetic
from helpers import normwise

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _gpu(L, D, theta=0.0, cu=None, x=None):
    dev = torch.device("cuda:0")
    w = {k: v.to(dev) for k, v in L.w.items()}
    c = None if cu is None else torch.tensor(cu, dtype=torch.int32, device=dev)
    xx = (L.x if x is None else x).to(dev)
    y = sbp.layer_fwd(xx, w, L.Hq, L.Hkv, L.dh, L.eps, D=D, cu_seqlens=c, rope_theta=theta)
    torch.cuda.synchronize()
    return y.float().cpu().numpy()


def _oracle(L, theta=0.0, cu=None, x=None):
    w = {k: synthetic.to_f64(v) for k, v in L.w.items()}
    xx = L.x if x is None else x
    y, _ = oracle.layer_fwd(synthetic.to_f64(xx), w, L.Hq, L.Hkv, L.dh, L.eps, cu_seqlens=cu,
                            rope_theta=theta)
    return y


@pytest.mark.parametrize("T,d,Hq,Hkv,dh,F,D,theta,cu", [
    (300, 256, 4, 2, 64, 512, 3, 0.0, None),                         # ragged chunks
    (512, 512, 8, 2, 128, 1024, 4, 1e6, None),                        # rotary, dh 128
    (257, 128, 2, 1, 64, 256, 1, 1e4, None),                          # one chunk, MQA
    (64, 64, 2, 2, 64, 128, 64, 0.0, None),                           # D = T
    (640, 256, 4, 2, 128, 512, 5, 1e4, [0, 1, 1, 333, 639, 640]),     # packed, rotary
])
def test_parity(T, d, Hq, Hkv, dh, F, D, theta, cu):
    L = synthetic.layer_inputs(T, d, Hq, Hkv, dh, F, "bf16", seed=5 * T + d + D, w_std=0.05,
                               gain_std=0.1)
    y = _gpu(L, D, theta, cu)
    assert normwise(y, _oracle(L, theta, cu)) <= TOL


def test_D_invariance():
    L = synthetic.layer_inputs(1024, 256, 4, 2, 128, 512, "bf16", seed=19, w_std=0.05,
                               gain_std=0.1)
    base = _gpu(L, 1, 1e4)
    for D in (2, 8):
        assert normwise(_gpu(L, D, 1e4), base) < 1e-2


def test_zero_output_projections_give_identity():
    L = synthetic.layer_inputs(300, 128, 2, 1, 64, 256, "bf16", seed=21, w_std=0.05,
                               gain_std=0.1)
    L.w["Wo"] = torch.zeros_like(L.w["Wo"])
    L.w["W2"] = torch.zeros_like(L.w["W2"])
    y = _gpu(L, 3, 1e4)
    assert np.array_equal(y, L.x.float().numpy())


def test_full_size_T65536_first_and_last_sequence():
    """Workload-3 shapes (T=65536, d=4096, 32/8 heads of 128, F=14336, D=16),
    rotary base 1e6.  One causal row: y of the first P tokens depends on
    those tokens only, so the oracle on P tokens is exact.  Packed as
    [0, T-P) + [T-P, T): the last sequence's y is the oracle on its P tokens
    alone, its positions restarting at 0."""
    cfg = synthetic.WORKLOADS[3]
    L = synthetic.workload_inputs(3)
    T, P = cfg["T"], 128
    y = _gpu(L, cfg["D"], 1e6)
    w = {k: synthetic.to_f64(v) for k, v in L.w.items()}
    ref_head, _ = oracle.layer_fwd(synthetic.to_f64(L.x[:P]), w, L.Hq, L.Hkv, L.dh, L.eps,
                                   rope_theta=1e6)
    assert normwise(y[:P], ref_head) <= TOL
    yp = _gpu(L, cfg["D"], 1e6, cu=[0, T - P, T])
    ref_tail, _ = oracle.layer_fwd(synthetic.to_f64(L.x[T - P:]), w, L.Hq, L.Hkv, L.dh, L.eps,
                                   rope_theta=1e6)
    assert normwise(yp[T - P:], ref_tail) <= TOL
    assert normwise(yp[:P], ref_head) <= TOL


@pytest.mark.parametrize("theta,cu", [(1e4, None), (0.0, [0, 100, 257])])
def test_qk_norm_parity(theta, cu):
    L = synthetic.layer_inputs(257, 256, 4, 2, 128, 512, "bf16", seed=23, w_std=0.05,
                               gain_std=0.1, qk_norm=True)
    y = _gpu(L, 3, theta, cu)
    assert normwise(y, _oracle(L, theta, cu)) <= TOL
