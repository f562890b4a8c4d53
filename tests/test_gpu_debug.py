"""Debug mode (SBP_DEBUG=1): device-side checks of target ids and packed
sequence boundaries before any of a call's own kernels run, and a stream
synchronisation after them.  Bad packed-sequence bounds are only ever
passed with debug mode on (without it the kernels clamp them but do not
check them); target ids past the vocabulary without debug mode are covered
in test_gpu_edge.py (NaN outputs, every read in bounds)."""
import pytest
import torch

import memory_efficient_exact_amd as sbp
from memory_efficient_exact_amd import _lib
import synthetic

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture
def debug_mode(monkeypatch):
    monkeypatch.setenv("SBP_DEBUG", "1")


def _lm(T=200, d=64, V=300):
    inp = synthetic.lmhead_inputs(T, d, V, "bf16", seed=5, w_std=0.05)
    return inp.H.to(DEV), inp.W.to(DEV), inp.targets.to(DEV)


def test_debug_mode_gives_the_same_results(debug_mode, monkeypatch):
    H, W, y = _lm()
    loss, dH, dW, _ = sbp.lmhead_ce(H, W, y, D=3)
    torch.cuda.synchronize()
    monkeypatch.setenv("SBP_DEBUG", "0")
    loss2, dH2, dW2, _ = sbp.lmhead_ce(H, W, y, D=3)
    torch.cuda.synchronize()
    assert torch.equal(loss, loss2) and torch.equal(dH, dH2) and torch.equal(dW, dW2)


def test_target_ids_past_the_vocabulary_are_rejected(debug_mode):
    H, W, y = _lm()
    y[17] = W.shape[0]
    y[150] = W.shape[0] + 5
    with pytest.raises(_lib.StreamBPError) as e:
        sbp.lmhead_ce(H, W, y, D=3)
    assert e.value.status == _lib.SBP_ERR_INVALID_ARG and "2 target ids" in str(e.value)
    with pytest.raises(_lib.StreamBPError) as e:
        sbp.lmhead_logprob(H, W, y, D=3)
    assert e.value.status == _lib.SBP_ERR_INVALID_ARG


@pytest.mark.parametrize("cu", [[0, 50, 40, 128], [0, 50, 100], [3, 50, 128]])
def test_bad_sequence_boundaries_are_rejected(debug_mode, cu):
    a = synthetic.attn_inputs(1, 128, 4, 2, 64, "bf16", seed=6)
    c = torch.tensor(cu, dtype=torch.int32, device=DEV)
    with pytest.raises(_lib.StreamBPError) as e:
        sbp.attn_bwd(a.Q.to(DEV), a.K.to(DEV), a.V.to(DEV), a.dO.to(DEV), D=2, cu_seqlens=c)
    assert e.value.status == _lib.SBP_ERR_INVALID_ARG
    L = synthetic.layer_inputs(128, 128, 4, 2, 64, 256, "bf16", seed=7, w_std=0.05)
    w = {k: v.to(DEV) for k, v in L.w.items()}
    with pytest.raises(_lib.StreamBPError) as e:
        sbp.layer_bwd(L.x.to(DEV), L.dy.to(DEV), w, L.Hq, L.Hkv, L.dh, L.eps, D=2, cu_seqlens=c)
    assert e.value.status == _lib.SBP_ERR_INVALID_ARG
    with pytest.raises(_lib.StreamBPError) as e:
        sbp.layer_fwd(L.x.to(DEV), w, L.Hq, L.Hkv, L.dh, L.eps, D=2, cu_seqlens=c)
    assert e.value.status == _lib.SBP_ERR_INVALID_ARG


def test_model_call_checks_its_targets(debug_mode):
    M = synthetic.model_inputs(96, 128, 2, 1, 64, 256, 300, 1, "bf16", seed=8, w_std=0.05)
    layers = [{k: v.to(DEV) for k, v in w.items()} for w in M.layers]
    xs = sbp.model_fwd(M.x0.to(DEV), layers, M.Hq, M.Hkv, M.dh, M.eps, 2)
    y = M.targets.clone()
    y[5] = 300
    with pytest.raises(_lib.StreamBPError) as e:
        sbp.model_bwd(xs, layers, M.g_final.to(DEV), M.W.to(DEV), y.to(DEV), Hq=M.Hq, Hkv=M.Hkv,
                      dh=M.dh, eps=M.eps, D_lm=2, D_layer=2)
    assert e.value.status == _lib.SBP_ERR_INVALID_ARG
