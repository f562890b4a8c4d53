"""The seeded input generators: determinism and workload structure (CPU)."""
import torch

import synthetic


def test_seeded_and_deterministic():
    a = synthetic.lmhead_inputs(64, 8, 32, "bf16", seed=5)
    b = synthetic.lmhead_inputs(64, 8, 32, "bf16", seed=5)
    assert torch.equal(a.H, b.H) and torch.equal(a.W, b.W) and torch.equal(a.targets, b.targets)
    c = synthetic.lmhead_inputs(64, 8, 32, "bf16", seed=6)
    assert not torch.equal(a.H, c.H)


def test_packed_masked_weighted_structure():
    # 8 packed sequences, first quarter of each masked, one weight per sequence
    x = synthetic.lmhead_inputs(8 * 64, 4, 50, "bf16", seed=1, n_seq=8,
                                masked_frac=0.25, weighted=True)
    t = x.targets.view(8, 64)
    assert (t[:, :16] == -1).all() and (t[:, 16:] >= 0).all() and (t < 50).all()
    w = x.weights.view(8, 64)
    assert (w == w[:, :1]).all()
    assert x.targets.dtype == torch.int32 and x.weights.dtype == torch.float32


def test_dtypes_and_shapes():
    a = synthetic.attn_inputs(2, 33, 8, 2, 64, "bf16", seed=3)
    assert a.Q.shape == (2, 33, 8, 64) and a.K.shape == (2, 33, 2, 64)
    assert a.Q.dtype == torch.bfloat16
    L = synthetic.layer_inputs(16, 32, 4, 2, 8, 48, "f32", seed=2)
    assert L.w["Wq"].shape == (32, 32) and L.w["Wk"].shape == (16, 32)
    assert L.w["Wo"].shape == (32, 32) and L.w["W2"].shape == (32, 48)
    assert torch.equal(L.w["g1"], torch.ones(32))


def test_workload_table():
    assert synthetic.WORKLOADS[1]["T"] == 32768 and synthetic.WORKLOADS[1]["V"] == 128256
    x = synthetic.workload_inputs(0)
    assert x.H.shape == (256, 64) and x.W.shape == (512, 64) and x.H.dtype == torch.float32
    # N(0, 1/d) weights for the small fp32 workload
    assert abs(x.W.float().std().item() - 64 ** -0.5) < 0.01
