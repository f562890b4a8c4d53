"""Seeded synthetic inputs shared by the tests, the benchmark and smoke().

This module draws random numbers and nothing else: it holds none of the
arithmetic of the method (no logits, softmax, attention or gradients), so
that the CPU oracle and the HIP path can both be fed from it without sharing
any computation.

Every generator uses a CPU ``torch.Generator`` seeded explicitly, draws in a
fixed order, and returns CPU tensors.  In bf16 mode a tensor is drawn in
fp32 and rounded to bf16 with round-to-nearest-even (``.to(torch.bfloat16)``);
the oracle then receives those bf16 values upcast exactly to fp64, so input
rounding never counts as error.

Workload shapes follow the long-sequence SFT / GRPO / DPO training the
StreamBP pages describe (8B-class decoder: hidden 4096, vocab 128256, 32
query / 8 key-value heads of width 128, MLP width 14336; and a 3584 / 152064
variant).  No dataset or trained weight is used: the distributions stand in
for post-norm hidden states and freshly initialised weights.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _normal(g: torch.Generator, shape, std: float, dtype: torch.dtype) -> torch.Tensor:
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


# ---------------------------------------------------------------------------
# LM head + cross-entropy inputs
# ---------------------------------------------------------------------------
@dataclass
class LMHeadInputs:
    H: torch.Tensor            # [T, d]   hidden states (dtype)
    W: torch.Tensor            # [V, d]   LM-head weight, [out, in] (dtype)
    targets: torch.Tensor      # [T]      int32, < 0 means "ignored"
    weights: Optional[torch.Tensor]  # [T] fp32 per-token weights or None


def lmhead_inputs(T: int, d: int, V: int, dtype: str = "bf16", seed: int = 0,
                  h_std: float = 1.0, w_std: Optional[float] = None,
                  n_seq: int = 1, masked_frac: float = 0.0,
                  weighted: bool = False, ignore_frac: float = 0.0) -> LMHeadInputs:
    """Draw order: H, W, targets, per-sequence weights, random ignore mask.

    ``masked_frac`` masks the first fraction of every one of ``n_seq`` packed
    sequences (target = -1), as a prompt would be in SFT/GRPO.  ``weighted``
    gives each sequence one N(0,1) weight repeated over its tokens (a
    sequence-level advantage).  ``ignore_frac`` additionally ignores a random
    subset of tokens (edge-case tests).
    """
    g = _gen(seed)
    tdt = DTYPES[dtype]
    if w_std is None:
        w_std = d ** -0.5
    H = _normal(g, (T, d), h_std, tdt)
    W = _normal(g, (V, d), w_std, tdt)
    targets = torch.randint(0, V, (T,), generator=g, dtype=torch.int64).to(torch.int32)
    weights = None
    if n_seq < 1 or T % n_seq != 0:
        raise ValueError("T must split into n_seq equal sequences")
    L = T // n_seq
    if weighted:
        w_seq = torch.randn(n_seq, generator=g, dtype=torch.float32)
        weights = w_seq.repeat_interleave(L).contiguous()
    if masked_frac > 0.0:
        m = int(round(L * masked_frac))
        for s in range(n_seq):
            targets[s * L: s * L + m] = -1
    if ignore_frac > 0.0:
        drop = torch.rand(T, generator=g) < ignore_frac
        targets[drop] = -1
    return LMHeadInputs(H, W, targets, weights)


# ---------------------------------------------------------------------------
# Causal GQA attention inputs, token-major [B, T, heads, dh]
# ---------------------------------------------------------------------------
@dataclass
class AttnInputs:
    Q: torch.Tensor   # [B, T, Hq, dh]
    K: torch.Tensor   # [B, T, Hkv, dh]
    V: torch.Tensor   # [B, T, Hkv, dh]
    dO: torch.Tensor  # [B, T, Hq, dh]


def attn_inputs(B: int, T: int, Hq: int, Hkv: int, dh: int, dtype: str = "bf16",
                seed: int = 0, std: float = 1.0) -> AttnInputs:
    """Draw order: Q, K, V, dO, each N(0, std^2)."""
    g = _gen(seed)
    tdt = DTYPES[dtype]
    Q = _normal(g, (B, T, Hq, dh), std, tdt)
    K = _normal(g, (B, T, Hkv, dh), std, tdt)
    V = _normal(g, (B, T, Hkv, dh), std, tdt)
    dO = _normal(g, (B, T, Hq, dh), std, tdt)
    return AttnInputs(Q, K, V, dO)


# ---------------------------------------------------------------------------
# Decoder layer inputs (pre-norm: RMSNorm -> GQA attention -> RMSNorm -> SwiGLU)
# ---------------------------------------------------------------------------
LAYER_WEIGHT_NAMES = ("g1", "Wq", "Wk", "Wv", "Wo", "g2", "W1", "W3", "W2")


@dataclass
class LayerInputs:
    x: torch.Tensor     # [T, d]
    dy: torch.Tensor    # [T, d]
    w: dict             # name -> tensor, linear weights [out, in], gains [d]
    Hq: int
    Hkv: int
    dh: int
    F: int
    eps: float


def layer_inputs(T: int, d: int, Hq: int, Hkv: int, dh: int, F: int,
                 dtype: str = "bf16", seed: int = 0, w_std: float = 0.02,
                 gain_std: float = 0.0, eps: float = 1e-6,
                 x_std: float = 1.0, dy_std: float = 1.0, qk_norm: bool = False) -> LayerInputs:
    """Draw order: x, Wq, Wk, Wv, Wo, W1, W3, W2, g1, g2, dy, then (QK-norm)
    qn, kn.

    Gains are exactly one when ``gain_std`` is 0 (the benchmark setting) and
    1 + N(0, gain_std^2) otherwise (to exercise the gain gradients).
    """
    g = _gen(seed)
    tdt = DTYPES[dtype]
    x = _normal(g, (T, d), x_std, tdt)
    shapes = {"Wq": (Hq * dh, d), "Wk": (Hkv * dh, d), "Wv": (Hkv * dh, d),
              "Wo": (d, Hq * dh), "W1": (F, d), "W3": (F, d), "W2": (d, F)}
    w = {}
    for name in ("Wq", "Wk", "Wv", "Wo", "W1", "W3", "W2"):
        w[name] = _normal(g, shapes[name], w_std, tdt)
    for name in ("g1", "g2"):
        gg = torch.ones(d, dtype=torch.float32)
        if gain_std > 0.0:
            gg = gg + gain_std * torch.randn(d, generator=g, dtype=torch.float32)
        w[name] = gg.to(tdt)
    dy = _normal(g, (T, d), dy_std, tdt)
    if qk_norm:
        for name in ("qn", "kn"):
            gg = torch.ones(dh, dtype=torch.float32)
            if gain_std > 0.0:
                gg = gg + gain_std * torch.randn(dh, generator=g, dtype=torch.float32)
            w[name] = gg.to(tdt)
    return LayerInputs(x, dy, w, Hq, Hkv, dh, F, eps)


@dataclass
class ModelInputs:
    x0: torch.Tensor            # [T, d]  output of the embedding lookup
    layers: list                # per layer: name -> tensor, as LayerInputs.w
    g_final: torch.Tensor       # [d]     final RMSNorm gain
    W: torch.Tensor             # [V, d]  LM-head weight
    targets: torch.Tensor       # [T]     int32, < 0 = ignored
    weights: Optional[torch.Tensor]  # [T] fp32 or None
    Hq: int
    Hkv: int
    dh: int
    F: int
    eps: float
    rope_theta: float


def model_inputs(T: int, d: int, Hq: int, Hkv: int, dh: int, F: int, V: int, n_layers: int,
                 dtype: str = "bf16", seed: int = 0, w_std: float = 0.02,
                 gain_std: float = 0.0, eps: float = 1e-6, rope_theta: float = 0.0,
                 ignore_frac: float = 0.0, weighted: bool = False,
                 lm_w_std: Optional[float] = None, qk_norm: bool = False) -> ModelInputs:
    """Draw order: x0; per layer Wq, Wk, Wv, Wo, W1, W3, W2, g1, g2 (then qn,
    kn with QK-norm); g_final; W; targets; per-token weights; random ignore
    mask."""
    g = _gen(seed)
    tdt = DTYPES[dtype]
    x0 = _normal(g, (T, d), 1.0, tdt)
    shapes = {"Wq": (Hq * dh, d), "Wk": (Hkv * dh, d), "Wv": (Hkv * dh, d),
              "Wo": (d, Hq * dh), "W1": (F, d), "W3": (F, d), "W2": (d, F)}

    def gain(n=d):
        gg = torch.ones(n, dtype=torch.float32)
        if gain_std > 0.0:
            gg = gg + gain_std * torch.randn(n, generator=g, dtype=torch.float32)
        return gg.to(tdt)

    layers = []
    for _ in range(n_layers):
        w = {n: _normal(g, shapes[n], w_std, tdt) for n in ("Wq", "Wk", "Wv", "Wo", "W1", "W3", "W2")}
        w["g1"] = gain()
        w["g2"] = gain()
        if qk_norm:
            w["qn"] = gain(dh)
            w["kn"] = gain(dh)
        layers.append(w)
    g_final = gain()
    W = _normal(g, (V, d), w_std if lm_w_std is None else lm_w_std, tdt)
    targets = torch.randint(0, V, (T,), generator=g, dtype=torch.int64).to(torch.int32)
    weights = torch.randn(T, generator=g, dtype=torch.float32) if weighted else None
    if ignore_frac > 0.0:
        targets[torch.rand(T, generator=g) < ignore_frac] = -1
    return ModelInputs(x0, layers, g_final, W, targets, weights, Hq, Hkv, dh, F, eps, rope_theta)


def to_f64(t: Optional[torch.Tensor]):
    """Exact upcast of a CPU tensor to a float64 numpy array (None passes)."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()


# ---------------------------------------------------------------------------
# The five workloads (index 0..4), seed = 1000 + index, the forward-only
# log-probability workload (index 5), packed-sequence variants of the
# attention and layer workloads (6, 7) and a whole-model backward (8).
# ---------------------------------------------------------------------------
WORKLOADS = {
    0: dict(kind="lmhead", name="lmhead_ce_f32_T256_d64_V512_D4",
            T=256, d=64, V=512, D=4, dtype="f32"),
    1: dict(kind="lmhead", name="lmhead_ce_bf16_T32768_d4096_V128256_D16",
            T=32768, d=4096, V=128256, D=16, dtype="bf16", w_std=0.02),
    2: dict(kind="attn", name="attn_bwd_bf16_B1_T16384_Hq32_Hkv8_dh128_D8",
            B=1, T=16384, Hq=32, Hkv=8, dh=128, D=8, dtype="bf16"),
    3: dict(kind="layer", name="layer_bwd_bf16_T65536_d4096_F14336_D16",
            T=65536, d=4096, Hq=32, Hkv=8, dh=128, F=14336, D=16, dtype="bf16"),
    4: dict(kind="lmhead", name="lmhead_ce_weighted_bf16_T131072x8seq_d3584_V152064_D32",
            T=131072, d=3584, V=152064, D=32, dtype="bf16", w_std=0.02,
            n_seq=8, masked_frac=0.25, weighted=True),
    # forward-only per-token log-probability on the weighted workload's
    # shapes (the front end that forms its token weights); not a backward
    5: dict(kind="logprob", name="lmhead_logprob_bf16_T131072x8seq_d3584_V152064_D32",
            T=131072, d=3584, V=152064, D=32, dtype="bf16", w_std=0.02,
            n_seq=8, masked_frac=0.25),
    # workloads 2 and 3 with 8 packed sequences of random lengths
    6: dict(kind="attn", name="attn_bwd_packed_bf16_T16384x8seq_Hq32_Hkv8_dh128_D8",
            B=1, T=16384, Hq=32, Hkv=8, dh=128, D=8, dtype="bf16", n_seq=8),
    7: dict(kind="layer", name="layer_bwd_packed_bf16_T65536x8seq_d4096_F14336_D16",
            T=65536, d=4096, Hq=32, Hkv=8, dh=128, F=14336, D=16, dtype="bf16", n_seq=8),
    # whole-model backward: 4 layers of workload 3's shape with rotary
    # embedding under workload 1's LM head, chunk lengths of those workloads
    8: dict(kind="model", name="model_bwd_bf16_L4_T16384_d4096_F14336_V128256_rope",
            T=16384, d=4096, Hq=32, Hkv=8, dh=128, F=14336, V=128256, n_layers=4,
            D_lm=8, D=4, rope_theta=500000.0, dtype="bf16"),
}


def packed_cuts(T: int, n_seq: int, seed: int):
    """Boundaries 0 = cu[0] < ... < cu[n_seq] = T of n_seq packed sequences:
    n_seq - 1 distinct cut points drawn uniformly from [1, T)."""
    g = _gen(seed)
    cuts = torch.randperm(T - 1, generator=g)[: n_seq - 1] + 1
    return [0] + sorted(int(c) for c in cuts) + [T]


def workload_cu(index: int, T: Optional[int] = None):
    """Sequence boundaries of a packed workload (None if it is not packed);
    seed 2000 + index."""
    cfg = WORKLOADS[index]
    if cfg["kind"] not in ("attn", "layer") or "n_seq" not in cfg:
        return None
    return packed_cuts(cfg["T"] if T is None else T, cfg["n_seq"], 2000 + index)


def workload_inputs(index: int, **override):
    """Inputs of workload ``index`` (seed 1000 + index); sizes may be overridden."""
    cfg = dict(WORKLOADS[index])
    cfg.update(override)
    seed = cfg.get("seed", 1000 + index)
    kind = cfg["kind"]
    if kind in ("lmhead", "logprob"):
        return lmhead_inputs(cfg["T"], cfg["d"], cfg["V"], cfg["dtype"], seed,
                             w_std=cfg.get("w_std"), n_seq=cfg.get("n_seq", 1),
                             masked_frac=cfg.get("masked_frac", 0.0),
                             weighted=cfg.get("weighted", False))
    if kind == "attn":
        return attn_inputs(cfg["B"], cfg["T"], cfg["Hq"], cfg["Hkv"], cfg["dh"],
                           cfg["dtype"], seed)
    if kind == "layer":
        return layer_inputs(cfg["T"], cfg["d"], cfg["Hq"], cfg["Hkv"], cfg["dh"],
                            cfg["F"], cfg["dtype"], seed)
    if kind == "model":
        return model_inputs(cfg["T"], cfg["d"], cfg["Hq"], cfg["Hkv"], cfg["dh"], cfg["F"],
                            cfg["V"], cfg["n_layers"], cfg["dtype"], seed,
                            rope_theta=cfg["rope_theta"])
    raise ValueError(kind)
