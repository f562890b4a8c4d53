"""libstreambp Python binding: argument marshalling over the C ABI.

Every step of the computation runs in the HIP kernels of libstreambp
(``csrc/``); this module only checks tensor shapes/dtypes, allocates the
outputs and the workspace with torch, and passes raw device pointers and the
current HIP stream.  There is no CPU or PyTorch fallback: if the library is
not built, or a tensor is not on the GPU, the call raises.

Names follow ``include/streambp.h``:

* ``lmhead_ce``      -> ``sbp_lmhead_ce_fwd_bwd``
* ``lmhead_logprob`` -> ``sbp_lmhead_logprob_fwd``
* ``attn_bwd``       -> ``sbp_attn_bwd_chunked`` (``sbp_attn_bwd_packed`` with ``cu_seqlens``)
* ``layer_bwd``      -> ``sbp_layer_bwd`` (``sbp_layer_bwd_packed`` with ``cu_seqlens``)
"""
from __future__ import annotations

import ctypes as C
import math
from contextlib import contextmanager
from typing import Dict, List, Optional

import torch

from . import _lib
from ._lib import (SBP_BF16, SBP_F32, SBP_MEAN_VALID, SBP_SUM, LAYER_NAMES, QK_NORM_NAMES, LayerDesc,
                   LayerGrads, LayerWeights, StreamBPError, check, load)

__all__ = ["lmhead_ce", "lmhead_logprob", "attn_bwd", "layer_bwd", "lmhead_ce_workspace_size",
           "lmhead_logprob_workspace_size", "attn_bwd_packed_workspace_size",
           "layer_bwd_packed_workspace_size",
           "attn_bwd_workspace_size", "layer_bwd_workspace_size", "profile", "load",
           "StreamBPError", "chunk_table"]

_DT = {torch.float32: SBP_F32, torch.bfloat16: SBP_BF16}
_RED = {"mean_valid": SBP_MEAN_VALID, "sum": SBP_SUM}


def chunk_table(T: int, D: int):
    """The chunk boundaries the library uses: size = T // D, last chunk to T."""
    if not 1 <= D <= T:
        raise ValueError("need 1 <= D <= T")
    s = T // D
    return [(i * s, (i + 1) * s if i < D - 1 else T) for i in range(D)]


def _dev(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the GPU")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(device) -> C.c_void_p:
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise ValueError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------
def lmhead_ce_workspace_size(T, d, V, D, dtype=torch.bfloat16, dw_group: int = 1) -> int:
    """Workspace bytes of ``lmhead_ce`` when the weight gradient is taken once
    per ``dw_group`` chunks (1: the smallest workspace)."""
    out = C.c_size_t(0)
    check(load().sbp_lmhead_ce_workspace_size_grouped(T, d, V, D, _DT[dtype], int(dw_group),
                                                      C.byref(out)))
    return out.value


def lmhead_ce_max_group(T, D) -> int:
    """The largest weight-gradient group the call uses: about 4096 tokens."""
    tcp = -(-(T - (D - 1) * (T // D)) // 128) * 128
    return max(1, min(D, 4096 // tcp))


def lmhead_ce(H: torch.Tensor, W: torch.Tensor, targets: torch.Tensor,
              weights: Optional[torch.Tensor] = None, D: int = 1,
              reduction: str = "mean_valid", dW: Optional[torch.Tensor] = None,
              accumulate: bool = False, token_loss: bool = False,
              workspace: Optional[torch.Tensor] = None, dw_group: int = 1):
    """Chunked LM head + cross-entropy.  Returns ``(loss, dH, dW, token_loss)``.

    ``loss`` is a 1-element fp32 tensor; ``token_loss`` is None unless asked.
    ``dW`` may be passed in (fp32 [V, d]) to accumulate into it.
    ``dw_group``: chunks per weight-gradient GEMM the allocated workspace is
    sized for (1: least memory; the call uses the largest group a given
    ``workspace`` holds, up to about 4096 tokens).
    """
    lib = load()
    _dev(H, W, targets, weights, dW)
    T, d = H.shape
    V = W.shape[0]
    if W.shape[1] != d or W.dtype != H.dtype or targets.shape != (T,) or targets.dtype != torch.int32:
        raise ValueError("shape/dtype mismatch")
    if weights is not None and (weights.shape != (T,) or weights.dtype != torch.float32):
        raise ValueError("weights must be fp32 [T]")
    dt = _dtype(H)
    dev = H.device
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    dH = torch.empty_like(H)
    if dW is None:
        dW = torch.empty(V, d, dtype=torch.float32, device=dev)
    elif dW.shape != (V, d) or dW.dtype != torch.float32:
        raise ValueError("dW must be fp32 [V, d]")
    tl = torch.empty(T, dtype=torch.float32, device=dev) if token_loss else None
    nb = lmhead_ce_workspace_size(T, d, V, D, H.dtype, dw_group)
    ws = workspace if workspace is not None and workspace.numel() >= nb else _ws(nb, dev)
    check(lib.sbp_lmhead_ce_fwd_bwd(_ptr(H), _ptr(W), _ptr(targets), _ptr(weights), T, d, V, D,
                                    dt, _RED[reduction], int(accumulate), _ptr(loss), _ptr(tl),
                                    _ptr(dH), _ptr(dW), _ptr(ws), ws.numel(), _stream(dev)))
    return loss, dH, dW, tl


def lmhead_logprob_workspace_size(T, d, V, D, dtype=torch.bfloat16) -> int:
    out = C.c_size_t(0)
    check(load().sbp_lmhead_logprob_workspace_size(T, d, V, D, _DT[dtype], C.byref(out)))
    return out.value


def lmhead_logprob(H: torch.Tensor, W: torch.Tensor, targets: torch.Tensor, D: int = 1,
                   lse: bool = False, workspace: Optional[torch.Tensor] = None):
    """Chunked forward-only per-token target log-probability.

    Returns ``(logprob, lse)``: fp32 [T] each (``lse`` is None unless asked);
    both are 0 for ignored tokens (target < 0).
    """
    lib = load()
    _dev(H, W, targets)
    T, d = H.shape
    V = W.shape[0]
    if W.shape[1] != d or W.dtype != H.dtype or targets.shape != (T,) or targets.dtype != torch.int32:
        raise ValueError("shape/dtype mismatch")
    dt = _dtype(H)
    dev = H.device
    lp = torch.empty(T, dtype=torch.float32, device=dev)
    ls = torch.empty(T, dtype=torch.float32, device=dev) if lse else None
    nb = lmhead_logprob_workspace_size(T, d, V, D, H.dtype)
    ws = workspace if workspace is not None and workspace.numel() >= nb else _ws(nb, dev)
    check(lib.sbp_lmhead_logprob_fwd(_ptr(H), _ptr(W), _ptr(targets), T, d, V, D, dt, _ptr(lp),
                                     _ptr(ls), _ptr(ws), ws.numel(), _stream(dev)))
    return lp, ls


# ----------------------------------------------------------------------------
def attn_bwd_workspace_size(B, T, Hq, Hkv, dh, D, dtype=torch.bfloat16) -> int:
    out = C.c_size_t(0)
    check(load().sbp_attn_bwd_workspace_size(B, T, Hq, Hkv, dh, D, _DT[dtype], C.byref(out)))
    return out.value


def attn_bwd_packed_workspace_size(T, Hq, Hkv, dh, D, dtype=torch.bfloat16) -> int:
    out = C.c_size_t(0)
    check(load().sbp_attn_bwd_packed_workspace_size(T, Hq, Hkv, dh, D, _DT[dtype], C.byref(out)))
    return out.value


def attn_bwd(Q, K, V, dO, D: int = 1, scale: Optional[float] = None, O=None, lse=None,
             dK: Optional[torch.Tensor] = None, dV: Optional[torch.Tensor] = None,
             accumulate: bool = False, workspace: Optional[torch.Tensor] = None,
             cu_seqlens: Optional[torch.Tensor] = None):
    """Chunked causal GQA attention backward.  Returns ``(dQ, dK, dV)``;
    dK/dV are fp32.  Layout [B, T, heads, dh].

    ``cu_seqlens`` (int32 [nseq + 1] on the GPU, B = 1): packed independent
    sequences [cu[n], cu[n+1]); a query then sees only keys of its own
    sequence (``sbp_attn_bwd_packed``)."""
    lib = load()
    _dev(Q, K, V, dO, O, lse, dK, dV, cu_seqlens)
    B, T, Hq, dh = Q.shape
    Hkv = K.shape[2]
    if K.shape != (B, T, Hkv, dh) or V.shape != K.shape or dO.shape != Q.shape:
        raise ValueError("shape mismatch")
    if not (Q.dtype == K.dtype == V.dtype == dO.dtype):
        raise ValueError("dtype mismatch")
    if cu_seqlens is not None and (B != 1 or cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1
                                   or cu_seqlens.numel() < 2):
        raise ValueError("cu_seqlens must be int32 [nseq + 1] with B = 1")
    dt = _dtype(Q)
    dev = Q.device
    if scale is None:
        scale = 1.0 / math.sqrt(dh)
    dQ = torch.empty_like(Q)
    if dK is None:
        dK = torch.empty(B, T, Hkv, dh, dtype=torch.float32, device=dev)
    if dV is None:
        dV = torch.empty(B, T, Hkv, dh, dtype=torch.float32, device=dev)
    if cu_seqlens is None:
        nb = attn_bwd_workspace_size(B, T, Hq, Hkv, dh, D, Q.dtype)
    else:
        nb = attn_bwd_packed_workspace_size(T, Hq, Hkv, dh, D, Q.dtype)
    ws = workspace if workspace is not None and workspace.numel() >= nb else _ws(nb, dev)
    if cu_seqlens is None:
        check(lib.sbp_attn_bwd_chunked(_ptr(Q), _ptr(K), _ptr(V), _ptr(dO), _ptr(O), _ptr(lse), B,
                                       T, Hq, Hkv, dh, float(scale), D, dt, int(accumulate),
                                       _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(ws), ws.numel(),
                                       _stream(dev)))
    else:
        check(lib.sbp_attn_bwd_packed(_ptr(Q), _ptr(K), _ptr(V), _ptr(dO), _ptr(O), _ptr(lse),
                                      _ptr(cu_seqlens), cu_seqlens.numel() - 1, T, Hq, Hkv, dh,
                                      float(scale), D, dt, int(accumulate), _ptr(dQ), _ptr(dK),
                                      _ptr(dV), _ptr(ws), ws.numel(), _stream(dev)))
    return dQ, dK, dV


# ----------------------------------------------------------------------------
def _desc(T, d, Hq, Hkv, dh, F, eps, dtype, rope_theta=0.0, qk_norm=False) -> LayerDesc:
    return LayerDesc(T, d, Hq, Hkv, dh, F, eps, _DT[dtype], float(rope_theta), int(bool(qk_norm)))


def _names(weights) -> tuple:
    """The weight names a layer uses: the nine always, qn / kn with QK-norm."""
    return LAYER_NAMES + QK_NORM_NAMES if "qn" in weights else LAYER_NAMES


def _wstruct(weights) -> LayerWeights:
    return LayerWeights(*[weights[n].data_ptr() if n in weights else None
                          for n in LAYER_NAMES + QK_NORM_NAMES])


def _gstruct(grads) -> LayerGrads:
    return LayerGrads(*[grads[n].data_ptr() if n in grads else None
                        for n in LAYER_NAMES + QK_NORM_NAMES])


def layer_bwd_workspace_size(T, d, Hq, Hkv, dh, F, D, dtype=torch.bfloat16, eps=1e-6,
                             rope_theta=0.0, qk_norm=False) -> int:
    out = C.c_size_t(0)
    desc = _desc(T, d, Hq, Hkv, dh, F, eps, dtype, rope_theta, qk_norm)
    check(load().sbp_layer_bwd_workspace_size(C.byref(desc), D, C.byref(out)))
    return out.value


def layer_bwd_packed_workspace_size(T, d, Hq, Hkv, dh, F, D, dtype=torch.bfloat16,
                                    eps=1e-6, rope_theta=0.0, qk_norm=False) -> int:
    out = C.c_size_t(0)
    desc = _desc(T, d, Hq, Hkv, dh, F, eps, dtype, rope_theta, qk_norm)
    check(load().sbp_layer_bwd_packed_workspace_size(C.byref(desc), D, C.byref(out)))
    return out.value


def layer_bwd(x, dy, weights: Dict[str, torch.Tensor], Hq: int, Hkv: int, dh: int,
              eps: float = 1e-6, D: int = 1, grads: Optional[Dict[str, torch.Tensor]] = None,
              accumulate: bool = False, workspace: Optional[torch.Tensor] = None,
              cu_seqlens: Optional[torch.Tensor] = None, rope_theta: float = 0.0):
    """Streamed backward of one pre-norm decoder layer.  Returns ``(dx, grads)``
    with fp32 weight/gain gradients keyed like ``weights``.  ``cu_seqlens``
    (int32 [nseq + 1] on the GPU): packed independent sequences
    (``sbp_layer_bwd_packed``).  ``rope_theta`` > 0: rotary embedding of q
    and k with that base."""
    lib = load()
    _dev(x, dy, cu_seqlens, *weights.values())
    if cu_seqlens is not None and (cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1
                                   or cu_seqlens.numel() < 2):
        raise ValueError("cu_seqlens must be int32 [nseq + 1]")
    T, d = x.shape
    F = weights["W1"].shape[0]
    dev = x.device
    dt = x.dtype
    names = _names(weights)
    qk = "qn" in weights
    if grads is None:
        grads = {n: torch.empty(weights[n].shape, dtype=torch.float32, device=dev) for n in names}
    _dev(*grads.values())
    for n in names:
        if weights[n].dtype != dt or grads[n].dtype != torch.float32 or grads[n].shape != weights[n].shape:
            raise ValueError(f"bad weight/grad {n}")
    dx = torch.empty_like(x)
    desc = _desc(T, d, Hq, Hkv, dh, F, eps, dt, rope_theta, qk)
    wst = _wstruct(weights)
    gst = _gstruct(grads)
    if cu_seqlens is None:
        nb = layer_bwd_workspace_size(T, d, Hq, Hkv, dh, F, D, dt, eps, rope_theta, qk)
    else:
        nb = layer_bwd_packed_workspace_size(T, d, Hq, Hkv, dh, F, D, dt, eps, rope_theta, qk)
    ws = workspace if workspace is not None and workspace.numel() >= nb else _ws(nb, dev)
    if cu_seqlens is None:
        check(lib.sbp_layer_bwd(C.byref(desc), _ptr(x), _ptr(dy), C.byref(wst), D,
                                int(accumulate), _ptr(dx), C.byref(gst), _ptr(ws), ws.numel(),
                                _stream(dev)))
    else:
        check(lib.sbp_layer_bwd_packed(C.byref(desc), _ptr(cu_seqlens), cu_seqlens.numel() - 1,
                                       _ptr(x), _ptr(dy), C.byref(wst), D, int(accumulate),
                                       _ptr(dx), C.byref(gst), _ptr(ws), ws.numel(),
                                       _stream(dev)))
    return dx, grads


def layer_fwd_workspace_size(T, d, Hq, Hkv, dh, F, D, dtype=torch.bfloat16, eps=1e-6,
                             rope_theta=0.0, qk_norm=False) -> int:
    out = C.c_size_t(0)
    desc = _desc(T, d, Hq, Hkv, dh, F, eps, dtype, rope_theta, qk_norm)
    check(load().sbp_layer_fwd_workspace_size(C.byref(desc), D, C.byref(out)))
    return out.value


def layer_fwd(x, weights: Dict[str, torch.Tensor], Hq: int, Hkv: int, dh: int,
              eps: float = 1e-6, D: int = 1, cu_seqlens: Optional[torch.Tensor] = None,
              rope_theta: float = 0.0, out: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None):
    """Chunked forward of one pre-norm decoder layer (``sbp_layer_fwd``);
    returns ``y`` [T, d] in x's dtype."""
    lib = load()
    _dev(x, cu_seqlens, *weights.values())
    if cu_seqlens is not None and (cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1
                                   or cu_seqlens.numel() < 2):
        raise ValueError("cu_seqlens must be int32 [nseq + 1]")
    T, d = x.shape
    F = weights["W1"].shape[0]
    dt = x.dtype
    for n in _names(weights):
        if weights[n].dtype != dt:
            raise ValueError(f"bad weight {n}")
    y = torch.empty_like(x) if out is None else out
    if y.shape != x.shape or y.dtype != dt:
        raise ValueError("out must match x")
    _dev(y)
    desc = _desc(T, d, Hq, Hkv, dh, F, eps, dt, rope_theta, "qn" in weights)
    wst = _wstruct(weights)
    nb = layer_fwd_workspace_size(T, d, Hq, Hkv, dh, F, D, dt, eps, rope_theta, "qn" in weights)
    ws = workspace if workspace is not None and workspace.numel() >= nb else _ws(nb, x.device)
    nseq = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    check(lib.sbp_layer_fwd(C.byref(desc), _ptr(cu_seqlens), nseq, _ptr(x), C.byref(wst), D,
                            _ptr(y), _ptr(ws), ws.numel(), _stream(x.device)))
    return y


# ----------------------------------------------------------------------------
def model_fwd(x0: torch.Tensor, layers: List[Dict[str, torch.Tensor]], Hq: int, Hkv: int,
              dh: int, eps: float = 1e-6, D: int = 1, cu_seqlens: Optional[torch.Tensor] = None,
              rope_theta: float = 0.0) -> List[torch.Tensor]:
    """Forward through a stack of layers (one ``sbp_layer_fwd`` per layer);
    returns ``[x_0, ..., x_L]``, the inputs ``sbp_model_bwd`` starts from."""
    xs = [x0]
    ws = None
    for w in layers:
        if ws is None:
            T, d = x0.shape
            nb = layer_fwd_workspace_size(T, d, Hq, Hkv, dh, w["W1"].shape[0], D, x0.dtype, eps,
                                          rope_theta, "qn" in w)
            ws = _ws(nb, x0.device)
        xs.append(layer_fwd(xs[-1], w, Hq, Hkv, dh, eps, D, cu_seqlens, rope_theta, workspace=ws))
    return xs


def model_bwd_workspace_size(T, d, Hq, Hkv, dh, F, n_layers, V, D_lm, D_layer, packed=False,
                             dtype=torch.bfloat16, eps=1e-6, rope_theta=0.0, qk_norm=False) -> int:
    out = C.c_size_t(0)
    desc = _desc(T, d, Hq, Hkv, dh, F, eps, dtype, rope_theta, qk_norm)
    check(load().sbp_model_bwd_workspace_size(C.byref(desc), n_layers, int(packed), V, D_lm,
                                              D_layer, C.byref(out)))
    return out.value


def model_bwd(xs: List[torch.Tensor], layers: List[Dict[str, torch.Tensor]],
              g_final: torch.Tensor, W_lm: torch.Tensor, targets: torch.Tensor,
              weights: Optional[torch.Tensor] = None, *, Hq: int, Hkv: int, dh: int,
              eps: float = 1e-6, D_lm: int = 1, D_layer: int = 1,
              reduction: str = "mean_valid", cu_seqlens: Optional[torch.Tensor] = None,
              rope_theta: float = 0.0, grads: Optional[List[Dict[str, torch.Tensor]]] = None,
              dg_final: Optional[torch.Tensor] = None, dW_lm: Optional[torch.Tensor] = None,
              accumulate: bool = False, token_loss: bool = False,
              workspace: Optional[torch.Tensor] = None):
    """Streamed backward of a whole model (``sbp_model_bwd``) from the layer
    inputs ``xs = [x_0, ..., x_L]`` (``model_fwd``).  Returns ``(loss, dx0,
    grads, dg_final, dW_lm, token_loss)`` with fp32 gradients."""
    lib = load()
    L = len(layers)
    if len(xs) != L + 1:
        raise ValueError("xs must hold the L inputs and the last output")
    _dev(*xs, g_final, W_lm, targets, weights, cu_seqlens, dg_final, dW_lm)
    T, d = xs[0].shape
    V = W_lm.shape[0]
    dev, dt = xs[0].device, xs[0].dtype
    for x in xs:
        if x.shape != (T, d) or x.dtype != dt:
            raise ValueError("every x must be [T, d] of one dtype")
    if W_lm.shape != (V, d) or W_lm.dtype != dt or g_final.shape != (d,) or g_final.dtype != dt:
        raise ValueError("bad W_lm / g_final")
    if targets.shape != (T,) or targets.dtype != torch.int32:
        raise ValueError("targets must be int32 [T]")
    if weights is not None and (weights.shape != (T,) or weights.dtype != torch.float32):
        raise ValueError("weights must be fp32 [T]")
    if cu_seqlens is not None and (cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1
                                   or cu_seqlens.numel() < 2):
        raise ValueError("cu_seqlens must be int32 [nseq + 1]")
    F = layers[0]["W1"].shape[0] if L else 8
    Hd = (Hq, Hkv, dh)
    qk = L > 0 and "qn" in layers[0]
    if grads is None:
        grads = [{n: torch.empty(w[n].shape, dtype=torch.float32, device=dev) for n in _names(w)}
                 for w in layers]
    for w, g in zip(layers, grads):
        _dev(*w.values(), *g.values())
        if ("qn" in w) != qk:
            raise ValueError("every layer must have QK-norm gains, or none")
        for n in _names(w):
            if w[n].dtype != dt or g[n].dtype != torch.float32 or g[n].shape != w[n].shape:
                raise ValueError(f"bad weight/grad {n}")
    if dg_final is None:
        dg_final = torch.empty(d, dtype=torch.float32, device=dev)
    if dW_lm is None:
        dW_lm = torch.empty(V, d, dtype=torch.float32, device=dev)
    if dg_final.shape != (d,) or dW_lm.shape != (V, d):
        raise ValueError("bad dg_final / dW_lm")
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    tl = torch.empty(T, dtype=torch.float32, device=dev) if token_loss else None
    dx0 = torch.empty_like(xs[0])
    desc = _desc(T, d, *Hd, F, eps, dt, rope_theta, qk)
    nb = model_bwd_workspace_size(T, d, *Hd, F, L, V, D_lm, D_layer, cu_seqlens is not None, dt,
                                  eps, rope_theta, qk)
    ws = workspace if workspace is not None and workspace.numel() >= nb else _ws(nb, dev)
    xp = (C.c_void_p * (L + 1))(*[x.data_ptr() for x in xs])
    wa = (LayerWeights * max(L, 1))(*[_wstruct(w) for w in layers])
    ga = (LayerGrads * max(L, 1))(*[_gstruct(g) for g in grads])
    nseq = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    check(lib.sbp_model_bwd(C.byref(desc), L, _ptr(cu_seqlens), nseq, xp, wa, _ptr(g_final),
                            _ptr(W_lm), V, _ptr(targets), _ptr(weights), _RED[reduction], D_lm,
                            D_layer, int(accumulate), _ptr(loss), _ptr(tl), _ptr(dx0), ga,
                            _ptr(dg_final), _ptr(dW_lm), _ptr(ws), ws.numel(), _stream(dev)))
    return loss, dx0, grads, dg_final, dW_lm, tl


# ----------------------------------------------------------------------------
@contextmanager
def profile(max_launches: int = 65536):
    """Per-kernel timing of every library launch inside the block.

    Yields a dict that, after the block, maps kernel name ->
    ``{"launches", "ms", "flops", "bytes"}`` (totals over the block)."""
    lib = load()
    res: Dict[str, dict] = {}
    check(lib.sbp_profile_begin(max_launches))
    try:
        yield res
    finally:
        n = C.c_int32(0)
        check(lib.sbp_profile_end(C.byref(n)))
        for i in range(n.value):
            name = C.c_char_p()
            L, ms, fl, by = C.c_int64(), C.c_double(), C.c_double(), C.c_double()
            check(lib.sbp_profile_entry(i, C.byref(name), C.byref(L), C.byref(ms), C.byref(fl),
                                        C.byref(by)))
            res[name.value.decode()] = {"launches": L.value, "ms": ms.value, "flops": fl.value,
                                        "bytes": by.value}
