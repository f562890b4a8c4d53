"""A stack of decoder layers under a final RMSNorm and the LM head with
softmax cross-entropy: loss and every gradient, fp64, unchunked.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources: StreamBP skill page, "Architecture Overview" (the "Layer-Wise
Application" item: the sequence-chunked backward is applied layer by layer
through the model) and "Implementation" (the LM-head logits gradient, and the
streaming layer backward that starts from the input each layer kept from
the forward pass).  The pages give no model beyond that; the plain reading of
a decoder-only language model is used, the embedding lookup left to the
caller (its gradient is a scatter-add of the rows of dx0)::

    x_{l+1} = Layer_l(x_l),   l = 0 .. L-1      (layer.layer_fwd)
    h       = RMSNorm(x_L; g_f)                  (same eps as the layers)
    loss    = CE(h W^T; targets, weights)        (lmhead.lmhead_ce)

Backward by the chain rule: dh from the LM head, dx_L = RMSNorm'(dh), then
dx_l from Layer_l's backward at upstream dx_{l+1}, for l = L-1 .. 0.
"""
from __future__ import annotations

import numpy as np

from .layer import layer_bwd, layer_fwd, rmsnorm_bwd, rmsnorm_fwd
from .lmhead import lmhead_ce


def model_fwd(x0, layers, Hq, Hkv, dh, eps, cu_seqlens=None, rope_theta=0.0):
    """Inputs of every layer and the last output: ``[x_0, ..., x_L]``."""
    xs = [np.asarray(x0, dtype=np.float64)]
    for w in layers:
        y, _ = layer_fwd(xs[-1], w, Hq, Hkv, dh, eps, cu_seqlens, rope_theta)
        xs.append(y)
    return xs


def model_bwd(x0, layers, g_f, W, targets, weights=None, reduction="mean_valid", *, Hq, Hkv,
              dh, eps, cu_seqlens=None, rope_theta=0.0):
    """Returns ``(loss, dx0, layer_grads, dg_f, dW)``; ``layer_grads[l]`` maps
    the names of ``layers[l]`` to their gradients."""
    xs = model_fwd(x0, layers, Hq, Hkv, dh, eps, cu_seqlens, rope_theta)
    return model_bwd_at(xs, layers, g_f, W, targets, weights, reduction, Hq=Hq, Hkv=Hkv, dh=dh,
                        eps=eps, cu_seqlens=cu_seqlens, rope_theta=rope_theta)


def model_bwd_at(xs, layers, g_f, W, targets, weights=None, reduction="mean_valid", *, Hq, Hkv,
                 dh, eps, cu_seqlens=None, rope_theta=0.0):
    """The same chain rule evaluated at given layer inputs ``xs = [x_0, ...,
    x_L]`` (kept from a forward pass): the loss and dx_L at x_L, then each
    layer's backward at its own input x_l with upstream dx_{l+1}.  This is
    what a streamed backward from stored layer inputs computes; it equals
    ``model_bwd`` when ``xs[l+1] = Layer_l(xs[l])`` exactly, and otherwise
    (inputs from a lower-precision forward) it is the exact backward at the
    inputs actually given."""
    xs = [np.asarray(x, dtype=np.float64) for x in xs]
    if len(xs) != len(layers) + 1:
        raise ValueError("xs must hold L + 1 arrays")
    h, _, _ = rmsnorm_fwd(xs[-1], g_f, eps)
    loss, dh_, dW, _, _ = lmhead_ce(h, W, targets, weights, reduction)
    dx, dg_f = rmsnorm_bwd(xs[-1], g_f, dh_, eps)
    grads = [None] * len(layers)
    for l in reversed(range(len(layers))):
        dx, grads[l], _ = layer_bwd(xs[l], dx, layers[l], Hq, Hkv, dh, eps, cu_seqlens,
                                    rope_theta)
    return loss, dx, grads, dg_f, dW
