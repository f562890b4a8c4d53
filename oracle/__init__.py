"""CPU oracle for the StreamBP hot path -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The library (``libstreambp`` and its
Python binding) never imports, links or calls it, and it imports nothing from
the library: the two share no code.

What it computes: the plain definition of the gradient of the *unchunked*
objective, in float64 with NumPy.  StreamBP claims to reach exactly this
result with less memory (StreamBP skill page, "Architecture Overview", the
"Exact Gradients" item; arXiv abstract as quoted on the tomesphere and
mlsanity pages: "memory-efficient and exact BP method").  So the oracle is a
full, unchunked backpropagation, written from the definitions, not from the
chunked algorithm:

* ``lmhead.lmhead_ce``      -- LM head + softmax cross-entropy loss and
  gradients dH, dW (skill page, "Implementation": the per-token cross-entropy,
  the softmax-minus-one-hot logits gradient and the linear-layer gradients).
* ``lmhead.lmhead_logprob`` -- forward-only per-token target log-probability
  and log-sum-exp, the quantity GRPO and DPO weights are formed from (skill
  page, "Practical Guidance", "Loss Objectives").
* ``attention.attn_bwd``    -- causal GQA attention forward and backward;
  ``attn_bwd_packed`` the same over packed independent sequences.
* ``layer.layer_bwd``       -- one pre-norm decoder layer, forward and
  backward by the chain rule, optionally with the rotary position embedding
  of q and k (``layer.rope``).
* ``model.model_bwd``       -- a stack of layers under a final RMSNorm and the
  LM head with cross-entropy: loss and every gradient (skill page,
  "Architecture Overview", "Layer-Wise Application").
* ``chunked``               -- a separate fp64 *chunked* evaluation of the
  same three functions (sequence decomposition of the skill page's
  "Implementation"), used only to show that chunking is algebraically exact
  (D-invariance); it is not the parity reference.

Parity pins: every function is checked in ``tests/test_oracle_*.py`` against
central finite differences, against independent torch fp64 autograd, against
closed forms and special cases, and against hand-derived golden values.
No function here is "parity unpinned".
"""
from .lmhead import lmhead_ce, lmhead_ce_rows, lmhead_dW_rows, lmhead_logprob, lmhead_logprob_rows
from .attention import attn_fwd, attn_bwd, attn_bwd_sampled, attn_bwd_packed
from .layer import layer_fwd, layer_bwd, rmsnorm_fwd, rmsnorm_bwd, rope, rope_positions
from .model import model_fwd, model_bwd, model_bwd_at
from . import chunked

__all__ = ["lmhead_ce", "lmhead_ce_rows", "lmhead_dW_rows", "lmhead_logprob", "lmhead_logprob_rows", "attn_fwd", "attn_bwd",
           "attn_bwd_sampled", "attn_bwd_packed", "layer_fwd", "layer_bwd", "rmsnorm_fwd",
           "rmsnorm_bwd", "rope", "rope_positions", "model_fwd", "model_bwd", "model_bwd_at", "chunked"]
