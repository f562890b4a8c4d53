/*
 * libstreambp -- sequence-chunked exact backward (StreamBP) for MI355X (gfx950).
 *
 * The method (StreamBP pages: the skill page "StreamBP: Memory-Efficient
 * Backpropagation", sections "Core Concept", "Architecture Overview" and
 * "Implementation"; the arXiv abstract quoted on the tomesphere and mlsanity
 * pages): the chain rule of a layer is split linearly along the sequence into
 * D chunks.  Each chunk's activations are (re)computed and back-propagated on
 * their own, weight gradients are summed over the chunks, and the result is
 * the exact gradient of the unchunked objective.  Causal attention makes a
 * query chunk depend only on its key prefix.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.   Every array argument is a DEVICE pointer (HIP device memory of
 *             the current device), except `desc`, `weights` and `grads`
 *             structs and `bytes` out-params, which are HOST pointers.  All
 *             device pointers must be 16-byte aligned.  Arrays are dense and
 *             row-major with the shapes given below; weights are stored
 *             [out, in] (y = x W^T).
 * Ownership.  The caller owns every buffer, including the workspace `ws`
 *             (size from the matching *_workspace_size call).  The library
 *             allocates no device memory, keeps no pointer after a call
 *             returns, and holds no state between calls besides the
 *             thread-local error text and the optional profiler.
 * Streams.    `stream` is a hipStream_t passed as void* (NULL = the legacy
 *             default stream).  Every call only enqueues work on `stream`
 *             and returns; no host synchronisation.  Outputs are valid once
 *             the stream reaches that point.  Two calls that share a
 *             workspace must be ordered on one stream.
 * Chunks.     D chunks of a length-T sequence (skill page, "Implementation",
 *             the sequence decomposition): size = T / D (integer division);
 *             chunk i is [i*size, (i+1)*size), the last chunk ends at T.
 *             1 <= D <= T is required.  Results do not depend on D beyond
 *             floating-point summation order.
 * Precision.  dtype SBP_F32: every tensor fp32.  SBP_BF16: activations,
 *             weights and activation gradients (dH, dQ, dx) bf16; products
 *             accumulate in fp32; weight gradients, dK/dV and gain gradients
 *             are always fp32.
 * Accumulate. accumulate = 1 adds into the fp32 gradient outputs (dW, dK,
 *             dV, the layer's weight and gain gradients) -- gradient
 *             accumulation over micro-batches, which the skill page's
 *             "Practical Guidance" calls orthogonal to StreamBP;
 *             accumulate = 0 overwrites them.  Activation gradients (dH, dQ,
 *             dx) are always overwritten.
 * Errors.     Arguments are checked before anything is enqueued; a bad
 *             argument returns SBP_ERR_INVALID_ARG / SBP_ERR_UNSUPPORTED /
 *             SBP_ERR_WORKSPACE with a message in sbp_last_error() (per host
 *             thread) and touches no output.  A failed kernel launch returns
 *             SBP_ERR_HIP; outputs are then unspecified.  No C++ exception
 *             crosses this interface.
 */
#ifndef STREAMBP_H
#define STREAMBP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SBP_OK = 0,
  SBP_ERR_INVALID_ARG = 1, /* null / misaligned pointer, bad size, D out of range */
  SBP_ERR_UNSUPPORTED = 2, /* valid but not implemented (head dim, dtype, alignment of a size) */
  SBP_ERR_WORKSPACE = 3,   /* ws_bytes smaller than the *_workspace_size result */
  SBP_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} sbp_status;

typedef enum { SBP_F32 = 0, SBP_BF16 = 1 } sbp_dtype;

typedef enum {
  SBP_MEAN_VALID = 0, /* divide by N = number of tokens with target >= 0 */
  SBP_SUM = 1         /* N = 1 */
} sbp_reduction;

/* ------------------------------------------------------------------------
 * 1. LM head + softmax cross-entropy, forward and backward.
 *
 * Passage: skill page, "Implementation" -- the logits-gradient routine
 * (per-token cross-entropy; softmax with one subtracted at the target) and
 * the linear-layer chunk gradient (weight gradient from activations and
 * upstream gradient, input gradient from upstream gradient and weight);
 * "Core Concept" / arXiv abstract: the memory of the logits is what
 * StreamBP removes.  Per chunk the [T_c, V] logits are formed, consumed and
 * dropped; the full [T, V] logits never exist.
 *
 *   Z = H W^T,  l_t = logsumexp(Z_t) - Z_{t,y_t},  c_t = w_t [y_t >= 0]
 *   loss = (1/N) sum_t c_t l_t          (N: see sbp_reduction; N = 0 -> 0)
 *   dZ_t = (c_t/N) (softmax(Z_t) - e_{y_t}),  dH = dZ W,  dW (+)= dZ^T H
 *
 * H        [T, d]   dtype       hidden states
 * W        [V, d]   dtype       LM-head weight
 * targets  [T]      int32       target ids in [0, V); < 0 = ignored token.
 *                               An id >= V is a caller error: without debug
 *                               mode nothing is read out of bounds and the
 *                               loss, dH and dW come out NaN (token_loss of
 *                               that token NaN); debug mode rejects it before
 *                               any launch (SBP_ERR_INVALID_ARG)
 * weights  [T]      fp32 or NULL  per-token weights w_t (GRPO advantage, DPO
 *                               sequence weight); NULL = all ones
 * loss     [1]      fp32 out    the loss above
 * token_loss [T]    fp32 out or NULL  unweighted per-token l_t (0 if ignored)
 * dH       [T, d]   dtype out   (ignored tokens give zero rows)
 * dW       [V, d]   fp32 out    accumulate semantics as above
 * Requires d % 8 == 0 (bf16) or d % 4 == 0 (f32), V >= 1, T >= 1.
 * Chunks with no valid token are skipped on the device (their dH rows are
 * zero-filled).
 * ---------------------------------------------------------------------- */
sbp_status sbp_lmhead_ce_workspace_size(int64_t T, int64_t d, int64_t V, int32_t D,
                                        int32_t dtype, size_t* bytes);

/* Workspace size when the weight gradient is taken once per group of G
 * consecutive chunks (G >= 1; dW += dZ_g^T H_g over the group's tokens).
 * The call uses the largest G whose workspace fits in ws_bytes, up to a
 * group of about 4096 tokens (G <= max(1, 4096 / (T_c rounded up to 128)));
 * sbp_lmhead_ce_workspace_size is this size for G = 1, the smallest
 * workspace, which falls with D.  A larger G holds G chunks of dZ (G T_c V
 * bf16) and makes the weight-gradient GEMM longer in K, so its fp32
 * read-modify-write of dW is paid once per group. */
sbp_status sbp_lmhead_ce_workspace_size_grouped(int64_t T, int64_t d, int64_t V, int32_t D,
                                                int32_t dtype, int32_t G, size_t* bytes);

sbp_status sbp_lmhead_ce_fwd_bwd(const void* H, const void* W, const int32_t* targets,
                                 const float* weights, int64_t T, int64_t d, int64_t V,
                                 int32_t D, int32_t dtype, int32_t reduction,
                                 int32_t accumulate, float* loss, float* token_loss,
                                 void* dH, float* dW, void* ws, size_t ws_bytes,
                                 void* stream);

/* ------------------------------------------------------------------------
 * 1b. LM head, forward only: per-token target log-probability.
 *
 * Passage: skill page, "Practical Guidance", "Loss Objectives" -- StreamBP
 * serves GRPO and DPO as well as SFT.  Their per-token weights (a policy
 * ratio, a sequence log-likelihood) are formed from the log-probability the
 * model gives each target token; the caller forms them from this call's
 * output and passes them as `weights` to sbp_lmhead_ce_fwd_bwd.  Chunked as
 * in (1): per chunk the [T_c, V] logits are reduced as they are produced
 * and never stored whole (with bf16 and d % 128 == 0 they are not written to
 * memory at all).
 *
 *   Z = H W^T,  lse_t = logsumexp(Z_t),  logprob_t = Z_{t,y_t} - lse_t
 *
 * H, W, targets  as in (1)
 * logprob  [T]      fp32 out    logprob_t; 0 for ignored tokens (y_t < 0);
 *                               NaN for an id >= V (caller error; rejected
 *                               before any launch in debug mode)
 * lse      [T]      fp32 out or NULL  lse_t; 0 for ignored tokens, NaN for ids >= V
 * Chunks with no valid token are skipped on the device.
 * ---------------------------------------------------------------------- */
sbp_status sbp_lmhead_logprob_workspace_size(int64_t T, int64_t d, int64_t V, int32_t D,
                                             int32_t dtype, size_t* bytes);

sbp_status sbp_lmhead_logprob_fwd(const void* H, const void* W, const int32_t* targets,
                                  int64_t T, int64_t d, int64_t V, int32_t D, int32_t dtype,
                                  float* logprob, float* lse, void* ws, size_t ws_bytes,
                                  void* stream);

/* ------------------------------------------------------------------------
 * 2. Causal GQA attention backward, chunked over queries.
 *
 * Passage: skill page, "Architecture Overview" (causal structure
 * exploitation) and "Practical Guidance" (masks across chunk boundaries;
 * causal masking); arXiv abstract: the causal structure lowers the FLOPs.
 * Query chunk c = [s_c, e_c) reads keys/values [0, e_c) only; key blocks
 * that lie entirely above the diagonal are never visited.  Chunks run in
 * reverse order; dK/dV are accumulated in fp32 across chunks and across the
 * G = Hq/Hkv query heads of a group (query head h uses kv head h / G).
 *
 *   S = scale Q K^T (key j visible to query i iff j <= i), P = softmax(S),
 *   O = P V, dV = P^T dO, dP = dO V^T, dS = P (dP - rowsum(dO O)),
 *   dQ = scale dS K, dK = scale dS^T Q
 *
 * Q, dO  [B, T, Hq, dh]  dtype     K, V  [B, T, Hkv, dh]  dtype
 * O      [B, T, Hq, dh]  dtype or NULL   forward output; with `lse`, skips
 * lse    [B, T, Hq]      fp32 or NULL    the forward recomputation (both or
 *                                        neither; natural-log log-sum-exp of
 *                                        the scaled scores)
 * dQ     [B, T, Hq, dh]  dtype out
 * dK, dV [B, T, Hkv, dh] fp32 out  (accumulate semantics)
 * Supported: dtype SBP_BF16 or SBP_F32 (fp32: every array fp32, every
 * product an fp32 multiply-add); dh in {64, 128}; Hq % Hkv == 0.
 * ---------------------------------------------------------------------- */
sbp_status sbp_attn_bwd_workspace_size(int64_t B, int64_t T, int32_t Hq, int32_t Hkv,
                                       int32_t dh, int32_t D, int32_t dtype, size_t* bytes);

sbp_status sbp_attn_bwd_chunked(const void* Q, const void* K, const void* V, const void* dO,
                                const void* O, const float* lse, int64_t B, int64_t T,
                                int32_t Hq, int32_t Hkv, int32_t dh, float scale, int32_t D,
                                int32_t dtype, int32_t accumulate, void* dQ, float* dK,
                                float* dV, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * 2a. The attention backward of (2) without a workspace argument.
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight training or serving loops, harnesses that forbid hipMalloc.
 * Same arguments, computation and results as sbp_attn_bwd_chunked, minus
 * `ws` and `ws_bytes`: the call allocates nothing, and its scratch (the
 * per-chunk LSE and Delta rows, 8 * B * Hq * (chunk length rounded up to 64,
 * plus 64) bytes) lives in a static device array of 16 MiB that each GPU the
 * library runs on holds until the process ends.  A call whose scratch would
 * exceed 16 MiB returns SBP_ERR_UNSUPPORTED before any launch (raise D, or
 * use sbp_attn_bwd_chunked).  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (several streams or host threads) race, and
 * must be ordered by the caller.  The first call on a device looks up that
 * device's copy of the array (it must be the current device).
 * ---------------------------------------------------------------------- */
sbp_status sbp_attn_bwd_chunked_noalloc(const void* Q, const void* K, const void* V,
                                        const void* dO, const void* O, const float* lse,
                                        int64_t B, int64_t T, int32_t Hq, int32_t Hkv,
                                        int32_t dh, float scale, int32_t D, int32_t dtype,
                                        int32_t accumulate, void* dQ, float* dK, float* dV,
                                        void* stream);

/* ------------------------------------------------------------------------
 * 2b. Causal GQA attention backward over packed independent sequences.
 *
 * Passage: skill page, "Practical Guidance" -- attention masks must hold
 * across chunk boundaries; with several sequences packed end to end in one
 * row (the packed-batch layout of long-sequence training) the reading is
 * that a query sees only keys of its own sequence at or before it.  Same
 * computation, chunking and outputs as (2) with B = 1, and the mask
 *
 *   key j visible to query i  iff  cu[n] <= j <= i  for the n with
 *                                  cu[n] <= i < cu[n+1]
 *
 * Key blocks that no query of a chunk sees are skipped, so the work falls
 * with the sequence lengths (block-diagonal, not full causal).
 *
 * cu_seqlens [nseq+1] int32 (device)  sequence boundaries,
 *                               0 = cu[0] <= cu[1] <= ... <= cu[nseq] = T;
 *                               empty sequences are allowed.  Other
 *                               contents are a caller error, not checked:
 *                               results are then unspecified, but every
 *                               access stays in bounds.
 * nseq     number of sequences, >= 1
 * Q, K, V, dO, O, lse, dQ, dK, dV   as in (2) with B = 1
 * ---------------------------------------------------------------------- */
sbp_status sbp_attn_bwd_packed_workspace_size(int64_t T, int32_t Hq, int32_t Hkv, int32_t dh,
                                              int32_t D, int32_t dtype, size_t* bytes);

sbp_status sbp_attn_bwd_packed(const void* Q, const void* K, const void* V, const void* dO,
                               const void* O, const float* lse, const int32_t* cu_seqlens,
                               int32_t nseq, int64_t T, int32_t Hq, int32_t Hkv, int32_t dh,
                               float scale, int32_t D, int32_t dtype, int32_t accumulate,
                               void* dQ, float* dK, float* dV, void* ws, size_t ws_bytes,
                               void* stream);

/* ------------------------------------------------------------------------
 * 3. One pre-norm decoder layer, streamed backward.
 *
 * Passage: skill page, "Implementation" -- the streaming layer backward
 * (per chunk: run the layer forward on the chunk, back-propagate the chunk's
 * upstream gradient, add the weight gradients, keep the chunk's input
 * gradient) and "Architecture Overview" (layer-wise application).  Layer:
 *
 *   h1 = RMSNorm(x; g1); q,k,v = h1 Wq^T, h1 Wk^T, h1 Wv^T
 *   q, k = HeadNorm(q; qn), HeadNorm(k; kn)   (only when desc->qk_norm)
 *   q, k = Rope(q), Rope(k)        (only when desc->rope_theta > 0)
 *   o = causal GQA attention (scale 1/sqrt(dh)); a = x + o Wo^T
 *   n2 = RMSNorm(a; g2); m = silu(n2 W1^T) * (n2 W3^T); y = a + m W2^T
 *   RMSNorm(x; g) = g x / sqrt(mean(x^2) + eps)
 *   Rope: rotary position embedding (RoFormer, Su et al.; the pages name no
 *   position encoding): each head vector's halves (x1, x2) of width dh/2 turn
 *   pair by pair, pair i by p * rope_theta^(-2i/dh) with p the token's
 *   position (0 at the start of the row, or of its sequence when packed):
 *   (x1 cos - x2 sin, x2 cos + x1 sin).  The workspace then also holds a
 *   (cos, sin) table of T * dh/2 float pairs.
 *   HeadNorm (QK-norm, as in Qwen 3; not on the pages): the RMSNorm above
 *   over every head vector of width dh, one gain [dh] shared by all q heads
 *   (qn) and one by all k heads (kn), eps = desc->eps.
 *
 * Keys and values of all T tokens are formed once (the causal prefix); then
 * chunks run in reverse order, each recomputing its own forward, so the MLP
 * activations exist for one chunk at a time.
 *
 * x, dy   [T, d] dtype;  dx [T, d] dtype out
 * weights (host struct of device pointers, dtype): g1, g2 [d];
 *   Wq [Hq*dh, d]; Wk, Wv [Hkv*dh, d]; Wo [d, Hq*dh]; W1, W3 [F, d]; W2 [d, F]
 * grads   (host struct of device pointers, fp32, same shapes; accumulate
 *          semantics)
 * Supported: desc->dtype SBP_BF16 or SBP_F32 (fp32: x, dy, dx, weights and
 * every intermediate fp32); dh in {64, 128}; Hq % Hkv == 0; d % 8 == 0;
 * F % 8 == 0.
 * ---------------------------------------------------------------------- */
typedef struct {
  int64_t T, d;
  int32_t Hq, Hkv, dh;
  int64_t F;
  float eps;
  int32_t dtype;
  float rope_theta;  /* rotary embedding base; 0 = no rotary embedding; must be >= 0 */
  int32_t qk_norm;   /* 1: per-head RMSNorm of q and k with gains qn, kn; 0: none */
} sbp_layer_desc;

typedef struct {
  const void *g1, *Wq, *Wk, *Wv, *Wo, *g2, *W1, *W3, *W2;
  const void *qn, *kn;  /* [dh] each; read only when desc->qk_norm */
} sbp_layer_weights;

typedef struct {
  float *g1, *Wq, *Wk, *Wv, *Wo, *g2, *W1, *W3, *W2;
  float *qn, *kn;       /* [dh] each; written only when desc->qk_norm */
} sbp_layer_grads;

sbp_status sbp_layer_bwd_workspace_size(const sbp_layer_desc* desc, int32_t D, size_t* bytes);

sbp_status sbp_layer_bwd(const sbp_layer_desc* desc, const void* x, const void* dy,
                         const sbp_layer_weights* weights, int32_t D, int32_t accumulate,
                         void* dx, sbp_layer_grads* grads, void* ws, size_t ws_bytes,
                         void* stream);

/* ------------------------------------------------------------------------
 * 3b. Decoder-layer backward over packed independent sequences.
 *
 * As (3) with the tokens [0, T) being several sequences laid end to end,
 * sequence n holding tokens [cu[n], cu[n+1]): attention stays inside each
 * sequence (the mask of 2b); RMSNorm, the projections and the MLP are
 * token-wise and unchanged.  cu_seqlens / nseq as in 2b.
 * ---------------------------------------------------------------------- */
sbp_status sbp_layer_bwd_packed_workspace_size(const sbp_layer_desc* desc, int32_t D,
                                               size_t* bytes);

sbp_status sbp_layer_bwd_packed(const sbp_layer_desc* desc, const int32_t* cu_seqlens,
                                int32_t nseq, const void* x, const void* dy,
                                const sbp_layer_weights* weights, int32_t D, int32_t accumulate,
                                void* dx, sbp_layer_grads* grads, void* ws, size_t ws_bytes,
                                void* stream);

/* ------------------------------------------------------------------------
 * 3c. One pre-norm decoder layer, chunked forward: y = Layer(x).
 *
 * Passage: skill page, "Architecture Overview" (layer-wise application) and
 * "Implementation" (the streaming layer backward starts from each layer's
 * input, kept from a forward pass): this call is that forward, so that a
 * caller can run a stack of layers and keep the input of every layer for
 * sbp_layer_bwd.  The layer is the one of (3), rotary embedding included.
 *
 * Chunks run in order; chunk c forms its own keys and values, then its
 * queries attend over keys [0, e_c) (inside their own sequence when
 * cu_seqlens is given).  Keys and values of all T tokens stay in the
 * workspace; every other activation exists for one chunk at a time.
 *
 * cu_seqlens  device int32 [nseq + 1] packed-sequence boundaries as in 2b, or
 *             NULL for one causal row of T tokens (nseq then ignored)
 * x           [T, d] dtype (device);  y [T, d] dtype out, must not alias x
 * weights     as in (3)
 * Errors: as in (3); y == x -> SBP_ERR_INVALID_ARG.
 * ---------------------------------------------------------------------- */
sbp_status sbp_layer_fwd_workspace_size(const sbp_layer_desc* desc, int32_t D, size_t* bytes);

sbp_status sbp_layer_fwd(const sbp_layer_desc* desc, const int32_t* cu_seqlens, int32_t nseq,
                         const void* x, const sbp_layer_weights* weights, int32_t D, void* y,
                         void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * 4. Whole decoder-only model, streamed backward layer by layer.
 *
 * Passage: skill page, "Architecture Overview" -- the "Layer-Wise
 * Application" item (the chunked backward applied through the model one
 * layer at a time) -- and "Implementation" (the LM-head logits gradient; the
 * streaming layer backward that starts from each layer's stored input).
 *
 *   x_{l+1} = Layer_l(x_l), l = 0 .. L-1     (the layer of (3), desc shared)
 *   h = RMSNorm(x_L; g_final)                (eps = desc->eps)
 *   loss = CE(h W_lm^T; targets, weights)    (as in (1), reduction likewise)
 *
 * The caller keeps x_0 .. x_L from a forward pass (sbp_layer_fwd per layer)
 * and the embedding lookup: dx0 is the gradient of x_0, its rows are what a
 * scatter-add into the embedding table takes.  The call runs the final norm,
 * the LM head over D_lm chunks (never the [T, V] logits), the final norm's
 * backward, then every layer's streamed backward over D_layer chunks, last
 * layer first.  Transient memory: the larger of the LM-head and layer
 * workspaces plus three [T, d] buffers of the dtype.
 *
 * desc        layer shape, rope_theta included; desc->dtype SBP_BF16 or
 *             SBP_F32 (fp32: the activations, weights, g_final, W_lm and dx0
 *             fp32, every product in fp32, as in the fp32 modes of (1), (3))
 * n_layers    L >= 0 (0: final norm under the LM head)
 * cu_seqlens  packed-sequence boundaries as in 2b, or NULL (one causal row)
 * x_layers    host array of L + 1 device pointers [T, d] dtype: the input
 *             of every layer, then the last layer's output
 * layers      host array of L weight structs (as in 3); grads host array of
 *             L grad structs (fp32, accumulate semantics)
 * g_final     [d] dtype; dg_final [d] fp32 out (accumulate semantics)
 * W_lm        [V, d] dtype; dW_lm [V, d] fp32 out (accumulate semantics)
 * targets, weights, reduction, loss, token_loss   as in (1)
 * dx0         [T, d] dtype out; must not alias any x_layers entry
 * Errors: as in (1) and (3); argument errors are returned before any launch.
 * ---------------------------------------------------------------------- */
sbp_status sbp_model_bwd_workspace_size(const sbp_layer_desc* desc, int32_t n_layers,
                                        int32_t packed, int64_t V, int32_t D_lm,
                                        int32_t D_layer, size_t* bytes);

sbp_status sbp_model_bwd(const sbp_layer_desc* desc, int32_t n_layers,
                         const int32_t* cu_seqlens, int32_t nseq, const void* const* x_layers,
                         const sbp_layer_weights* layers, const void* g_final, const void* W_lm,
                         int64_t V, const int32_t* targets, const float* weights,
                         int32_t reduction, int32_t D_lm, int32_t D_layer, int32_t accumulate,
                         float* loss, float* token_loss, void* dx0, sbp_layer_grads* grads,
                         float* dg_final, float* dW_lm, void* ws, size_t ws_bytes,
                         void* stream);

/* ------------------------------------------------------------------------
 * Debug mode.  With the environment variable SBP_DEBUG set (to anything but
 * "0"), every call checks on the device, before any of its own kernels run,
 * the inputs it otherwise trusts -- target ids >= V (calls 1, 1b, 4) and
 * cu_seqlens that do not rise from 0 to T without decreasing (2b, 3b, 3c, 4)
 * -> SBP_ERR_INVALID_ARG -- and synchronises its stream after its last
 * launch, so that a failing kernel is reported (SBP_ERR_HIP) by the call that
 * launched it.  Debug mode blocks the host and is not for graph capture.
 * ---------------------------------------------------------------------- */

/* ------------------------------------------------------------------------
 * Diagnostics.
 * ---------------------------------------------------------------------- */
const char* sbp_status_string(int32_t status);
/* Message of the last failed call on this host thread ("" if none). */
const char* sbp_last_error(void);
int32_t sbp_version(void);

/* Kernel timer, for benchmarking.  While enabled, every kernel the library
 * enqueues is bracketed by hipEvents on its stream (events come from a pool
 * created by sbp_profile_begin; no device memory is allocated).
 * sbp_profile_end waits for those events and folds them into per-kernel
 * totals; sbp_profile_entry then reads entry i (0 <= i < count) as kernel
 * name, launch count, total milliseconds and the algorithmic flop and byte
 * counts of those launches.  Profiling is process-wide and not thread-safe. */
sbp_status sbp_profile_begin(int32_t max_launches);
sbp_status sbp_profile_end(int32_t* count);
sbp_status sbp_profile_entry(int32_t i, const char** name, int64_t* launches,
                             double* total_ms, double* flops, double* bytes);
#ifdef __cplusplus
}
#endif

#endif /* STREAMBP_H */
