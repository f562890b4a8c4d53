// sbp_model_bwd: streamed backward of a whole decoder-only model, layer by
// layer.
//
// StreamBP skill page, "Architecture Overview" (the "Layer-Wise Application"
// item: the sequence-chunked backward is applied through the model one
// layer at a time) and "Implementation" (the LM-head logits gradient; the
// streaming layer backward starting from each layer's stored input).  Model:
//   x_{l+1} = Layer_l(x_l) for l < L;  h = RMSNorm(x_L; g_f);
//   loss = CE(h W^T; targets, weights)
// Given the layer inputs x_0 .. x_{L-1} and the last output x_L (a forward
// pass with sbp_layer_fwd keeps them), the call runs:
//   h = RMSNorm(x_L; g_f)                              one [T, d] buffer
//   LM head + CE over D_lm chunks -> loss, dh, dW      (sbp_lmhead_ce_fwd_bwd)
//   dx_L = RMSNorm'(dh), dg_f +=                       D_layer chunks
//   dx_l = Layer_l'(x_l, dx_{l+1}), l = L-1 .. 0       (sbp_layer_bwd)
// Activations and upstream gradients are of the call's dtype (bf16, or fp32
// throughout); the upstream gradients alternate between two [T, d] buffers.
// The LM-head and layer calls run one after another on the caller's stream
// and share one workspace region, so the call's transient memory is the
// larger of theirs plus three [T, d] buffers.
#include "common.h"
#include "kernels.h"

namespace sbp {
namespace {

inline bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }
inline size_t dtype_size(int dtype) { return dtype == SBP_F32 ? sizeof(float) : sizeof(bf16_t); }

struct ModelWs {
  char *h, *gA, *gB;  // [T, d] of the call's dtype
  float *rinv, *dn, *gpart;
  char* sub;
};

// es: bytes per element of the dtype.  dn (the final norm's upstream
// gradient of a chunk in fp32) is needed only when dh is bf16.
size_t model_plan(int64_t T, int64_t d, int64_t Tcm, size_t es, size_t sub_bytes, char* base, ModelWs* w) {
  WsPlan P;
  P.base = base;
  ModelWs x;
  x.h = (char*)P.take(es * T * d);
  x.gA = (char*)P.take(es * T * d);
  x.gB = (char*)P.take(es * T * d);
  x.rinv = (float*)P.take(sizeof(float) * T);
  x.dn = es == sizeof(float) ? nullptr : (float*)P.take(sizeof(float) * Tcm * d);
  x.gpart = (float*)P.take(sizeof(float) * gain_grad_splits(Tcm) * d);
  x.sub = (char*)P.take(sub_bytes);
  if (w) *w = x;
  return round_up((int64_t)P.off, 256);
}

// Workspace of the inner calls (LM head, one layer): the larger of the two.
sbp_status model_sub_bytes(const sbp_layer_desc* desc, bool packed, int64_t V, int32_t D_lm,
                           int32_t D_layer, size_t* out) {
  size_t lm = 0, lay = 0;
  sbp_status st = sbp_lmhead_ce_workspace_size(desc->T, desc->d, V, D_lm, desc->dtype, &lm);
  if (st != SBP_OK) return st;
  st = packed ? sbp_layer_bwd_packed_workspace_size(desc, D_layer, &lay)
              : sbp_layer_bwd_workspace_size(desc, D_layer, &lay);
  if (st != SBP_OK) return st;
  *out = lm > lay ? lm : lay;
  return SBP_OK;
}

sbp_status model_check(const sbp_layer_desc* desc, int32_t n_layers, int64_t V, int32_t D_lm,
                       int32_t D_layer) {
  if (!desc) return set_error(SBP_ERR_INVALID_ARG, "desc is NULL");
  if (n_layers < 0 || n_layers > 4096) return set_error(SBP_ERR_INVALID_ARG, "n_layers must be in [0, 4096] (got %d)", n_layers);
  if (V < 1) return set_error(SBP_ERR_INVALID_ARG, "V must be >= 1");
  if (desc->dtype != SBP_BF16 && desc->dtype != SBP_F32)
    return set_error(SBP_ERR_INVALID_ARG, "dtype must be SBP_BF16 or SBP_F32 (got %d)", desc->dtype);
  if (D_lm < 1 || D_lm > desc->T || D_layer < 1 || D_layer > desc->T)
    return set_error(SBP_ERR_INVALID_ARG, "need 1 <= D_lm, D_layer <= T");
  return SBP_OK;
}

}  // namespace
}  // namespace sbp

using namespace sbp;

extern "C" sbp_status sbp_model_bwd_workspace_size(const sbp_layer_desc* desc, int32_t n_layers,
                                                   int32_t packed, int64_t V, int32_t D_lm,
                                                   int32_t D_layer, size_t* bytes) {
  clear_error();
  if (!bytes) return set_error(SBP_ERR_INVALID_ARG, "bytes is NULL");
  sbp_status st = model_check(desc, n_layers, V, D_lm, D_layer);
  if (st != SBP_OK) return st;
  size_t sub = 0;
  st = model_sub_bytes(desc, packed != 0, V, D_lm, D_layer, &sub);
  if (st != SBP_OK) return st;
  *bytes = model_plan(desc->T, desc->d, max_chunk_len(desc->T, D_layer), dtype_size(desc->dtype), sub,
                      nullptr, nullptr);
  return SBP_OK;
}

extern "C" sbp_status sbp_model_bwd(const sbp_layer_desc* desc, int32_t n_layers,
                                    const int32_t* cu_seqlens, int32_t nseq,
                                    const void* const* x_layers,
                                    const sbp_layer_weights* layers, const void* g_final,
                                    const void* W_lm, int64_t V, const int32_t* targets,
                                    const float* weights, int32_t reduction, int32_t D_lm,
                                    int32_t D_layer, int32_t accumulate, float* loss,
                                    float* token_loss, void* dx0, sbp_layer_grads* grads,
                                    float* dg_final, float* dW_lm, void* ws, size_t ws_bytes,
                                    void* stream) {
  clear_error();
  hipStream_t str = (hipStream_t)stream;
  sbp_status st = model_check(desc, n_layers, V, D_lm, D_layer);
  if (st != SBP_OK) return st;
  if (!x_layers || (n_layers > 0 && (!layers || !grads)) || !g_final || !W_lm || !targets ||
      !loss || !dx0 || !dg_final || !dW_lm)
    return set_error(SBP_ERR_INVALID_ARG, "a required pointer is NULL");
  for (int32_t l = 0; l <= n_layers; ++l)
    if (!x_layers[l] || misaligned(x_layers[l]))
      return set_error(SBP_ERR_INVALID_ARG, "x_layers[%d] is NULL or not 16-byte aligned", l);
  if (misaligned(g_final) || misaligned(dx0) || misaligned(dg_final) || misaligned(ws))
    return set_error(SBP_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  for (int32_t l = 0; l <= n_layers; ++l)
    if (x_layers[l] == dx0) return set_error(SBP_ERR_INVALID_ARG, "dx0 must not alias x_layers[%d]", l);
  if (cu_seqlens && nseq < 1) return set_error(SBP_ERR_INVALID_ARG, "nseq must be >= 1 (got %d)", nseq);
  if (desc->d % 8) return set_error(SBP_ERR_UNSUPPORTED, "d must be a multiple of 8");
  const bool packed = cu_seqlens != nullptr;
  size_t sub = 0;
  st = model_sub_bytes(desc, packed, V, D_lm, D_layer, &sub);
  if (st != SBP_OK) return st;
  const int64_t T = desc->T, d = desc->d;
  const int dt = desc->dtype;
  const size_t es = dtype_size(dt);
  const int64_t Tcm = max_chunk_len(T, D_layer);
  const size_t need = model_plan(T, d, Tcm, es, sub, nullptr, nullptr);
  if (!ws || ws_bytes < need)
    return set_error(SBP_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
  ModelWs W;
  model_plan(T, d, Tcm, es, sub, (char*)ws, &W);
  auto row = [&](const void* p, int64_t r) { return (const char*)p + (int64_t)es * r * d; };
#define SBP_TRY(e_)                  \
  do {                               \
    sbp_status _s = (e_);            \
    if (_s != SBP_OK) return _s;     \
  } while (0)

  // final norm and the LM head; dh lands in gA
  const void* xL = x_layers[n_layers];
  SBP_TRY(rmsnorm_fwd(xL, d, g_final, T, d, desc->eps, W.h, d, W.rinv, str, dt));
  SBP_TRY(sbp_lmhead_ce_fwd_bwd(W.h, W_lm, targets, weights, T, d, V, D_lm, dt, reduction,
                                accumulate, loss, token_loss, W.gA, dW_lm, W.sub, sub, stream));
  // dx_L = RMSNorm'(dh) into gB (into dx0 if there are no layers), dg_f +=;
  // the norm's backward takes dh in fp32: converted per chunk from bf16, or
  // read in place in fp32 mode
  char* up = n_layers > 0 ? W.gB : (char*)dx0;
  for (int32_t c = 0; c < D_layer; ++c) {
    int64_t s0, e0;
    chunk_bounds(T, D_layer, c, &s0, &e0);
    const int64_t Tc = e0 - s0;
    const float* dn = (const float*)row(W.gA, s0);
    if (dt == SBP_BF16) {
      SBP_TRY(rows_to_f32(row(W.gA, s0), d, Tc, d, W.dn, d, str));
      dn = W.dn;
    }
    SBP_TRY(rmsnorm_bwd(row(xL, s0), d, g_final, dn, d, W.rinv + s0, nullptr, 0, Tc, d,
                        (void*)row(up, s0), d, str, dt));
    SBP_TRY(gain_grad(dn, d, row(xL, s0), d, W.rinv + s0, Tc, d, dg_final,
                      c == 0 ? (accumulate ? 1 : 0) : 1, W.gpart, str, dt));
  }
  // layers, last to first
  char* other = W.gA;
  for (int32_t l = n_layers - 1; l >= 0; --l) {
    char* out = l == 0 ? (char*)dx0 : other;
    if (packed)
      SBP_TRY(sbp_layer_bwd_packed(desc, cu_seqlens, nseq, x_layers[l], up, &layers[l], D_layer,
                                   accumulate, out, &grads[l], W.sub, sub, stream));
    else
      SBP_TRY(sbp_layer_bwd(desc, x_layers[l], up, &layers[l], D_layer, accumulate, out,
                            &grads[l], W.sub, sub, stream));
    other = up;
    up = out;
  }
#undef SBP_TRY
  return debug_sync(str, "sbp_model_bwd");
}
