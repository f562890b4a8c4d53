// sbp_layer_bwd: streamed backward of one pre-norm decoder layer.
#include "common.h"
#include "kernels.h"

namespace sbp {
namespace {

inline bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

sbp_status layer_check(const sbp_layer_desc* L, int32_t D) {
  if (!L) return set_error(SBP_ERR_INVALID_ARG, "desc is NULL");
  if (L->dtype != SBP_F32 && L->dtype != SBP_BF16) return set_error(SBP_ERR_INVALID_ARG, "dtype %d is not SBP_F32 or SBP_BF16", L->dtype);
  if (L->T < 1 || L->d < 1 || L->Hq < 1 || L->Hkv < 1 || L->dh < 1 || L->F < 1)
    return set_error(SBP_ERR_INVALID_ARG, "T, d, Hq, Hkv, dh, F must be >= 1");
  if (D < 1 || D > L->T) return set_error(SBP_ERR_INVALID_ARG, "need 1 <= D <= T (D=%d, T=%lld)", D, (long long)L->T);
  if (L->Hq % L->Hkv) return set_error(SBP_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", L->Hq, L->Hkv);
  if (!(L->eps >= 0.f)) return set_error(SBP_ERR_INVALID_ARG, "eps must be >= 0");
  if (L->dh != 64 && L->dh != 128) return set_error(SBP_ERR_UNSUPPORTED, "head dim %d not supported (64 or 128)", L->dh);
  if (L->d % 8 || L->F % 8) return set_error(SBP_ERR_UNSUPPORTED, "d and F must be multiples of 8");
  return SBP_OK;
}

size_t layer_ws(const sbp_layer_desc* L, int32_t D) {
  const int64_t T = L->T, d = L->d, F = L->F;
  const int64_t qd = (int64_t)L->Hq * L->dh, kd = (int64_t)L->Hkv * L->dh;
  const int64_t Tcm = max_chunk_len(T, D);
  const size_t esz = L->dtype == SBP_BF16 ? 2 : 4;
  WsPlan P;
  P.take(esz * T * kd * 2);                 // K, V of every token
  P.take(sizeof(float) * T * kd * 2);       // dK, dV accumulators
  P.take(esz * Tcm * (3 * d + 2 * qd + 3 * F));  // chunk activations
  P.take(sizeof(float) * Tcm * (2 * d + F));     // chunk fp32 temporaries
  return round_up((int64_t)P.off, 256);
}

}  // namespace
}  // namespace sbp

using namespace sbp;

extern "C" sbp_status sbp_layer_bwd_workspace_size(const sbp_layer_desc* desc, int32_t D,
                                                   size_t* bytes) {
  clear_error();
  if (!bytes) return set_error(SBP_ERR_INVALID_ARG, "bytes is NULL");
  sbp_status st = layer_check(desc, D);
  if (st != SBP_OK) return st;
  *bytes = layer_ws(desc, D);
  return SBP_OK;
}

extern "C" sbp_status sbp_layer_bwd(const sbp_layer_desc* desc, const void* x, const void* dy,
                                    const sbp_layer_weights* w, int32_t D, int32_t accumulate,
                                    void* dx, sbp_layer_grads* g, void* ws, size_t ws_bytes,
                                    void* stream) {
  clear_error();
  sbp_status st = layer_check(desc, D);
  if (st != SBP_OK) return st;
  if (!x || !dy || !w || !dx || !g) return set_error(SBP_ERR_INVALID_ARG, "x, dy, weights, dx, grads must be non-NULL");
  const void* wp[9] = {w->g1, w->Wq, w->Wk, w->Wv, w->Wo, w->g2, w->W1, w->W3, w->W2};
  float* gp[9] = {g->g1, g->Wq, g->Wk, g->Wv, g->Wo, g->g2, g->W1, g->W3, g->W2};
  for (int i = 0; i < 9; ++i) {
    if (!wp[i] || !gp[i]) return set_error(SBP_ERR_INVALID_ARG, "weight/grad pointer %d is NULL", i);
    if (misaligned(wp[i]) || misaligned(gp[i])) return set_error(SBP_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  }
  if (misaligned(x) || misaligned(dy) || misaligned(dx) || misaligned(ws))
    return set_error(SBP_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  const size_t need = layer_ws(desc, D);
  if (!ws || ws_bytes < need)
    return set_error(SBP_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
  (void)accumulate;
  (void)stream;
  return set_error(SBP_ERR_UNSUPPORTED, "decoder-layer backward is not built in this version");
}
