// sbp_attn_bwd_chunked: causal GQA attention backward, chunked over queries.
#include "common.h"
#include "kernels.h"

namespace sbp {
namespace {

inline bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

sbp_status attn_check(int64_t B, int64_t T, int32_t Hq, int32_t Hkv, int32_t dh, int32_t D,
                      int32_t dtype) {
  if (dtype != SBP_F32 && dtype != SBP_BF16) return set_error(SBP_ERR_INVALID_ARG, "dtype %d is not SBP_F32 or SBP_BF16", dtype);
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || dh < 1) return set_error(SBP_ERR_INVALID_ARG, "B, T, Hq, Hkv, dh must be >= 1");
  if (D < 1 || D > T) return set_error(SBP_ERR_INVALID_ARG, "need 1 <= D <= T (D=%d, T=%lld)", D, (long long)T);
  if (Hq % Hkv) return set_error(SBP_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (dh != 64 && dh != 128) return set_error(SBP_ERR_UNSUPPORTED, "head dim %d not supported (64 or 128)", dh);
  if (B * T > (1ll << 30)) return set_error(SBP_ERR_UNSUPPORTED, "B*T out of supported range");
  return SBP_OK;
}

size_t attn_ws(int64_t B, int64_t T, int32_t Hq, int32_t dh, int32_t D, int32_t dtype) {
  // per query chunk: O_c (dtype), LSE_c and Delta_c (fp32)
  const int64_t Tcm = max_chunk_len(T, D);
  const size_t esz = dtype == SBP_BF16 ? 2 : 4;
  WsPlan P;
  P.take(esz * B * Tcm * Hq * dh);
  P.take(sizeof(float) * B * Tcm * Hq);
  P.take(sizeof(float) * B * Tcm * Hq);
  return round_up((int64_t)P.off, 256);
}

}  // namespace
}  // namespace sbp

using namespace sbp;

extern "C" sbp_status sbp_attn_bwd_workspace_size(int64_t B, int64_t T, int32_t Hq, int32_t Hkv,
                                                  int32_t dh, int32_t D, int32_t dtype,
                                                  size_t* bytes) {
  clear_error();
  if (!bytes) return set_error(SBP_ERR_INVALID_ARG, "bytes is NULL");
  sbp_status st = attn_check(B, T, Hq, Hkv, dh, D, dtype);
  if (st != SBP_OK) return st;
  *bytes = attn_ws(B, T, Hq, dh, D, dtype);
  return SBP_OK;
}

extern "C" sbp_status sbp_attn_bwd_chunked(const void* Q, const void* K, const void* V,
                                           const void* dO, const void* O, const float* lse,
                                           int64_t B, int64_t T, int32_t Hq, int32_t Hkv,
                                           int32_t dh, float scale, int32_t D, int32_t dtype,
                                           int32_t accumulate, void* dQ, float* dK, float* dV,
                                           void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  sbp_status st = attn_check(B, T, Hq, Hkv, dh, D, dtype);
  if (st != SBP_OK) return st;
  if (!Q || !K || !V || !dO || !dQ || !dK || !dV)
    return set_error(SBP_ERR_INVALID_ARG, "Q, K, V, dO, dQ, dK and dV must be non-NULL");
  if ((O == nullptr) != (lse == nullptr))
    return set_error(SBP_ERR_INVALID_ARG, "O and lse must be given together or not at all");
  if (misaligned(Q) || misaligned(K) || misaligned(V) || misaligned(dO) || misaligned(O) ||
      misaligned(lse) || misaligned(dQ) || misaligned(dK) || misaligned(dV) || misaligned(ws))
    return set_error(SBP_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  if (!(scale > 0.f) || !(scale < 1e30f)) return set_error(SBP_ERR_INVALID_ARG, "scale must be positive and finite");
  const size_t need = attn_ws(B, T, Hq, dh, D, dtype);
  if (!ws || ws_bytes < need)
    return set_error(SBP_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
  (void)accumulate;
  (void)stream;
  return set_error(SBP_ERR_UNSUPPORTED, "attention backward kernels are not built in this version");
}
