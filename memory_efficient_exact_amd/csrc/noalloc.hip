// sbp_attn_bwd_chunked_noalloc: the chunked causal GQA attention backward
// of sbp_attn_bwd_chunked without a workspace argument, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// or training loops, harnesses that forbid hipMalloc).
//
// Its scratch -- per query chunk the LSE and Delta rows, fp32 [B, Hq, Lp] each
// -- lives in one file-scope device array of fixed size.  Each GPU the library
// runs on holds its own copy until the process ends; every call on that GPU
// uses it, so calls that overlap on one GPU (two streams, two host threads)
// race.  Nothing in it must start at zero: every chunk writes its statistics
// rows before its backward reads them, and rows past the chunk are padding
// that the kernels select away.  The entry point allocates nothing: no
// hipMalloc, no hipFree, no allocating library routine.
#include <mutex>

#include "attn.h"
#include "common.h"
#include "kernels.h"

namespace sbp {
namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;  // 16 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};  // device address of `scratch`, per device

// The device address of the current device's copy of `scratch`, looked up
// once per device with that device current.  The array's name in host code
// is only a host-side stand-in: kernels get this address, never the name.
sbp_status scratch_address(void** out) {
  int dev = -1;
  SBP_HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices)
    return set_error(SBP_ERR_UNSUPPORTED, "device index %d out of range (< %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(SBP_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                       hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return SBP_OK;
}

}  // namespace
}  // namespace sbp

using namespace sbp;

extern "C" sbp_status sbp_attn_bwd_chunked_noalloc(const void* Q, const void* K, const void* V,
                                                   const void* dO, const void* O, const float* lse,
                                                   int64_t B, int64_t T, int32_t Hq, int32_t Hkv,
                                                   int32_t dh, float scale, int32_t D,
                                                   int32_t dtype, int32_t accumulate, void* dQ,
                                                   float* dK, float* dV, void* stream) {
  clear_error();
  size_t need = 0;
  sbp_status st = attn_bwd_ws_size(B, T, Hq, Hkv, dh, D, dtype, &need);
  if (st != SBP_OK) return st;
  if (need > kScratchBytes)
    return set_error(SBP_ERR_UNSUPPORTED,
                     "needs %zu bytes of scratch (B * Hq * chunk length too large); the static "
                     "scratch holds %zu: use sbp_attn_bwd_chunked with a workspace, or a larger D",
                     need, kScratchBytes);
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != SBP_OK) return st;
  st = attn_bwd_run(Q, K, V, dO, O, lse, B, T, Hq, Hkv, dh, scale, D, dtype, accumulate, dQ, dK,
                    dV, ws, kScratchBytes, (hipStream_t)stream);
  return st == SBP_OK ? debug_sync((hipStream_t)stream, "sbp_attn_bwd_chunked_noalloc") : st;
}
