// Debug mode (environment variable SBP_DEBUG set to anything but "0"): every
// entry point checks, on the device and before any of its own kernels run,
// the inputs whose bad values it otherwise does not look at (target ids of
// the LM head at or past V, packed-sequence boundaries that are not
// non-decreasing from 0 to T), and synchronises its stream after its last
// launch so that a failing kernel is reported by the call that launched it.
// The checks count into one static device word; debug mode is therefore
// not for graph capture, and calls from several host threads at once may
// mix their counts.
#include <stdlib.h>
#include <string.h>

#include "common.h"
#include "kernels.h"

namespace sbp {

__device__ int g_debug_count;

bool debug_on() {
  const char* v = getenv("SBP_DEBUG");
  return v && *v && strcmp(v, "0") != 0;
}

__global__ __launch_bounds__(256) void count_bad_targets_kernel(const int32_t* __restrict__ t, int64_t T,
                                                                int64_t V, int* __restrict__ cnt) {
  int bad = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < T; i += (int64_t)gridDim.x * 256)
    bad += t[i] >= V;
  bad = (int)wave_sum((float)bad);
  if ((threadIdx.x & 63) == 0 && bad) atomicAdd(cnt, bad);
}

__global__ __launch_bounds__(256) void count_bad_cu_kernel(const int32_t* __restrict__ cu, int nseq,
                                                           int64_t T, int* __restrict__ cnt) {
  int bad = 0;
  for (int i = blockIdx.x * 256 + threadIdx.x; i <= nseq; i += gridDim.x * 256) {
    if (i == 0) bad += cu[0] != 0;
    if (i == nseq) bad += (int64_t)cu[nseq] != T;
    if (i < nseq) bad += cu[i] > cu[i + 1];
  }
  bad = (int)wave_sum((float)bad);
  if ((threadIdx.x & 63) == 0 && bad) atomicAdd(cnt, bad);
}

namespace {

// zero the counter, run `launch`, read the counter back (stream-ordered)
template <typename F>
sbp_status debug_count(hipStream_t st, F launch, int* out) {
  int* cnt = nullptr;
  SBP_HIP_CHECK(hipGetSymbolAddress(reinterpret_cast<void**>(&cnt), HIP_SYMBOL(g_debug_count)));
  SBP_HIP_CHECK(hipMemsetAsync(cnt, 0, sizeof(int), st));
  launch(cnt);
  SBP_LAUNCH_CHECK();
  SBP_HIP_CHECK(hipMemcpyAsync(out, cnt, sizeof(int), hipMemcpyDeviceToHost, st));
  SBP_HIP_CHECK(hipStreamSynchronize(st));
  return SBP_OK;
}

}  // namespace

sbp_status debug_check_targets(const int32_t* targets, int64_t T, int64_t V, hipStream_t st) {
  if (!debug_on() || !targets || T < 1) return SBP_OK;
  int bad = 0;
  const unsigned grid = (unsigned)std::min<int64_t>(cdiv(T, 256), 1024);
  sbp_status s = debug_count(st, [&](int* c) {
    hipLaunchKernelGGL(count_bad_targets_kernel, dim3(grid), dim3(256), 0, st, targets, T, V, c);
  }, &bad);
  if (s != SBP_OK) return s;
  if (bad) return set_error(SBP_ERR_INVALID_ARG, "SBP_DEBUG: %d target ids are >= V = %lld", bad, (long long)V);
  return SBP_OK;
}

sbp_status debug_check_cu(const int32_t* cu, int nseq, int64_t T, hipStream_t st) {
  if (!debug_on() || !cu || nseq < 1) return SBP_OK;
  int bad = 0;
  const unsigned grid = (unsigned)cdiv((int64_t)nseq + 1, 256);
  sbp_status s = debug_count(st, [&](int* c) {
    hipLaunchKernelGGL(count_bad_cu_kernel, dim3(grid), dim3(256), 0, st, cu, nseq, T, c);
  }, &bad);
  if (s != SBP_OK) return s;
  if (bad)
    return set_error(SBP_ERR_INVALID_ARG, "SBP_DEBUG: cu_seqlens must rise from 0 to T = %lld without decreasing (%d violations)",
                     (long long)T, bad);
  return SBP_OK;
}

sbp_status debug_sync(hipStream_t st, const char* call) {
  if (!debug_on()) return SBP_OK;
  const hipError_t e = hipStreamSynchronize(st);
  const hipError_t l = hipGetLastError();
  if (e != hipSuccess || l != hipSuccess)
    return set_error(SBP_ERR_HIP, "SBP_DEBUG: %s: %s", call, hipGetErrorString(e != hipSuccess ? e : l));
  return SBP_OK;
}

}  // namespace sbp
