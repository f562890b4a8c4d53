// Shared device/host helpers for libstreambp (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <algorithm>

#include "streambp.h"

namespace sbp {

// ---------------------------------------------------------------------------
// Element types.  bf16 is kept as raw 16-bit storage; arithmetic is fp32.
// ---------------------------------------------------------------------------
typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// fp32 -> bf16 by the gfx950 conversion instruction (v_cvt_pk_bf16_f32:
// round-to-nearest-even under the default rounding mode, NaN stays NaN).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
__device__ __forceinline__ bf16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t* p, int64_t i) { return bf2f(p[i]); }
  __device__ __forceinline__ static void store(bf16_t* p, int64_t i, float v) { p[i] = f2bf(v); }
};

// ---------------------------------------------------------------------------
// Wave / block reductions (wave64).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ---------------------------------------------------------------------------
// Host side: errors and launch bookkeeping.
// ---------------------------------------------------------------------------
sbp_status set_error(sbp_status s, const char* fmt, ...);
void clear_error();

// Profiler hooks (no-ops unless sbp_profile_begin is active).
struct ProfScope {
  ProfScope(const char* name, hipStream_t st, double flops, double bytes);
  ~ProfScope();
  int slot;
  hipStream_t stream;
};

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// Chunk table: size = T / D, last chunk ends at T.
inline void chunk_bounds(int64_t T, int32_t D, int32_t c, int64_t* s, int64_t* e) {
  int64_t size = T / D;
  *s = c * size;
  *e = (c == D - 1) ? T : (c + 1) * size;
}
inline int64_t max_chunk_len(int64_t T, int32_t D) { return T - (int64_t)(D - 1) * (T / D); }

// Bump allocator over the caller's workspace (256-byte aligned slices).
struct WsPlan {
  size_t off = 0;
  char* base = nullptr;
  void* take(size_t bytes) {
    off = (size_t)round_up((int64_t)off, 256);
    void* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  }
};

}  // namespace sbp

#define SBP_HIP_CHECK(expr)                                                   \
  do {                                                                        \
    hipError_t _e = (expr);                                                   \
    if (_e != hipSuccess)                                                     \
      return ::sbp::set_error(SBP_ERR_HIP, "%s failed: %s (%s:%d)", #expr,    \
                              hipGetErrorString(_e), __FILE__, __LINE__);     \
  } while (0)

#define SBP_LAUNCH_CHECK()                                                    \
  do {                                                                        \
    hipError_t _e = hipGetLastError();                                        \
    if (_e != hipSuccess)                                                     \
      return ::sbp::set_error(SBP_ERR_HIP, "kernel launch failed: %s (%s:%d)",\
                              hipGetErrorString(_e), __FILE__, __LINE__);     \
  } while (0)
