// Layout helpers: padded transpose, split-K reduction, zero fill.
#include "common.h"
#include "kernels.h"

namespace sbp {

// dst[c][r] = src[r][c] (r < R), 0 for R <= r < Rp.  64 x 64 tiles via LDS.
template <typename T>
__global__ __launch_bounds__(256) void transpose_pad_kernel(const T* __restrict__ src, int64_t lds_,
                                                            int64_t R, int64_t C, T* __restrict__ dst,
                                                            int64_t ldd, int64_t Rp,
                                                            const int* __restrict__ active) {
  if (active && *active == 0) return;
  __shared__ float tile[64][65];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * 64, r0 = (int64_t)blockIdx.y * 64;
#pragma unroll 4
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < R && c < C) ? Elem<T>::load(src, r * lds_ + c) : 0.f;
  }
  __syncthreads();
#pragma unroll 4
  for (int i = ty; i < 64; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < C && r < Rp) Elem<T>::store(dst, c * ldd + r, tile[tx][i]);
  }
}

// bf16 with 16-byte rows on both sides (C, pitches and bases multiples of 8
// elements, Rp a multiple of 8): each thread moves 8 elements per access.
// The 64 x 64 tile sits in LDS with a row pitch of 66 elements, so the 8
// strided reads of a column segment fall in distinct banks.
__global__ __launch_bounds__(256) void transpose_pad_bf16x8_kernel(
    const bf16_t* __restrict__ src, int64_t lds_, int64_t R, int64_t C, bf16_t* __restrict__ dst,
    int64_t ldd, int64_t Rp, const int* __restrict__ active) {
  if (active && *active == 0) return;
  __shared__ uint16_t tile[64][66];
  const int t = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * 64, r0 = (int64_t)blockIdx.y * 64;
  // load: 8 threads per row (8 columns each), 32 rows per pass
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int i = pass * 32 + (t >> 3), cc = (t & 7) * 8;
    const int64_t r = r0 + i, c = c0 + cc;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < R && c < C) v = *reinterpret_cast<const uint4*>(src + r * lds_ + c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      tile[i][cc + 2 * k] = (uint16_t)(w[k] & 0xffff);
      tile[i][cc + 2 * k + 1] = (uint16_t)(w[k] >> 16);
    }
  }
  __syncthreads();
  // store: 8 threads per output row (8 source rows each), 32 rows per pass
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int j = pass * 32 + (t >> 3), rr = (t & 7) * 8;
    const int64_t c = c0 + j, r = r0 + rr;
    if (c >= C || r >= Rp) continue;
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = (uint32_t)tile[rr + 2 * k][j] | ((uint32_t)tile[rr + 2 * k + 1][j] << 16);
    *reinterpret_cast<uint4*>(dst + c * ldd + r) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

sbp_status transpose_pad(int dtype, const void* src, int64_t lds_, int64_t R, int64_t C,
                         void* dst, int64_t ldd, int64_t Rp, const int* active, hipStream_t st) {
  const size_t esz = dtype == SBP_BF16 ? 2 : 4;
  ProfScope prof("transpose", st, 0.0, (double)esz * ((double)R * C + (double)Rp * C));
  dim3 grid((unsigned)cdiv(C, 64), (unsigned)cdiv(Rp, 64));
  const bool vec8 = dtype == SBP_BF16 && C % 8 == 0 && lds_ % 8 == 0 && ldd % 8 == 0 && Rp % 8 == 0 &&
                    (uintptr_t)src % 16 == 0 && (uintptr_t)dst % 16 == 0;
  if (vec8)
    hipLaunchKernelGGL(transpose_pad_bf16x8_kernel, grid, dim3(256), 0, st, (const bf16_t*)src, lds_, R, C,
                       (bf16_t*)dst, ldd, Rp, active);
  else if (dtype == SBP_BF16)
    hipLaunchKernelGGL(transpose_pad_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)src,
                       lds_, R, C, (bf16_t*)dst, ldd, Rp, active);
  else
    hipLaunchKernelGGL(transpose_pad_kernel<float>, grid, dim3(256), 0, st, (const float*)src,
                       lds_, R, C, (float*)dst, ldd, Rp, active);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

template <typename T>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            int64_t stride, int S, int64_t M,
                                                            int64_t N, int64_t ldp, T* __restrict__ out,
                                                            int64_t ldo, const int* __restrict__ active) {
  const bool on = !(active && *active == 0);
  const int64_t n4 = N / 4;
  const int64_t total = M * n4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / n4, n = (i - m * n4) * 4;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    if (on) {
      for (int s = 0; s < S; ++s) {
        const float4 b = *reinterpret_cast<const float4*>(part + s * stride + m * ldp + n);
        a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
      }
    }
    Elem<T>::store(out, m * ldo + n + 0, a.x);
    Elem<T>::store(out, m * ldo + n + 1, a.y);
    Elem<T>::store(out, m * ldo + n + 2, a.z);
    Elem<T>::store(out, m * ldo + n + 3, a.w);
  }
}

sbp_status splitk_reduce(int dtype, const float* part, int64_t split_stride, int S, int64_t M,
                         int64_t N, int64_t ldp, void* out, int64_t ldo, const int* active,
                         hipStream_t st) {
  if (N % 4 != 0 || ldp % 4 != 0)
    return set_error(SBP_ERR_UNSUPPORTED, "splitk_reduce needs N %% 4 == 0");
  const size_t esz = dtype == SBP_BF16 ? 2 : 4;
  ProfScope prof("splitk_reduce", st, 0.0, (double)M * N * (4.0 * S + esz));
  const int64_t total = M * (N / 4);
  const unsigned grid = (unsigned)std::min<int64_t>(cdiv(total, 256), 4096);
  if (dtype == SBP_BF16)
    hipLaunchKernelGGL(splitk_reduce_kernel<bf16_t>, dim3(grid), dim3(256), 0, st, part,
                       split_stride, S, M, N, ldp, (bf16_t*)out, ldo, active);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<float>, dim3(grid), dim3(256), 0, st, part,
                       split_stride, S, M, N, ldp, (float*)out, ldo, active);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n,
                                                        const int* __restrict__ when) {
  if (when && *when == 0) return;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

sbp_status fill_zero_f32(float* p, int64_t n, const int* when, hipStream_t st) {
  if (n <= 0) return SBP_OK;
  // a conditional fill is credited no bytes: whether it writes is decided on
  // the device (it returns at once unless *when != 0)
  ProfScope prof("fill_zero", st, 0.0, when ? 0.0 : 4.0 * n);
  const unsigned grid = (unsigned)std::min<int64_t>(cdiv(n, 256), 8192);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid), dim3(256), 0, st, p, n, when);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

__global__ __launch_bounds__(256) void fill_zero_u32_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

sbp_status fill_zero_bytes(void* p, int64_t nbytes, hipStream_t st) {
  if (nbytes <= 0) return SBP_OK;
  if (nbytes % 4 != 0) return set_error(SBP_ERR_INVALID_ARG, "fill_zero_bytes: size %% 4");
  const int64_t n = nbytes / 4;
  ProfScope prof("fill_zero", st, 0.0, (double)nbytes);
  const unsigned grid = (unsigned)std::min<int64_t>(cdiv(n, 256), 8192);
  hipLaunchKernelGGL(fill_zero_u32_kernel, dim3(grid), dim3(256), 0, st, (uint32_t*)p, n);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

}  // namespace sbp
