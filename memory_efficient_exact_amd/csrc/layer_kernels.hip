// Token-wise kernels of the decoder layer: RMSNorm forward/backward, the
// gain-gradient column sums, SwiGLU forward/backward and fp32 -> bf16 row
// conversion.  All are HBM-bound row/elementwise passes.
//
// RMSNorm(x; g) = g * x / r, r = sqrt(mean(x^2) + eps).  With upstream dy
// and xhat = x / r:  dx = (g * dy - xhat * mean(xhat * g * dy)) / r  and
// dg = sum over tokens of dy * xhat (from d xhat_k / d x_j =
// (delta_kj - xhat_k xhat_j / n) / r).
// SwiGLU: m = silu(u) * g with silu(u) = u sigma(u); du = dm * g * silu'(u),
// silu'(u) = sigma(u) (1 + u (1 - sigma(u))); dg = dm * silu(u).
#include "common.h"
#include "kernels.h"

namespace sbp {

__device__ __forceinline__ float block_sum256(float v, float* sh) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  return sh[0] + sh[1] + sh[2] + sh[3];
}

// one block per row
__global__ __launch_bounds__(256) void rmsnorm_fwd_kernel(const bf16_t* __restrict__ x, int64_t ldx,
                                                          const bf16_t* __restrict__ g, int d,
                                                          float eps, bf16_t* __restrict__ out,
                                                          int64_t ldo, float* __restrict__ rinv) {
  __shared__ float sh[4];
  const int64_t r = blockIdx.x;
  const bf16_t* xr = x + r * ldx;
  float ss = 0.f;
  for (int j = threadIdx.x; j < d; j += 256) {
    const float v = bf2f(xr[j]);
    ss += v * v;
  }
  ss = block_sum256(ss, sh);
  const float ri = rsqrtf(ss / (float)d + eps);
  if (threadIdx.x == 0) rinv[r] = ri;
  for (int j = threadIdx.x; j < d; j += 256) out[r * ldo + j] = f2bf(bf2f(g[j]) * bf2f(xr[j]) * ri);
}

sbp_status rmsnorm_fwd(const void* x, int64_t ldx, const void* g, int64_t rows, int64_t d,
                       float eps, void* out, int64_t ldo, float* rinv, hipStream_t st) {
  if (rows <= 0) return SBP_OK;
  ProfScope prof("rmsnorm_fwd", st, 0.0, 4.0 * rows * d);
  hipLaunchKernelGGL(rmsnorm_fwd_kernel, dim3((unsigned)rows), dim3(256), 0, st, (const bf16_t*)x, ldx,
                     (const bf16_t*)g, (int)d, eps, (bf16_t*)out, ldo, rinv);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

// out = resid + (g * dn - xhat * mean(xhat * g * dn)) * rinv, one block per row
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(
    const bf16_t* __restrict__ x, int64_t ldx, const bf16_t* __restrict__ g,
    const float* __restrict__ dn, int64_t ldn, const float* __restrict__ rinv,
    const bf16_t* __restrict__ resid, int64_t ldr, int d, bf16_t* __restrict__ out, int64_t ldo) {
  __shared__ float sh[4];
  const int64_t r = blockIdx.x;
  const float ri = rinv[r];
  float acc = 0.f;
  for (int j = threadIdx.x; j < d; j += 256) {
    const float xh = bf2f(x[r * ldx + j]) * ri;
    acc += xh * bf2f(g[j]) * dn[r * ldn + j];
  }
  const float mean = block_sum256(acc, sh) / (float)d;
  for (int j = threadIdx.x; j < d; j += 256) {
    const float xh = bf2f(x[r * ldx + j]) * ri;
    const float v = (bf2f(g[j]) * dn[r * ldn + j] - xh * mean) * ri;
    out[r * ldo + j] = f2bf(bf2f(resid[r * ldr + j]) + v);
  }
}

sbp_status rmsnorm_bwd(const void* x, int64_t ldx, const void* g, const float* dn, int64_t ldn,
                       const float* rinv, const void* resid, int64_t ldr, int64_t rows, int64_t d,
                       void* out, int64_t ldo, hipStream_t st) {
  if (rows <= 0) return SBP_OK;
  ProfScope prof("rmsnorm_bwd", st, 0.0, 10.0 * rows * d);
  hipLaunchKernelGGL(rmsnorm_bwd_kernel, dim3((unsigned)rows), dim3(256), 0, st, (const bf16_t*)x, ldx,
                     (const bf16_t*)g, dn, ldn, rinv, (const bf16_t*)resid, ldr, (int)d,
                     (bf16_t*)out, ldo);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

// dg[j] (+)= sum_r dn[r][j] * x[r][j] * rinv[r]; 64 columns per block,
// 4 row groups reduced through LDS (deterministic, no atomics).
__global__ __launch_bounds__(256) void gain_grad_kernel(const float* __restrict__ dn, int64_t ldn,
                                                        const bf16_t* __restrict__ x, int64_t ldx,
                                                        const float* __restrict__ rinv, int64_t rows,
                                                        int d, float* __restrict__ dg, int beta) {
  __shared__ float sh[4][64];
  const int c = threadIdx.x & 63, rg = threadIdx.x >> 6;
  const int j = blockIdx.x * 64 + c;
  float acc = 0.f;
  if (j < d)
    for (int64_t r = rg; r < rows; r += 4) acc += dn[r * ldn + j] * bf2f(x[r * ldx + j]) * rinv[r];
  sh[rg][c] = acc;
  __syncthreads();
  if (rg == 0 && j < d) {
    const float s = sh[0][c] + sh[1][c] + sh[2][c] + sh[3][c];
    dg[j] = beta ? dg[j] + s : s;
  }
}

sbp_status gain_grad(const float* dn, int64_t ldn, const void* x, int64_t ldx, const float* rinv,
                     int64_t rows, int64_t d, float* dg, int beta, hipStream_t st) {
  ProfScope prof("gain_grad", st, 0.0, 6.0 * rows * d);
  hipLaunchKernelGGL(gain_grad_kernel, dim3((unsigned)cdiv(d, 64)), dim3(256), 0, st, dn, ldn,
                     (const bf16_t*)x, ldx, rinv, rows, (int)d, dg, beta);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

__device__ __forceinline__ float sigmoidf_(float u) { return 1.f / (1.f + __expf(-u)); }

// ug = [u | g] rows of 2F; m = silu(u) * g
__global__ __launch_bounds__(256) void swiglu_fwd_kernel(const bf16_t* __restrict__ ug, int64_t rows,
                                                         int64_t F, bf16_t* __restrict__ m) {
  const int64_t n = rows * F;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / F, j = i - r * F;
    const float u = bf2f(ug[r * 2 * F + j]), gg = bf2f(ug[r * 2 * F + F + j]);
    m[i] = f2bf(u * sigmoidf_(u) * gg);
  }
}

sbp_status swiglu_fwd(const void* ug, int64_t rows, int64_t F, void* m, hipStream_t st) {
  ProfScope prof("swiglu_fwd", st, 0.0, 6.0 * rows * F);
  const unsigned grid = (unsigned)std::min<int64_t>(cdiv(rows * F, 256), 16384);
  hipLaunchKernelGGL(swiglu_fwd_kernel, dim3(grid), dim3(256), 0, st, (const bf16_t*)ug, rows, F,
                     (bf16_t*)m);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

// dudg = [du | dg] rows of 2F from dm [rows, F] and ug
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const bf16_t* __restrict__ dm,
                                                         const bf16_t* __restrict__ ug, int64_t rows,
                                                         int64_t F, bf16_t* __restrict__ dudg) {
  const int64_t n = rows * F;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / F, j = i - r * F;
    const float u = bf2f(ug[r * 2 * F + j]), gg = bf2f(ug[r * 2 * F + F + j]);
    const float d = bf2f(dm[i]);
    const float s = sigmoidf_(u);
    dudg[r * 2 * F + j] = f2bf(d * gg * s * (1.f + u * (1.f - s)));
    dudg[r * 2 * F + F + j] = f2bf(d * u * s);
  }
}

sbp_status swiglu_bwd(const void* dm, const void* ug, int64_t rows, int64_t F, void* dudg,
                      hipStream_t st) {
  ProfScope prof("swiglu_bwd", st, 0.0, 10.0 * rows * F);
  const unsigned grid = (unsigned)std::min<int64_t>(cdiv(rows * F, 256), 16384);
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3(grid), dim3(256), 0, st, (const bf16_t*)dm,
                     (const bf16_t*)ug, rows, F, (bf16_t*)dudg);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

__global__ __launch_bounds__(256) void rows_to_bf16_kernel(const float* __restrict__ src, int64_t lds_,
                                                           int64_t rows, int64_t cols,
                                                           bf16_t* __restrict__ dst, int64_t ldd) {
  const int64_t n = rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / cols, j = i - r * cols;
    dst[r * ldd + j] = f2bf(src[r * lds_ + j]);
  }
}

sbp_status rows_to_bf16(const float* src, int64_t lds_, int64_t rows, int64_t cols, void* dst,
                        int64_t ldd, hipStream_t st) {
  if (rows <= 0) return SBP_OK;
  ProfScope prof("rows_to_bf16", st, 0.0, 6.0 * rows * cols);
  const unsigned grid = (unsigned)std::min<int64_t>(cdiv(rows * cols, 256), 16384);
  hipLaunchKernelGGL(rows_to_bf16_kernel, dim3(grid), dim3(256), 0, st, src, lds_, rows, cols,
                     (bf16_t*)dst, ldd);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

}  // namespace sbp
