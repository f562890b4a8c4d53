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
// Rotary position embedding (RoFormer, Su et al.): a head vector of width dh
// is split into halves (x1, x2) and pair i turns by p * theta^(-2i/dh), p the
// token's position: out1 = x1 cos - x2 sin, out2 = x2 cos + x1 sin.  A
// rotation's inverse is its transpose, so gradients turn by the negative
// angle.
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

// 8 bf16 <-> 8 fp32 (16-byte vectors; every row pitch and base here is a
// multiple of 8 elements and 16-byte aligned).
__device__ __forceinline__ void unpack8(const uint4& u, float (&f)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[2 * k] = bf2f((bf16_t)(w[k] & 0xffff));
    f[2 * k + 1] = bf2f((bf16_t)(w[k] >> 16));
  }
}
__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  return make_uint4(pk_bf16(f[0], f[1]), pk_bf16(f[2], f[3]), pk_bf16(f[4], f[5]), pk_bf16(f[6], f[7]));
}
__device__ __forceinline__ void load8f(const float* p, float (&f)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
// 8 consecutive elements of a bf16 or fp32 row (16-byte aligned) <-> fp32
__device__ __forceinline__ void ld8(const bf16_t* p, float (&f)[8]) { unpack8(*reinterpret_cast<const uint4*>(p), f); }
__device__ __forceinline__ void ld8(const float* p, float (&f)[8]) { load8f(p, f); }
__device__ __forceinline__ void st8(bf16_t* p, const float (&f)[8]) { *reinterpret_cast<uint4*>(p) = pack8(f); }
__device__ __forceinline__ void st8(float* p, const float (&f)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(f[0], f[1], f[2], f[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(f[4], f[5], f[6], f[7]);
}
__device__ __forceinline__ float ld1(const bf16_t* p) { return bf2f(*p); }
__device__ __forceinline__ float ld1(const float* p) { return *p; }
__device__ __forceinline__ void st1(bf16_t* p, float v) { *p = f2bf(v); }
__device__ __forceinline__ void st1(float* p, float v) { *p = v; }

// one block per row, 8 elements per thread and step
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_fwd_kernel(const T* __restrict__ x, int64_t ldx,
                                                          const T* __restrict__ g, int d,
                                                          float eps, T* __restrict__ out,
                                                          int64_t ldo, float* __restrict__ rinv) {
  __shared__ float sh[4];
  const int64_t r = blockIdx.x;
  const T* xr = x + r * ldx;
  float ss = 0.f;
  for (int j = threadIdx.x * 8; j < d; j += 2048) {
    float v[8];
    ld8(xr + j, v);
#pragma unroll
    for (int k = 0; k < 8; ++k) ss += v[k] * v[k];
  }
  ss = block_sum256(ss, sh);
  const float ri = rsqrtf(ss / (float)d + eps);
  if (threadIdx.x == 0) rinv[r] = ri;
  for (int j = threadIdx.x * 8; j < d; j += 2048) {
    float v[8], gg[8];
    ld8(xr + j, v);
    ld8(g + j, gg);
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = gg[k] * v[k] * ri;
    st8(out + r * ldo + j, v);
  }
}

sbp_status rmsnorm_fwd(const void* x, int64_t ldx, const void* g, int64_t rows, int64_t d,
                       float eps, void* out, int64_t ldo, float* rinv, hipStream_t st, int dtype) {
  if (rows <= 0) return SBP_OK;
  if (d % 8 || ldx % 8 || ldo % 8) return set_error(SBP_ERR_INVALID_ARG, "rmsnorm_fwd: d and pitches must be multiples of 8");
  ProfScope prof("rmsnorm_fwd", st, 0.0, (dtype == SBP_F32 ? 8.0 : 4.0) * rows * d);
  if (dtype == SBP_F32)
    hipLaunchKernelGGL(rmsnorm_fwd_kernel<float>, dim3((unsigned)rows), dim3(256), 0, st, (const float*)x, ldx,
                       (const float*)g, (int)d, eps, (float*)out, ldo, rinv);
  else
    hipLaunchKernelGGL(rmsnorm_fwd_kernel<bf16_t>, dim3((unsigned)rows), dim3(256), 0, st, (const bf16_t*)x, ldx,
                       (const bf16_t*)g, (int)d, eps, (bf16_t*)out, ldo, rinv);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

// out = resid + (g * dn - xhat * mean(xhat * g * dn)) * rinv, one block per row
// (resid NULL: no residual term)
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(
    const T* __restrict__ x, int64_t ldx, const T* __restrict__ g,
    const float* __restrict__ dn, int64_t ldn, const float* __restrict__ rinv,
    const T* __restrict__ resid, int64_t ldr, int d, T* __restrict__ out, int64_t ldo) {
  __shared__ float sh[4];
  const int64_t r = blockIdx.x;
  const float ri = rinv[r];
  float acc = 0.f;
  for (int j = threadIdx.x * 8; j < d; j += 2048) {
    float xv[8], gv[8], dv[8];
    ld8(x + r * ldx + j, xv);
    ld8(g + j, gv);
    load8f(dn + r * ldn + j, dv);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += xv[k] * ri * gv[k] * dv[k];
  }
  const float mean = block_sum256(acc, sh) / (float)d;
  for (int j = threadIdx.x * 8; j < d; j += 2048) {
    float xv[8], gv[8], dv[8], rv[8];
    ld8(x + r * ldx + j, xv);
    ld8(g + j, gv);
    load8f(dn + r * ldn + j, dv);
    if (resid) {
      ld8(resid + r * ldr + j, rv);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) rv[k] = 0.f;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) rv[k] += (gv[k] * dv[k] - xv[k] * ri * mean) * ri;
    st8(out + r * ldo + j, rv);
  }
}

sbp_status rmsnorm_bwd(const void* x, int64_t ldx, const void* g, const float* dn, int64_t ldn,
                       const float* rinv, const void* resid, int64_t ldr, int64_t rows, int64_t d,
                       void* out, int64_t ldo, hipStream_t st, int dtype) {
  if (rows <= 0) return SBP_OK;
  if (d % 8 || ldx % 8 || ldn % 8 || ldr % 8 || ldo % 8)
    return set_error(SBP_ERR_INVALID_ARG, "rmsnorm_bwd: d and pitches must be multiples of 8");
  ProfScope prof("rmsnorm_bwd", st, 0.0, (dtype == SBP_F32 ? 16.0 : 10.0) * rows * d);
  if (dtype == SBP_F32)
    hipLaunchKernelGGL(rmsnorm_bwd_kernel<float>, dim3((unsigned)rows), dim3(256), 0, st, (const float*)x, ldx,
                       (const float*)g, dn, ldn, rinv, (const float*)resid, ldr, (int)d, (float*)out, ldo);
  else
    hipLaunchKernelGGL(rmsnorm_bwd_kernel<bf16_t>, dim3((unsigned)rows), dim3(256), 0, st, (const bf16_t*)x, ldx,
                       (const bf16_t*)g, dn, ldn, rinv, (const bf16_t*)resid, ldr, (int)d,
                       (bf16_t*)out, ldo);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

// dg[j] (+)= sum_r dn[r][j] * x[r][j] * rinv[r].
// Pass 1: block (256 columns, row split s); each thread owns 4 columns
// (float4 of dn, 4 bf16 of x), the 4 waves stride the split's rows and are
// summed through LDS into part[s][j].  Pass 2 sums the splits in order, so
// the result is deterministic.
__device__ __forceinline__ float4 ld4f(const bf16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(bf2f((bf16_t)(u.x & 0xffff)), bf2f((bf16_t)(u.x >> 16)),
                     bf2f((bf16_t)(u.y & 0xffff)), bf2f((bf16_t)(u.y >> 16)));
}
__device__ __forceinline__ float4 ld4f(const float* p) { return *reinterpret_cast<const float4*>(p); }

template <typename T>
__global__ __launch_bounds__(256) void gain_part_kernel(const float* __restrict__ dn, int64_t ldn,
                                                        const T* __restrict__ x, int64_t ldx,
                                                        const float* __restrict__ rinv, int64_t rows,
                                                        int d, int64_t rps, float* __restrict__ part) {
  __shared__ float4 sh[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = blockIdx.x * 256 + lane * 4;
  const int64_t r0 = (int64_t)blockIdx.y * rps, r1 = min(rows, r0 + rps);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (j < d)
    for (int64_t r = r0 + w; r < r1; r += 4) {
      const float4 g = *reinterpret_cast<const float4*>(dn + r * ldn + j);
      const float4 xv = ld4f(x + r * ldx + j);
      const float ri = rinv[r];
      acc.x += g.x * xv.x * ri;
      acc.y += g.y * xv.y * ri;
      acc.z += g.z * xv.z * ri;
      acc.w += g.w * xv.w * ri;
    }
  sh[w][lane] = acc;
  __syncthreads();
  if (w == 0 && j < d) {
    float4 t = sh[0][lane];
#pragma unroll
    for (int k = 1; k < 4; ++k) {
      t.x += sh[k][lane].x;
      t.y += sh[k][lane].y;
      t.z += sh[k][lane].z;
      t.w += sh[k][lane].w;
    }
    *reinterpret_cast<float4*>(part + (int64_t)blockIdx.y * d + j) = t;
  }
}

__global__ __launch_bounds__(256) void gain_sum_kernel(const float* __restrict__ part, int nsplit,
                                                       int d, float* __restrict__ dg, int beta) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= d) return;
  float s = 0.f;
  for (int k = 0; k < nsplit; ++k) s += part[(int64_t)k * d + j];
  dg[j] = beta ? dg[j] + s : s;
}

int gain_grad_splits(int64_t rows) { return (int)std::max<int64_t>(1, std::min<int64_t>(64, rows / 32)); }

sbp_status gain_grad(const float* dn, int64_t ldn, const void* x, int64_t ldx, const float* rinv,
                     int64_t rows, int64_t d, float* dg, int beta, float* part, hipStream_t st,
                     int dtype) {
  if ((uintptr_t)dn % 16 || (uintptr_t)x % (dtype == SBP_F32 ? 16 : 8) || (uintptr_t)part % 16 ||
      ldn % 4 || ldx % 4 || d % 4)
    return set_error(SBP_ERR_INVALID_ARG, "gain_grad: rows must be 16-byte (fp32) / 8-byte (bf16) aligned");
  ProfScope prof("gain_grad", st, 0.0, (dtype == SBP_F32 ? 8.0 : 6.0) * rows * d);
  const int ns = gain_grad_splits(rows);
  const int64_t rps = cdiv(std::max<int64_t>(rows, 1), ns);
  if (dtype == SBP_F32)
    hipLaunchKernelGGL(gain_part_kernel<float>, dim3((unsigned)cdiv(d, 256), (unsigned)ns), dim3(256), 0, st,
                       dn, ldn, (const float*)x, ldx, rinv, rows, (int)d, rps, part);
  else
    hipLaunchKernelGGL(gain_part_kernel<bf16_t>, dim3((unsigned)cdiv(d, 256), (unsigned)ns), dim3(256), 0, st,
                       dn, ldn, (const bf16_t*)x, ldx, rinv, rows, (int)d, rps, part);
  SBP_LAUNCH_CHECK();
  hipLaunchKernelGGL(gain_sum_kernel, dim3((unsigned)cdiv(d, 256)), dim3(256), 0, st, part, ns, (int)d,
                     dg, beta);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

__device__ __forceinline__ float sigmoidf_(float u) { return 1.f / (1.f + __expf(-u)); }

// ug = [u | g] rows of 2F; m = silu(u) * g, 8 elements per thread and step
template <typename T>
__global__ __launch_bounds__(256) void swiglu_fwd_kernel(const T* __restrict__ ug, int64_t rows,
                                                         int64_t F, T* __restrict__ m) {
  const int64_t F8 = F / 8, n = rows * F8;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / F8, j = (i - r * F8) * 8;
    float u[8], gg[8], o[8];
    ld8(ug + r * 2 * F + j, u);
    ld8(ug + r * 2 * F + F + j, gg);
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = u[k] * sigmoidf_(u[k]) * gg[k];
    st8(m + r * F + j, o);
  }
}

sbp_status swiglu_fwd(const void* ug, int64_t rows, int64_t F, void* m, hipStream_t st, int dtype) {
  if (F % 8) return set_error(SBP_ERR_INVALID_ARG, "swiglu_fwd: F must be a multiple of 8");
  ProfScope prof("swiglu_fwd", st, 0.0, (dtype == SBP_F32 ? 12.0 : 6.0) * rows * F);
  const unsigned grid = (unsigned)std::min<int64_t>(cdiv(rows * F / 8, 256), 16384);
  if (dtype == SBP_F32)
    hipLaunchKernelGGL(swiglu_fwd_kernel<float>, dim3(grid), dim3(256), 0, st, (const float*)ug, rows, F,
                       (float*)m);
  else
    hipLaunchKernelGGL(swiglu_fwd_kernel<bf16_t>, dim3(grid), dim3(256), 0, st, (const bf16_t*)ug, rows, F,
                       (bf16_t*)m);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

// dudg = [du | dg] rows of 2F from dm [rows, F] and ug
template <typename T>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const T* __restrict__ dm,
                                                         const T* __restrict__ ug, int64_t rows,
                                                         int64_t F, T* __restrict__ dudg) {
  const int64_t F8 = F / 8, n = rows * F8;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / F8, j = (i - r * F8) * 8;
    float u[8], gg[8], d[8], du[8], dg[8];
    ld8(ug + r * 2 * F + j, u);
    ld8(ug + r * 2 * F + F + j, gg);
    ld8(dm + r * F + j, d);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float sg = sigmoidf_(u[k]);
      du[k] = d[k] * gg[k] * sg * (1.f + u[k] * (1.f - sg));
      dg[k] = d[k] * u[k] * sg;
    }
    st8(dudg + r * 2 * F + j, du);
    st8(dudg + r * 2 * F + F + j, dg);
  }
}

sbp_status swiglu_bwd(const void* dm, const void* ug, int64_t rows, int64_t F, void* dudg,
                      hipStream_t st, int dtype) {
  if (F % 8) return set_error(SBP_ERR_INVALID_ARG, "swiglu_bwd: F must be a multiple of 8");
  ProfScope prof("swiglu_bwd", st, 0.0, (dtype == SBP_F32 ? 20.0 : 10.0) * rows * F);
  const unsigned grid = (unsigned)std::min<int64_t>(cdiv(rows * F / 8, 256), 16384);
  if (dtype == SBP_F32)
    hipLaunchKernelGGL(swiglu_bwd_kernel<float>, dim3(grid), dim3(256), 0, st, (const float*)dm,
                       (const float*)ug, rows, F, (float*)dudg);
  else
    hipLaunchKernelGGL(swiglu_bwd_kernel<bf16_t>, dim3(grid), dim3(256), 0, st, (const bf16_t*)dm,
                       (const bf16_t*)ug, rows, F, (bf16_t*)dudg);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

__global__ __launch_bounds__(256) void rows_to_bf16_kernel(const float* __restrict__ src, int64_t lds_,
                                                           int64_t rows, int64_t cols,
                                                           bf16_t* __restrict__ dst, int64_t ldd) {
  const int64_t C8 = cols / 8, n = rows * C8;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / C8, j = (i - r * C8) * 8;
    float v[8];
    load8f(src + r * lds_ + j, v);
    *reinterpret_cast<uint4*>(dst + r * ldd + j) = pack8(v);
  }
}

sbp_status rows_to_bf16(const float* src, int64_t lds_, int64_t rows, int64_t cols, void* dst,
                        int64_t ldd, hipStream_t st) {
  if (rows <= 0) return SBP_OK;
  if (cols % 8 || lds_ % 8 || ldd % 8) return set_error(SBP_ERR_INVALID_ARG, "rows_to_bf16: sizes must be multiples of 8");
  ProfScope prof("rows_to_bf16", st, 0.0, 6.0 * rows * cols);
  const unsigned grid = (unsigned)std::min<int64_t>(cdiv(rows * cols / 8, 256), 16384);
  hipLaunchKernelGGL(rows_to_bf16_kernel, dim3(grid), dim3(256), 0, st, src, lds_, rows, cols,
                     (bf16_t*)dst, ldd);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

__global__ __launch_bounds__(256) void rows_to_f32_kernel(const bf16_t* __restrict__ src, int64_t lds_,
                                                          int64_t rows, int64_t cols,
                                                          float* __restrict__ dst, int64_t ldd) {
  const int64_t C8 = cols / 8, n = rows * C8;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / C8, j = (i - r * C8) * 8;
    float v[8];
    unpack8(*reinterpret_cast<const uint4*>(src + r * lds_ + j), v);
    float4* o = reinterpret_cast<float4*>(dst + r * ldd + j);
    o[0] = make_float4(v[0], v[1], v[2], v[3]);
    o[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

sbp_status rows_to_f32(const void* src, int64_t lds_, int64_t rows, int64_t cols, float* dst,
                       int64_t ldd, hipStream_t st) {
  if (rows <= 0) return SBP_OK;
  if (cols % 8 || lds_ % 8 || ldd % 8) return set_error(SBP_ERR_INVALID_ARG, "rows_to_f32: sizes must be multiples of 8");
  ProfScope prof("rows_to_f32", st, 0.0, 6.0 * rows * cols);
  const unsigned grid = (unsigned)std::min<int64_t>(cdiv(rows * cols / 8, 256), 16384);
  hipLaunchKernelGGL(rows_to_f32_kernel, dim3(grid), dim3(256), 0, st, (const bf16_t*)src, lds_,
                     rows, cols, dst, ldd);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

// QK-norm: RMSNorm of every head vector (width dh = 64 or 128) of a [rows, H
// heads] tile with pitch ld, one gain of width dh for all heads.  One wave
// per (row, head); lane l holds elements l and l + 64.
template <typename T, int DH>
__global__ __launch_bounds__(256) void headnorm_fwd_kernel(const T* x, int64_t ldx,
                                                           T* out, int64_t ldo, int64_t rows,
                                                           int H, const T* __restrict__ g,
                                                           float eps) {
  constexpr int NE = DH / 64;
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= rows * H) return;
  const int64_t r = i / H;
  const int h = (int)(i - r * H);
  const T* xr = x + r * ldx + (int64_t)h * DH;
  float v[NE], ss = 0.f;
#pragma unroll
  for (int j = 0; j < NE; ++j) {
    v[j] = ld1(xr + lane + 64 * j);
    ss += v[j] * v[j];
  }
  const float ri = rsqrtf(wave_sum(ss) / (float)DH + eps);
  T* orow = out + r * ldo + (int64_t)h * DH;
#pragma unroll
  for (int j = 0; j < NE; ++j) st1(orow + lane + 64 * j, v[j] * ri * ld1(g + lane + 64 * j));
}

// dx = (g dy - xhat mean(xhat g dy)) / r per head vector (r recomputed from
// x), in place over dy allowed; per-block partial sums of dy * xhat into
// part[blockIdx.x][DH] (summed afterwards, so the result is deterministic).
template <typename T, int DH>
__global__ __launch_bounds__(256) void headnorm_bwd_kernel(const T* __restrict__ x, int64_t ldx,
                                                           const T* dy, int64_t ldy,
                                                           T* dx, int64_t ldd, int64_t rows,
                                                           int H, const T* __restrict__ g,
                                                           float eps, float* __restrict__ part) {
  constexpr int NE = DH / 64;
  __shared__ float sh[4][DH];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float gv[NE], acc[NE];
#pragma unroll
  for (int j = 0; j < NE; ++j) {
    gv[j] = ld1(g + lane + 64 * j);
    acc[j] = 0.f;
  }
  const int64_t n = rows * H;
  for (int64_t i = (int64_t)blockIdx.x * 4 + w; i < n; i += (int64_t)gridDim.x * 4) {
    const int64_t r = i / H;
    const int h = (int)(i - r * H);
    const T* xr = x + r * ldx + (int64_t)h * DH;
    const T* dr = dy + r * ldy + (int64_t)h * DH;
    float xv[NE], dv[NE], ss = 0.f, dot = 0.f;
#pragma unroll
    for (int j = 0; j < NE; ++j) {
      xv[j] = ld1(xr + lane + 64 * j);
      dv[j] = ld1(dr + lane + 64 * j);
      ss += xv[j] * xv[j];
    }
    const float ri = rsqrtf(wave_sum(ss) / (float)DH + eps);
#pragma unroll
    for (int j = 0; j < NE; ++j) {
      xv[j] *= ri;  // xhat
      dot += xv[j] * gv[j] * dv[j];
      acc[j] += dv[j] * xv[j];
    }
    const float mean = wave_sum(dot) / (float)DH;
    T* orow = dx + r * ldd + (int64_t)h * DH;
#pragma unroll
    for (int j = 0; j < NE; ++j) st1(orow + lane + 64 * j, (gv[j] * dv[j] - xv[j] * mean) * ri);
  }
#pragma unroll
  for (int j = 0; j < NE; ++j) sh[w][lane + 64 * j] = acc[j];
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int j = 0; j < NE; ++j) {
      const int c = lane + 64 * j;
      part[(int64_t)blockIdx.x * DH + c] = (sh[0][c] + sh[1][c]) + (sh[2][c] + sh[3][c]);
    }
  }
}

template <typename T>
static void headnorm_fwd_launch(const void* x, int64_t ldx, void* out, int64_t ldo, int64_t rows,
                                int H, int dh, const void* g, float eps, hipStream_t st) {
  const unsigned grid = (unsigned)cdiv(rows * H, 4);
  if (dh == 128)
    hipLaunchKernelGGL((headnorm_fwd_kernel<T, 128>), dim3(grid), dim3(256), 0, st, (const T*)x, ldx,
                       (T*)out, ldo, rows, H, (const T*)g, eps);
  else
    hipLaunchKernelGGL((headnorm_fwd_kernel<T, 64>), dim3(grid), dim3(256), 0, st, (const T*)x, ldx,
                       (T*)out, ldo, rows, H, (const T*)g, eps);
}

sbp_status headnorm_fwd(const void* x, int64_t ldx, void* out, int64_t ldo, int64_t rows, int H,
                        int dh, const void* g, float eps, hipStream_t st, int dtype) {
  if (rows <= 0) return SBP_OK;
  if ((dh != 64 && dh != 128) || ldx < (int64_t)H * dh || ldo < (int64_t)H * dh)
    return set_error(SBP_ERR_INVALID_ARG, "headnorm_fwd: bad head width or pitch");
  ProfScope prof("headnorm_fwd", st, 0.0, (dtype == SBP_F32 ? 8.0 : 4.0) * rows * H * dh);
  if (dtype == SBP_F32)
    headnorm_fwd_launch<float>(x, ldx, out, ldo, rows, H, dh, g, eps, st);
  else
    headnorm_fwd_launch<bf16_t>(x, ldx, out, ldo, rows, H, dh, g, eps, st);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

template <typename T>
static void headnorm_bwd_launch(const void* x, int64_t ldx, const void* dy, int64_t ldy, void* dx,
                                int64_t ldd, int64_t rows, int H, int dh, const void* g, float eps,
                                float* part, int nb, hipStream_t st) {
  if (dh == 128)
    hipLaunchKernelGGL((headnorm_bwd_kernel<T, 128>), dim3(nb), dim3(256), 0, st, (const T*)x, ldx,
                       (const T*)dy, ldy, (T*)dx, ldd, rows, H, (const T*)g, eps, part);
  else
    hipLaunchKernelGGL((headnorm_bwd_kernel<T, 64>), dim3(nb), dim3(256), 0, st, (const T*)x, ldx,
                       (const T*)dy, ldy, (T*)dx, ldd, rows, H, (const T*)g, eps, part);
}

sbp_status headnorm_bwd(const void* x, int64_t ldx, const void* dy, int64_t ldy, void* dx,
                        int64_t ldd, int64_t rows, int H, int dh, const void* g, float eps,
                        float* dg, int beta, float* part, hipStream_t st, int dtype) {
  if (rows <= 0) return SBP_OK;
  if ((dh != 64 && dh != 128) || ldx < (int64_t)H * dh || ldy < (int64_t)H * dh || ldd < (int64_t)H * dh)
    return set_error(SBP_ERR_INVALID_ARG, "headnorm_bwd: bad head width or pitch");
  ProfScope prof("headnorm_bwd", st, 0.0, (dtype == SBP_F32 ? 12.0 : 6.0) * rows * H * dh);
  const int nb = (int)std::min<int64_t>(cdiv(rows * H, 4), HEADNORM_PARTS);
  if (dtype == SBP_F32)
    headnorm_bwd_launch<float>(x, ldx, dy, ldy, dx, ldd, rows, H, dh, g, eps, part, nb, st);
  else
    headnorm_bwd_launch<bf16_t>(x, ldx, dy, ldy, dx, ldd, rows, H, dh, g, eps, part, nb, st);
  SBP_LAUNCH_CHECK();
  hipLaunchKernelGGL(gain_sum_kernel, dim3((unsigned)cdiv(dh, 256)), dim3(256), 0, st, part, nb, dh,
                     dg, beta);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

// tab[p * half + i] = (cos, sin) of p * theta^(-2i / (2 half)).  The angle is
// formed and reduced in double: at positions near 1e5 a float angle would
// already be off by ~1e-2 rad from rounding alone.
__global__ __launch_bounds__(256) void rope_table_kernel(float2* __restrict__ tab, int64_t P,
                                                         int half, double theta) {
  const int64_t n = P * half;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t p = i / half;
    const int j = (int)(i - p * half);
    const double f = pow(theta, -(double)j / (double)half);
    double sn, cs;
    sincos((double)p * f, &sn, &cs);
    tab[i] = make_float2((float)cs, (float)sn);
  }
}

sbp_status rope_table(float2* tab, int64_t P, int dh, double theta, hipStream_t st) {
  if (P <= 0) return SBP_OK;
  const int half = dh / 2;
  ProfScope prof("rope_table", st, 0.0, 8.0 * P * half);
  const unsigned grid = (unsigned)std::min<int64_t>(cdiv(P * half, 256), 8192);
  hipLaunchKernelGGL(rope_table_kernel, dim3(grid), dim3(256), 0, st, tab, P, half, theta);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

// One thread per (row, head, 8 consecutive pairs): reads 8 elements of each
// half and their 8 (cos, sin), writes both halves as bf16.  In place is safe
// (a thread reads all it writes first).
template <bool SRC_F32, typename TD>
__global__ __launch_bounds__(256) void rope_apply_kernel(const void* __restrict__ src, int64_t lds_,
                                                         TD* dst, int64_t ldd, int64_t rows,
                                                         int H, int dh, int64_t row0,
                                                         const int* __restrict__ seq_lo,
                                                         const float2* __restrict__ tab,
                                                         float sgn) {
  const int half = dh >> 1, G8 = half >> 3;
  const int64_t per_row = (int64_t)H * G8, n = rows * per_row;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / per_row;
    const int rem = (int)(i - r * per_row);
    const int h = rem / G8, g = rem - h * G8;
    const int64_t t = row0 + r;
    const int64_t p = seq_lo ? t - seq_lo[t] : t;
    const int64_t off = (int64_t)h * dh + g * 8;
    float x1[8], x2[8];
    if constexpr (SRC_F32) {
      const float* sp = reinterpret_cast<const float*>(src) + r * lds_ + off;
      load8f(sp, x1);
      load8f(sp + half, x2);
    } else {
      const bf16_t* sp = reinterpret_cast<const bf16_t*>(src) + r * lds_ + off;
      unpack8(*reinterpret_cast<const uint4*>(sp), x1);
      unpack8(*reinterpret_cast<const uint4*>(sp + half), x2);
    }
    const float4* tp = reinterpret_cast<const float4*>(tab + p * half + g * 8);
    float cs[8], sn[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 v = tp[k];
      cs[2 * k] = v.x; sn[2 * k] = sgn * v.y;
      cs[2 * k + 1] = v.z; sn[2 * k + 1] = sgn * v.w;
    }
    float o1[8], o2[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      o1[k] = x1[k] * cs[k] - x2[k] * sn[k];
      o2[k] = x2[k] * cs[k] + x1[k] * sn[k];
    }
    TD* dp = dst + r * ldd + off;
    st8(dp, o1);
    st8(dp + half, o2);
  }
}

sbp_status rope_apply(const void* src, bool src_f32, int64_t lds_, void* dst, int64_t ldd,
                      int64_t rows, int H, int dh, int64_t row0, const int* seq_lo,
                      const float2* tab, bool inverse, hipStream_t st, bool dst_f32) {
  if (rows <= 0) return SBP_OK;
  if (dh % 16 || lds_ % 8 || ldd % 8 || lds_ < (int64_t)H * dh || ldd < (int64_t)H * dh)
    return set_error(SBP_ERR_INVALID_ARG, "rope_apply: bad head width or pitch");
  if (dst_f32 && !src_f32) return set_error(SBP_ERR_INVALID_ARG, "rope_apply: fp32 output needs fp32 input");
  const int64_t n = rows * H * (dh / 16);
  const double eb = src_f32 ? 4.0 : 2.0;
  ProfScope prof("rope_apply", st, 0.0, (eb + (dst_f32 ? 4.0 : 2.0) + 4.0) * rows * H * dh);
  const unsigned grid = (unsigned)std::min<int64_t>(cdiv(n, 256), 16384);
  const float sgn = inverse ? -1.f : 1.f;
  if (dst_f32)
    hipLaunchKernelGGL((rope_apply_kernel<true, float>), dim3(grid), dim3(256), 0, st, src, lds_,
                       (float*)dst, ldd, rows, H, dh, row0, seq_lo, tab, sgn);
  else if (src_f32)
    hipLaunchKernelGGL((rope_apply_kernel<true, bf16_t>), dim3(grid), dim3(256), 0, st, src, lds_,
                       (bf16_t*)dst, ldd, rows, H, dh, row0, seq_lo, tab, sgn);
  else
    hipLaunchKernelGGL((rope_apply_kernel<false, bf16_t>), dim3(grid), dim3(256), 0, st, src, lds_,
                       (bf16_t*)dst, ldd, rows, H, dh, row0, seq_lo, tab, sgn);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

}  // namespace sbp
