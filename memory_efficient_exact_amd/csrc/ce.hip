// Softmax cross-entropy kernels of the chunked LM head.
//
// StreamBP skill page, "Implementation", logits-gradient routine: per-token
// cross-entropy, then softmax with one subtracted at the target column.  The
// normaliser is global (1/N over the valid tokens of the whole sequence, or
// 1 for a plain sum) so that the chunked gradient equals the unchunked one;
// a per-token weight multiplies (GRPO / DPO, "Practical Guidance", "Loss
// Objectives").
//
//   lm_prep     one block: N, 1/N, which chunks (and which groups of G
//               chunks sharing one dW GEMM) hold a valid token, and which
//               group's dW GEMM overwrites instead of adding.
//   ce_stats    one block per row: online max / sum-exp over the fp32 logits
//               row (wave64 shuffles, then LDS across waves) -> lse, l_t.
//   ce_merge    the same from the (max, sum-exp) partials that the bf16
//               logits GEMM writes per 64 columns (no pass over the row).
//   lp_rows     forward only: logprob = z_y - lse (and lse) per row, from
//               those partials and the GEMM's target logits, or from Z.
//   ce_grad     64 x 128 tiles: dZ = (c_t/N)(exp(z - lse) - onehot), written
//               twice in the GEMM operand layouts -- dZ [T_c, V] (K = V
//               contiguous for dH = dZ W) and dZ^T [V, T_c] (K = T_c
//               contiguous for dW = dZ^T H), the transpose staged in LDS.
//   loss_reduce one block, fp64 sum of c_t l_t, times 1/N.
#include "common.h"
#include "kernels.h"

namespace sbp {

__global__ __launch_bounds__(1024) void lm_prep_kernel(const int32_t* __restrict__ y, int64_t T,
                                                       int64_t V, int32_t D, int32_t G,
                                                       int reduction, int accumulate, LmPrep pr) {
  __shared__ int s_cnt[16];
  __shared__ int s_bad;
  __shared__ int s_first[16];
  const int tid = threadIdx.x;
  const int64_t size = T / D;
  for (int c = tid; c < D; c += blockDim.x) pr.chunk_active[c] = 0;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  int cnt = 0, bad = 0;
  for (int64_t t = tid; t < T; t += blockDim.x) {
    if (y[t] >= 0) {
      ++cnt;
      bad |= y[t] >= V;
      int64_t c = t / size;
      if (c > D - 1) c = D - 1;
      pr.chunk_active[c] = 1;
    }
  }
  // block sum of cnt
  for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
  if ((tid & 63) == 0) s_cnt[tid >> 6] = cnt;
  if (bad) s_bad = 1;
  __syncthreads();
  int first = D;
  for (int c = tid; c < D; c += blockDim.x)
    if (pr.chunk_active[c] && c < first) first = c;
  for (int o = 32; o > 0; o >>= 1) first = min(first, __shfl_xor(first, o, 64));
  if ((tid & 63) == 0) s_first[tid >> 6] = first;
  __syncthreads();
  if (tid == 0) {
    int n = 0, f = D;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
      n += s_cnt[w];
      f = min(f, s_first[w]);
    }
    s_cnt[0] = n;
    s_first[0] = f;
    *pr.n_valid = n;
    // a target id >= V (caller error) makes the normaliser NaN, and with it
    // the loss and every gradient the call writes
    *pr.inv_norm = s_bad ? __builtin_nanf("")
                         : (reduction == SBP_SUM ? 1.f : (n > 0 ? 1.f / (float)n : 0.f));
    *pr.none_active = (f == D) ? 1 : 0;
  }
  __syncthreads();
  const int f = s_first[0];
  const int ng = (D + G - 1) / G;
  for (int g = tid; g < ng; g += blockDim.x) {
    int any = 0;
    for (int c = g * G; c < min(D, (g + 1) * G); ++c) any |= pr.chunk_active[c];
    pr.group_active[g] = any;
    pr.beta_zero[g] = (!accumulate && f < D && g == f / G) ? 1 : 0;
  }
}

sbp_status lm_prep(const int32_t* targets, int64_t T, int64_t V, int32_t D, int32_t G,
                   int reduction, int accumulate, const LmPrep& pr, hipStream_t st) {
  ProfScope prof("lm_prep", st, 0.0, 4.0 * T);
  hipLaunchKernelGGL(lm_prep_kernel, dim3(1), dim3(1024), 0, st, targets, T, V, D, G, reduction,
                     accumulate, pr);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

// Merge two (max, sum-exp) pairs.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) {
    m = m2;
    s = s2;
    return;
  }
  const float mx = fmaxf(m, m2);
  s = s * __expf(m - mx) + s2 * __expf(m2 - mx);
  m = mx;
}

// Merge the (max, sum-exp) pairs of a 256-thread block (wave64 shuffles, then
// the four waves through LDS); the result is valid in thread 0.
__device__ __forceinline__ void block_lse(float& m, float& s) {
  __shared__ float sm[4], ss[4];
  const int tid = threadIdx.x;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64);
    const float s2 = __shfl_xor(s, o, 64);
    lse_merge(m, s, m2, s2);
  }
  if ((tid & 63) == 0) {
    sm[tid >> 6] = m;
    ss[tid >> 6] = s;
  }
  __syncthreads();
  if (tid == 0) {
    m = sm[0];
    s = ss[0];
    for (int w = 1; w < 4; ++w) lse_merge(m, s, sm[w], ss[w]);
  }
}

// Online (max, sum-exp) of this thread's share of a length-V fp32 row.
__device__ __forceinline__ void row_lse_partial(const float* __restrict__ z, int64_t V, float& m,
                                                float& s) {
  const int tid = threadIdx.x;
  const int64_t V4 = V & ~(int64_t)3;
  for (int64_t i = (int64_t)tid * 4; i < V4; i += 1024) {
    const float4 v = *reinterpret_cast<const float4*>(z + i);
    const float mx = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
    if (mx > m) {
      s = (m == -INFINITY) ? 0.f : s * __expf(m - mx);
      m = mx;
    }
    s += __expf(v.x - m) + __expf(v.y - m) + __expf(v.z - m) + __expf(v.w - m);
  }
  for (int64_t i = V4 + tid; i < V; i += 256) {
    const float v = z[i];
    if (v > m) {
      s = (m == -INFINITY) ? 0.f : s * __expf(m - v);
      m = v;
    }
    s += __expf(v - m);
  }
}

__global__ __launch_bounds__(256) void ce_stats_kernel(const float* __restrict__ Z, int64_t ldz,
                                                       const int32_t* __restrict__ targets,
                                                       const float* __restrict__ weights, int64_t s0,
                                                       int64_t V, float* __restrict__ lse_out,
                                                       float* __restrict__ loss_part,
                                                       float* __restrict__ token_loss) {
  const int r = blockIdx.x;
  const int64_t t = s0 + r;
  const int tid = threadIdx.x;
  const int y = targets[t];
  if (y < 0) {
    if (tid == 0) {
      loss_part[t] = 0.f;
      if (token_loss) token_loss[t] = 0.f;
      lse_out[r] = 0.f;
    }
    return;
  }
  const float* z = Z + (int64_t)r * ldz;
  float m = -INFINITY, s = 0.f;
  row_lse_partial(z, V, m, s);
  block_lse(m, s);
  if (tid == 0) {
    const float lse = m + __logf(s);
    // ids >= V are a caller error: the read stays inside the row, the loss is NaN
    const float ell = y < V ? lse - z[y] : __builtin_nanf("");
    const float w = weights ? weights[t] : 1.f;
    lse_out[r] = lse;
    loss_part[t] = w * ell;
    if (token_loss) token_loss[t] = ell;
  }
}

sbp_status ce_stats(const float* Z, int64_t ldz, const int32_t* targets, const float* weights,
                    int64_t s, int64_t Tc, int64_t V, float* lse, float* loss_part,
                    float* token_loss, hipStream_t st) {
  ProfScope prof("ce_stats", st, 0.0, 4.0 * (double)Tc * V);
  hipLaunchKernelGGL(ce_stats_kernel, dim3((unsigned)Tc), dim3(256), 0, st, Z, ldz, targets,
                     weights, s, V, lse, loss_part, token_loss);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

// Same outputs as ce_stats, from the logits GEMM's per-64-column (max,
// sum-exp) partials instead of a pass over the logits row, and the target
// logit the GEMM wrote in fp32.
__device__ __forceinline__ float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

__global__ __launch_bounds__(256) void ce_merge_kernel(const float2* __restrict__ parts, int64_t ldp,
                                                       int nparts, const float* __restrict__ ztgt,
                                                       const int32_t* __restrict__ targets,
                                                       const float* __restrict__ weights, int64_t s0,
                                                       int64_t V, float* __restrict__ lse_out,
                                                       float* __restrict__ loss_part,
                                                       float* __restrict__ token_loss) {
  const int r = blockIdx.x;
  const int64_t t = s0 + r;
  const int tid = threadIdx.x;
  const int y = targets[t];
  if (y < 0) {
    if (tid == 0) {
      loss_part[t] = 0.f;
      if (token_loss) token_loss[t] = 0.f;
      lse_out[r] = 0.f;
    }
    return;
  }
  float m = -INFINITY, sx = 0.f;
  for (int i = tid; i < nparts; i += 256) {
    const float2 q = parts[(int64_t)r * ldp + i];
    lse_merge(m, sx, q.x, q.y);
  }
  block_lse(m, sx);
  if (tid == 0) {
    const float lse = m + __logf(sx);
    // an id >= V has no target logit (caller error): NaN loss
    const float ell = y < V ? lse - ztgt[r] : __builtin_nanf("");
    const float w = weights ? weights[t] : 1.f;
    lse_out[r] = lse;
    loss_part[t] = w * ell;
    if (token_loss) token_loss[t] = ell;
  }
}

sbp_status ce_merge(const float2* parts, int64_t ldp, int nparts, const float* zt,
                    const int32_t* targets, const float* weights, int64_t s, int64_t Tc, int64_t V,
                    float* lse, float* loss_part, float* token_loss, hipStream_t st) {
  ProfScope prof("ce_merge", st, 0.0, 8.0 * (double)Tc * nparts);
  hipLaunchKernelGGL(ce_merge_kernel, dim3((unsigned)Tc), dim3(256), 0, st, parts, ldp, nparts, zt,
                     targets, weights, s, V, lse, loss_part, token_loss);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

// Per-token target log-probability (forward only): one block per row.
// PARTS: lse from the logits GEMM's per-64-column partials and the target
// logit from its target output; otherwise both from the fp32 logits row.
template <bool PARTS>
__global__ __launch_bounds__(256) void lp_rows_kernel(const float2* __restrict__ parts, int64_t ldp,
                                                      int nparts, const float* __restrict__ zt,
                                                      const float* __restrict__ Z, int64_t ldz,
                                                      int64_t V, const int32_t* __restrict__ targets,
                                                      int64_t s0, float* __restrict__ logprob,
                                                      float* __restrict__ lse_out) {
  const int r = blockIdx.x;
  const int64_t t = s0 + r;
  const int tid = threadIdx.x;
  const int y = targets[t];
  if (y < 0 || y >= V) {
    // ignored token: zeros; an id >= V (caller error): NaN, nothing read
    if (tid == 0) {
      const float f = y < 0 ? 0.f : __builtin_nanf("");
      logprob[t] = f;
      if (lse_out) lse_out[t] = f;
    }
    return;
  }
  float m = -INFINITY, sx = 0.f;
  if constexpr (PARTS) {
    for (int i = tid; i < nparts; i += 256) {
      const float2 q = parts[(int64_t)r * ldp + i];
      lse_merge(m, sx, q.x, q.y);
    }
  } else {
    row_lse_partial(Z + (int64_t)r * ldz, V, m, sx);
  }
  block_lse(m, sx);
  if (tid == 0) {
    const float lse = m + __logf(sx);
    const float zy = PARTS ? zt[r] : Z[(int64_t)r * ldz + y];
    logprob[t] = zy - lse;
    if (lse_out) lse_out[t] = lse;
  }
}

sbp_status lp_rows(const float2* parts, int64_t ldp, int nparts, const float* zt, const float* Z,
                   int64_t ldz, int64_t V, const int32_t* targets, int64_t s, int64_t Tc,
                   float* logprob, float* lse_out, hipStream_t st) {
  if (Tc <= 0) return SBP_OK;
  if (parts) {
    ProfScope prof("lp_rows", st, 0.0, 8.0 * (double)Tc * nparts);
    hipLaunchKernelGGL(lp_rows_kernel<true>, dim3((unsigned)Tc), dim3(256), 0, st, parts, ldp, nparts,
                       zt, Z, ldz, V, targets, s, logprob, lse_out);
  } else {
    ProfScope prof("lp_rows", st, 0.0, 4.0 * (double)Tc * V);
    hipLaunchKernelGGL(lp_rows_kernel<false>, dim3((unsigned)Tc), dim3(256), 0, st, parts, ldp, nparts,
                       zt, Z, ldz, V, targets, s, logprob, lse_out);
  }
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

template <typename OutT>
__device__ __forceinline__ void store8(OutT* p, const float* v);
template <>
__device__ __forceinline__ void store8<bf16_t>(bf16_t* p, const float* v) {
  uint4 u;
  u.x = pk_bf16(v[0], v[1]);
  u.y = pk_bf16(v[2], v[3]);
  u.z = pk_bf16(v[4], v[5]);
  u.w = pk_bf16(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = u;
}
template <>
__device__ __forceinline__ void store8<float>(float* p, const float* v) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// Tile: 64 rows (tokens of the chunk) x 128 columns (vocab).  With TR the
// tile is also written transposed (dZt, vocab-major).
// REL16: Z holds fp16 values relative to the max of their 64-column group
// (parts[r][v / 64].x), the logits GEMM's EPI_REL16_LSE output; dZ may then
// be Z itself (ldg == ldz): every thread writes exactly the 8 elements it
// read, after reading them.
template <typename OutT, bool TR, bool REL16>
__global__ __launch_bounds__(256) void ce_grad_kernel(
    const void* Zv, const float2* __restrict__ parts, int64_t ldp, int64_t ldz,
    const int32_t* __restrict__ targets,
    const float* __restrict__ weights, const float* __restrict__ inv_norm,
    const float* __restrict__ lse, int64_t s0, int64_t Tc, int64_t V, int64_t Vp,
    OutT* dZ, int64_t ldg, OutT* __restrict__ dZt, int64_t ldgt, int64_t Tcp,
    const int* __restrict__ active) {
  if (active && *active == 0) return;
  __shared__ float tile[TR ? 64 : 1][129];
  __shared__ float s_lse[64], s_sc[64];
  __shared__ int s_y[64];
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.y * 64;
  const int64_t v0 = (int64_t)blockIdx.x * 128;
  if (tid < 64) {
    const int64_t r = r0 + tid;
    int y = -1;
    float sc = 0.f, l = 0.f;
    if (r < Tc) {
      y = targets[s0 + r];
      if (y >= 0) {
        sc = (weights ? weights[s0 + r] : 1.f) * (*inv_norm);
        l = lse[r];
      }
    }
    s_y[tid] = y;
    s_sc[tid] = sc;
    s_lse[tid] = l;
  }
  __syncthreads();
  // pass 1: rows of dZ, 8 consecutive columns per thread
  {
    const int cg = tid & 15;       // 16 groups of 8 columns
    const int rr = tid >> 4;       // 16 rows per pass
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int lrow = rr + 16 * pass;
      const int64_t r = r0 + lrow;
      const int64_t v = v0 + cg * 8;
      float g[8];
      const int y = s_y[lrow];
      const float sc = s_sc[lrow], l = s_lse[lrow];
      if (REL16 && r < Tc && sc != 0.f) {
        // fp16 values relative to the group max: z = y + max (v is 8-aligned,
        // so the 8 columns share one 64-column group)
        const uint16_t* yr = reinterpret_cast<const uint16_t*>(Zv) + r * ldz;
        const float lm = (v < V ? parts[r * ldp + v / 64].x : 0.f) - l;
        if (v + 8 <= V) {
          const uint4 u = *reinterpret_cast<const uint4*>(yr + v);
          const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            g[2 * k] = f16_to_f32((uint16_t)(w4[k] & 0xffff));
            g[2 * k + 1] = f16_to_f32((uint16_t)(w4[k] >> 16));
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) g[j] = sc * (__expf(g[j] + lm) - ((v + j) == y ? 1.f : 0.f));
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            g[j] = (v + j < V) ? sc * (__expf(f16_to_f32(yr[v + j]) + lm) - ((v + j) == y ? 1.f : 0.f)) : 0.f;
        }
      } else if (!REL16 && r < Tc && sc != 0.f) {
        const float* zr = reinterpret_cast<const float*>(Zv) + r * ldz;
        if (v + 8 <= V) {
          const float4 a = *reinterpret_cast<const float4*>(zr + v);
          const float4 b = *reinterpret_cast<const float4*>(zr + v + 4);
          g[0] = a.x; g[1] = a.y; g[2] = a.z; g[3] = a.w;
          g[4] = b.x; g[5] = b.y; g[6] = b.z; g[7] = b.w;
#pragma unroll
          for (int j = 0; j < 8; ++j) g[j] = sc * (__expf(g[j] - l) - ((v + j) == y ? 1.f : 0.f));
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            g[j] = (v + j < V) ? sc * (__expf(zr[v + j] - l) - ((v + j) == y ? 1.f : 0.f)) : 0.f;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) g[j] = 0.f;
      }
      if (r < Tc && v < Vp) store8<OutT>(dZ + r * ldg + v, g);
      if constexpr (TR) {
#pragma unroll
        for (int j = 0; j < 8; ++j) tile[lrow][cg * 8 + j] = g[j];
      }
    }
  }
  if constexpr (!TR) return;
  __syncthreads();
  // pass 2: rows of dZ^T (vocab-major), 8 consecutive tokens per thread
  {
    const int rg = tid & 7;    // 8 groups of 8 tokens
    const int vc = tid >> 3;   // 32 vocab rows per pass
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int lcol = vc + 32 * pass;
      const int64_t v = v0 + lcol;
      const int64_t r = r0 + rg * 8;
      if (v < Vp && r < Tcp) {
        float g[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) g[j] = tile[TR ? rg * 8 + j : 0][lcol];
        store8<OutT>(dZt + v * ldgt + r, g);
      }
    }
  }
}

sbp_status ce_grad(int dtype, const void* Z, const float2* parts, int64_t ldp, int64_t ldz,
                   const int32_t* targets, const float* weights, const float* inv_norm,
                   const float* lse, int64_t s, int64_t Tc, int64_t V, int64_t Vp, void* dZ,
                   int64_t ldg, void* dZt, int64_t ldgt, int64_t Tcp, const int* active,
                   hipStream_t st) {
  const size_t esz = dtype == SBP_BF16 ? 2 : 4;
  if (parts && (dtype != SBP_BF16 || dZt || ldz % 8))
    return set_error(SBP_ERR_INVALID_ARG, "ce_grad: fp16 relative logits need bf16 output without dZ^T");
  ProfScope prof("ce_grad", st, 0.0, (double)Tc * V * ((parts ? 2.0 : 4.0) + (dZt ? 2.0 : 1.0) * esz));
  if (!dZt) Tcp = Tc;
  dim3 grid((unsigned)cdiv(Vp, 128), (unsigned)cdiv(Tcp, 64));
  if (parts)
    hipLaunchKernelGGL((ce_grad_kernel<bf16_t, false, true>), grid, dim3(256), 0, st, Z, parts, ldp, ldz,
                       targets, weights, inv_norm, lse, s, Tc, V, Vp, (bf16_t*)dZ, ldg, (bf16_t*)nullptr,
                       ldgt, Tcp, active);
  else if (dtype == SBP_BF16 && dZt)
    hipLaunchKernelGGL((ce_grad_kernel<bf16_t, true, false>), grid, dim3(256), 0, st, Z, parts, ldp, ldz,
                       targets, weights, inv_norm, lse, s, Tc, V, Vp, (bf16_t*)dZ, ldg, (bf16_t*)dZt,
                       ldgt, Tcp, active);
  else if (dtype == SBP_BF16)
    hipLaunchKernelGGL((ce_grad_kernel<bf16_t, false, false>), grid, dim3(256), 0, st, Z, parts, ldp, ldz,
                       targets, weights, inv_norm, lse, s, Tc, V, Vp, (bf16_t*)dZ, ldg, (bf16_t*)nullptr,
                       ldgt, Tcp, active);
  else if (dZt)
    hipLaunchKernelGGL((ce_grad_kernel<float, true, false>), grid, dim3(256), 0, st, Z, parts, ldp, ldz,
                       targets, weights, inv_norm, lse, s, Tc, V, Vp, (float*)dZ, ldg, (float*)dZt, ldgt,
                       Tcp, active);
  else
    hipLaunchKernelGGL((ce_grad_kernel<float, false, false>), grid, dim3(256), 0, st, Z, parts, ldp, ldz,
                       targets, weights, inv_norm, lse, s, Tc, V, Vp, (float*)dZ, ldg, (float*)nullptr,
                       ldgt, Tcp, active);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

__global__ __launch_bounds__(1024) void loss_reduce_kernel(const float* __restrict__ part,
                                                           int64_t T,
                                                           const float* __restrict__ inv_norm,
                                                           float* __restrict__ loss) {
  __shared__ double sh[16];
  double acc = 0.0;
  for (int64_t t = threadIdx.x; t < T; t += blockDim.x) acc += (double)part[t];
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) tot += sh[w];
    *loss = (float)(tot * (double)(*inv_norm));
  }
}

sbp_status loss_reduce(const float* loss_part, int64_t T, const float* inv_norm, float* loss,
                       hipStream_t st) {
  ProfScope prof("loss_reduce", st, 0.0, 4.0 * T);
  hipLaunchKernelGGL(loss_reduce_kernel, dim3(1), dim3(1024), 0, st, loss_part, T, inv_norm, loss);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

}  // namespace sbp
