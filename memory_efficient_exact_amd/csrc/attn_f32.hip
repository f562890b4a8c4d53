// fp32 mode of the chunked causal GQA attention: the same three steps as the
// bf16 kernels (forward statistics, dK/dV, dQ), every product an fp32 fused
// multiply-add, for the fp32 entry points (tolerance 1e-4 against the fp64
// definition).  Same chunking, masks and statistics layout as attn.hip
// (AttnArgs; its array pointers then hold fp32 data):
//
//   S = scale Q K^T, key j visible to query i iff j <= i (and, packed,
//   seq_lo[i] <= j); P = softmax(S); O = P V;  LSE in base-2 units;
//   Delta = rowsum(dO O);  dV += P^T dO;  dP = dO V^T;  dS = P (dP - Delta);
//   dQ = scale dS K;  dK += scale dS^T Q.
//
// Tiles live in LDS as rows of DH floats padded by 4 (16-byte aligned rows,
// consecutive rows 4 banks apart).  A block has 256 threads; score tiles are
// [32 or 64 queries x 64 keys], thread (ty = tid / 16, tx = tid % 16) holding
// rows ty + 16 i and columns tx + 16 j, so a row is spread over 16
// consecutive lanes and its reductions are 4 xor-shuffles.
#include "attn.h"
#include "common.h"

namespace sbp {
namespace {

constexpr float kL2E = 1.4426950408889634f;

__device__ __forceinline__ float row16_max(float v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// rows [0, R) of a [rows][DH] fp32 tile (global pitch ld) into LDS rows of
// pitch DH + 4; rows at or past nvalid are zeros
template <int DH, int R>
__device__ __forceinline__ void load_rows(float* lds, const float* __restrict__ src, int64_t ld,
                                          int nvalid) {
  constexpr int C4 = DH / 4, P = DH + 4;
  for (int i = threadIdx.x; i < R * C4; i += 256) {
    const int r = i / C4, c = (i - r * C4) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r < nvalid) v = *reinterpret_cast<const float4*>(src + (int64_t)r * ld + c);
    *reinterpret_cast<float4*>(lds + r * P + c) = v;
  }
}

__device__ __forceinline__ float dot4(const float4& a, const float4& b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

// Key j visible to query i (both absolute positions)?
__device__ __forceinline__ bool visible(const AttnArgs& a, int i, int j) {
  return j <= i && (!a.seq_lo || j >= a.seq_lo[i]);
}

// ---------------------------------------------------------------------------
// Forward statistics: block = 64 queries of one head; LSE (base 2), and O
// and Delta when asked for.
// ---------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(256) void attn_f32_fwd_kernel(AttnArgs a) {
  constexpr int P = DH + 4, NC = DH / 64;  // float4 column groups per thread
  __shared__ __attribute__((aligned(16))) float Qs[64 * P];
  __shared__ __attribute__((aligned(16))) float Ks[64 * P];
  __shared__ __attribute__((aligned(16))) float Vs[64 * P];
  __shared__ float Ps[64][68];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int h = blockIdx.y, b = blockIdx.z, kv = h / a.G;
  const int q0 = a.s + blockIdx.x * 64;
  const int64_t ldq = a.ldq, ldk = (int64_t)a.Hkv * DH;
  const float* Qg = reinterpret_cast<const float*>(a.Q) + (int64_t)b * a.q_bs + (int64_t)(q0 - a.qoff) * ldq + (int64_t)h * DH;
  const float* Kg = reinterpret_cast<const float*>(a.K) + (int64_t)b * a.T * ldk + (int64_t)kv * DH;
  const float* Vg = reinterpret_cast<const float*>(a.V) + (int64_t)b * a.T * ldk + (int64_t)kv * DH;
  const int nq = min(64, a.e - q0);
  load_rows<DH, 64>(Qs, Qg, ldq, nq);
  const float c2 = a.scale * kL2E;
  float m[4], l[4], o[4][NC][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int k = 0; k < 4; ++k) o[i][c][k] = 0.f;
  }
  const int qlast = q0 + nq - 1;
  const int kfirst = a.seq_lo ? (a.seq_lo[q0] & ~63) : 0;
  for (int k0 = kfirst; k0 <= qlast; k0 += 64) {
    __syncthreads();  // the previous tile's readers are done
    load_rows<DH, 64>(Ks, Kg + (int64_t)k0 * ldk, ldk, a.T - k0);
    load_rows<DH, 64>(Vs, Vg + (int64_t)k0 * ldk, ldk, a.T - k0);
    __syncthreads();
    float s[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) s[i][j] = 0.f;
    for (int kk = 0; kk < DH; kk += 4) {
      float4 qv[4], kvv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) qv[i] = *reinterpret_cast<const float4*>(Qs + (ty + 16 * i) * P + kk);
#pragma unroll
      for (int j = 0; j < 4; ++j) kvv[j] = *reinterpret_cast<const float4*>(Ks + (tx + 16 * j) * P + kk);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) s[i][j] += dot4(qv[i], kvv[j]);
    }
    float alpha[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int qi = q0 + ty + 16 * i;
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kj = k0 + tx + 16 * j;
        s[i][j] = (qi <= qlast && visible(a, qi, kj)) ? s[i][j] * c2 : -INFINITY;
        mx = fmaxf(mx, s[i][j]);
      }
      mx = row16_max(mx);
      const float mn = fmaxf(m[i], mx);
      // a row none of whose keys is visible yet keeps alpha = 1, p = 0
      alpha[i] = mn == -INFINITY ? 1.f : exp2f(m[i] - mn);
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = mn == -INFINITY ? 0.f : exp2f(s[i][j] - mn);
        Ps[ty + 16 * i][tx + 16 * j] = p;
        ps += p;
      }
      l[i] = l[i] * alpha[i] + row16_sum(ps);
      m[i] = mn;
    }
    __syncthreads();
    // O[q, dh] = alpha O + P V; columns tx*4 + 64 c
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int k = 0; k < 4; ++k) o[i][c][k] *= alpha[i];
    for (int kk = 0; kk < 64; ++kk) {
      float4 vv[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) vv[c] = *reinterpret_cast<const float4*>(Vs + kk * P + tx * 4 + 64 * c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = Ps[ty + 16 * i][kk];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          o[i][c][0] += p * vv[c].x;
          o[i][c][1] += p * vv[c].y;
          o[i][c][2] += p * vv[c].z;
          o[i][c][3] += p * vv[c].w;
        }
      }
    }
  }
  float* Og = a.O ? reinterpret_cast<float*>(a.O) + (int64_t)b * a.q_bs + (int64_t)(q0 - a.qoff) * ldq + (int64_t)h * DH : nullptr;
  const float* dOg = a.dO ? reinterpret_cast<const float*>(a.dO) + (int64_t)b * a.q_bs + (int64_t)(q0 - a.qoff) * ldq + (int64_t)h * DH : nullptr;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty + 16 * i;
    const bool ok = r < nq;
    const float inv = l[i] > 0.f ? 1.f / l[i] : 0.f;
    float dsum = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float4 ov = make_float4(o[i][c][0] * inv, o[i][c][1] * inv, o[i][c][2] * inv, o[i][c][3] * inv);
      const int col = tx * 4 + 64 * c;
      if (ok && Og) *reinterpret_cast<float4*>(Og + (int64_t)r * ldq + col) = ov;
      if (ok && dOg) dsum += dot4(ov, *reinterpret_cast<const float4*>(dOg + (int64_t)r * ldq + col));
    }
    dsum = row16_sum(dsum);
    if (ok && tx == 0) {
      const int t = q0 + r;
      a.lse[(int64_t)b * a.lse_sb + (int64_t)h * a.lse_sh + (int64_t)(t - a.s) * a.lse_st] = m[i] + log2f(l[i]);
      if (dOg) a.delta[(int64_t)b * a.dl_sb + (int64_t)h * a.dl_sh + (int64_t)(t - a.s) * a.dl_st] = dsum;
    }
  }
}

// Delta = rowsum(dO O) from a given fp32 O; optionally copies the caller's
// natural-log LSE ([B, T, Hq]) into the statistics layout in base 2.  One
// wave per (row, head).
template <int DH>
__global__ __launch_bounds__(256) void attn_f32_delta_kernel(AttnArgs a, const float* __restrict__ O,
                                                             const float* __restrict__ lse_src,
                                                             int64_t lsb, int64_t lst) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t idx = (int64_t)blockIdx.x * 4 + wave;
  const int Tc = a.e - a.s;
  if (idx >= (int64_t)Tc * a.Hq) return;
  const int b = blockIdx.y;
  const int h = (int)(idx % a.Hq);
  const int t = a.s + (int)(idx / a.Hq);
  const int64_t off = (int64_t)b * a.q_bs + (int64_t)(t - a.qoff) * a.ldq + (int64_t)h * DH;
  const float* dO = reinterpret_cast<const float*>(a.dO);
  float s = 0.f;
  for (int d = lane; d < DH; d += 64) s += dO[off + d] * O[off + d];
  s = wave_sum(s);
  if (lane == 0) {
    a.delta[(int64_t)b * a.dl_sb + (int64_t)h * a.dl_sh + (int64_t)(t - a.s) * a.dl_st] = s;
    if (lse_src)
      a.lse[(int64_t)b * a.lse_sb + (int64_t)h * a.lse_sh + (int64_t)(t - a.s) * a.lse_st] =
          lse_src[(int64_t)b * lsb + (int64_t)t * lst + h] * kL2E;
  }
}

// ---------------------------------------------------------------------------
// dK, dV: block = 64 keys of one kv head; the queries that see them, 32 at a
// time, for each of the G query heads of the group.
// ---------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(256) void attn_f32_dkdv_kernel(AttnArgs a) {
  constexpr int P = DH + 4, NC = DH / 64;
  __shared__ __attribute__((aligned(16))) float Ks[64 * P];
  __shared__ __attribute__((aligned(16))) float Vs[64 * P];
  __shared__ __attribute__((aligned(16))) float Qs[32 * P];
  __shared__ __attribute__((aligned(16))) float Os[32 * P];  // dO
  __shared__ float Ps[32][68], Ss[32][68];
  __shared__ float Ls[32], Ds[32];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int kv = blockIdx.y, b = blockIdx.z;
  const int k0 = blockIdx.x * 64;
  const int64_t ldq = a.ldq, ldk = (int64_t)a.Hkv * DH;
  const float* Kg = reinterpret_cast<const float*>(a.K) + (int64_t)b * a.T * ldk + (int64_t)kv * DH;
  const float* Vg = reinterpret_cast<const float*>(a.V) + (int64_t)b * a.T * ldk + (int64_t)kv * DH;
  const int nk = min(64, a.T - k0);
  // queries that see some key of the block: [max(s, k0), qend), qend the
  // end of the chunk or, packed, of the last key's sequence
  const int qbeg = max(a.s, k0);
  const int qend = a.seq_hi ? min(a.e, a.seq_hi[k0 + nk - 1]) : a.e;
  float dk[4][NC][4], dv[4][NC][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int k = 0; k < 4; ++k) dk[i][c][k] = dv[i][c][k] = 0.f;
  if (qbeg < qend) {
    load_rows<DH, 64>(Ks, Kg + (int64_t)k0 * ldk, ldk, nk);
    load_rows<DH, 64>(Vs, Vg + (int64_t)k0 * ldk, ldk, nk);
    const float c2 = a.scale * kL2E;
    for (int g = 0; g < a.G; ++g) {
      const int h = kv * a.G + g;
      for (int q0 = qbeg; q0 < qend; q0 += 32) {
        const int nq = min(32, qend - q0);
        __syncthreads();  // previous tile's readers are done
        const int64_t qo = (int64_t)b * a.q_bs + (int64_t)(q0 - a.qoff) * ldq + (int64_t)h * DH;
        load_rows<DH, 32>(Qs, reinterpret_cast<const float*>(a.Q) + qo, ldq, nq);
        load_rows<DH, 32>(Os, reinterpret_cast<const float*>(a.dO) + qo, ldq, nq);
        if (tid < 32) {
          const int t = q0 + tid;
          const bool ok = tid < nq;
          Ls[tid] = ok ? a.lse[(int64_t)b * a.lse_sb + (int64_t)h * a.lse_sh + (int64_t)(t - a.s) * a.lse_st] : 0.f;
          Ds[tid] = ok ? a.delta[(int64_t)b * a.dl_sb + (int64_t)h * a.dl_sh + (int64_t)(t - a.s) * a.dl_st] : 0.f;
        }
        __syncthreads();
        // S = Q K^T and dP = dO V^T, rows ty, ty + 16; columns tx + 16 j
        float s[2][4], dp[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) s[i][j] = dp[i][j] = 0.f;
        for (int kk = 0; kk < DH; kk += 4) {
          float4 qv[2], ov[2], kvv[4], vvv[4];
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            qv[i] = *reinterpret_cast<const float4*>(Qs + (ty + 16 * i) * P + kk);
            ov[i] = *reinterpret_cast<const float4*>(Os + (ty + 16 * i) * P + kk);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            kvv[j] = *reinterpret_cast<const float4*>(Ks + (tx + 16 * j) * P + kk);
            vvv[j] = *reinterpret_cast<const float4*>(Vs + (tx + 16 * j) * P + kk);
          }
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              s[i][j] += dot4(qv[i], kvv[j]);
              dp[i][j] += dot4(ov[i], vvv[j]);
            }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = ty + 16 * i, qi = q0 + r;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int cj = tx + 16 * j, kj = k0 + cj;
            const bool on = r < nq && cj < nk && visible(a, qi, kj);
            const float p = on ? exp2f(s[i][j] * c2 - Ls[r]) : 0.f;
            Ps[r][cj] = p;
            Ss[r][cj] = p * (dp[i][j] - Ds[r]);
          }
        }
        __syncthreads();
        // dV[key, dh] += P^T dO; dK[key, dh] += dS^T Q: keys ty + 16 i,
        // columns tx*4 + 64 c
        for (int qq = 0; qq < 32; ++qq) {
          float4 ov[NC], qv[NC];
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            ov[c] = *reinterpret_cast<const float4*>(Os + qq * P + tx * 4 + 64 * c);
            qv[c] = *reinterpret_cast<const float4*>(Qs + qq * P + tx * 4 + 64 * c);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = Ps[qq][ty + 16 * i], d = Ss[qq][ty + 16 * i];
#pragma unroll
            for (int c = 0; c < NC; ++c) {
              dv[i][c][0] += p * ov[c].x; dv[i][c][1] += p * ov[c].y;
              dv[i][c][2] += p * ov[c].z; dv[i][c][3] += p * ov[c].w;
              dk[i][c][0] += d * qv[c].x; dk[i][c][1] += d * qv[c].y;
              dk[i][c][2] += d * qv[c].z; dk[i][c][3] += d * qv[c].w;
            }
          }
        }
      }
    }
  }
  if (qbeg >= qend && a.beta) return;  // nothing to add
  float* dKg = a.dK + (int64_t)b * a.T * ldk + (int64_t)kv * DH;
  float* dVg = a.dV + (int64_t)b * a.T * ldk + (int64_t)kv * DH;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = k0 + ty + 16 * i;
    if (key >= a.T) continue;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int64_t off = (int64_t)key * ldk + tx * 4 + 64 * c;
      float4 nk4 = make_float4(a.scale * dk[i][c][0], a.scale * dk[i][c][1], a.scale * dk[i][c][2], a.scale * dk[i][c][3]);
      float4 nv4 = make_float4(dv[i][c][0], dv[i][c][1], dv[i][c][2], dv[i][c][3]);
      if (a.beta) {
        const float4 ok = *reinterpret_cast<const float4*>(dKg + off);
        const float4 ov = *reinterpret_cast<const float4*>(dVg + off);
        nk4 = make_float4(nk4.x + ok.x, nk4.y + ok.y, nk4.z + ok.z, nk4.w + ok.w);
        nv4 = make_float4(nv4.x + ov.x, nv4.y + ov.y, nv4.z + ov.z, nv4.w + ov.w);
      }
      *reinterpret_cast<float4*>(dKg + off) = nk4;
      *reinterpret_cast<float4*>(dVg + off) = nv4;
    }
  }
}

// ---------------------------------------------------------------------------
// dQ: block = 32 queries of one head, key tiles of 64 up to the diagonal.
// ---------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(256) void attn_f32_dq_kernel(AttnArgs a) {
  constexpr int P = DH + 4, NC = DH / 64;
  __shared__ __attribute__((aligned(16))) float Qs[32 * P];
  __shared__ __attribute__((aligned(16))) float Os[32 * P];  // dO
  __shared__ __attribute__((aligned(16))) float Ks[64 * P];
  __shared__ __attribute__((aligned(16))) float Vs[64 * P];
  __shared__ float Ss[32][68];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int h = blockIdx.y, b = blockIdx.z, kv = h / a.G;
  const int q0 = a.s + blockIdx.x * 32;
  const int nq = min(32, a.e - q0);
  const int64_t ldq = a.ldq, ldk = (int64_t)a.Hkv * DH;
  const int64_t qo = (int64_t)b * a.q_bs + (int64_t)(q0 - a.qoff) * ldq + (int64_t)h * DH;
  const float* Kg = reinterpret_cast<const float*>(a.K) + (int64_t)b * a.T * ldk + (int64_t)kv * DH;
  const float* Vg = reinterpret_cast<const float*>(a.V) + (int64_t)b * a.T * ldk + (int64_t)kv * DH;
  load_rows<DH, 32>(Qs, reinterpret_cast<const float*>(a.Q) + qo, ldq, nq);
  load_rows<DH, 32>(Os, reinterpret_cast<const float*>(a.dO) + qo, ldq, nq);
  float L[2], Dl[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = ty + 16 * i, t = q0 + r;
    const bool ok = r < nq;
    L[i] = ok ? a.lse[(int64_t)b * a.lse_sb + (int64_t)h * a.lse_sh + (int64_t)(t - a.s) * a.lse_st] : 0.f;
    Dl[i] = ok ? a.delta[(int64_t)b * a.dl_sb + (int64_t)h * a.dl_sh + (int64_t)(t - a.s) * a.dl_st] : 0.f;
  }
  const float c2 = a.scale * kL2E;
  float dq[2][NC][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int k = 0; k < 4; ++k) dq[i][c][k] = 0.f;
  const int qlast = q0 + nq - 1;
  const int kfirst = a.seq_lo ? (a.seq_lo[q0] & ~63) : 0;
  for (int k0 = kfirst; k0 <= qlast; k0 += 64) {
    __syncthreads();
    load_rows<DH, 64>(Ks, Kg + (int64_t)k0 * ldk, ldk, a.T - k0);
    load_rows<DH, 64>(Vs, Vg + (int64_t)k0 * ldk, ldk, a.T - k0);
    __syncthreads();
    float s[2][4], dp[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) s[i][j] = dp[i][j] = 0.f;
    for (int kk = 0; kk < DH; kk += 4) {
      float4 qv[2], ov[2], kvv[4], vvv[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        qv[i] = *reinterpret_cast<const float4*>(Qs + (ty + 16 * i) * P + kk);
        ov[i] = *reinterpret_cast<const float4*>(Os + (ty + 16 * i) * P + kk);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kvv[j] = *reinterpret_cast<const float4*>(Ks + (tx + 16 * j) * P + kk);
        vvv[j] = *reinterpret_cast<const float4*>(Vs + (tx + 16 * j) * P + kk);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s[i][j] += dot4(qv[i], kvv[j]);
          dp[i][j] += dot4(ov[i], vvv[j]);
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = ty + 16 * i, qi = q0 + r;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kj = k0 + tx + 16 * j;
        const bool on = r < nq && kj < a.T && visible(a, qi, kj);
        const float p = on ? exp2f(s[i][j] * c2 - L[i]) : 0.f;
        Ss[r][tx + 16 * j] = p * (dp[i][j] - Dl[i]);
      }
    }
    __syncthreads();
    // dQ[q, dh] += dS K; rows ty + 16 i, columns tx*4 + 64 c
    for (int kk = 0; kk < 64; ++kk) {
      float4 kvv[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) kvv[c] = *reinterpret_cast<const float4*>(Ks + kk * P + tx * 4 + 64 * c);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float d = Ss[ty + 16 * i][kk];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          dq[i][c][0] += d * kvv[c].x; dq[i][c][1] += d * kvv[c].y;
          dq[i][c][2] += d * kvv[c].z; dq[i][c][3] += d * kvv[c].w;
        }
      }
    }
  }
  float* dQg = reinterpret_cast<float*>(a.dQ) + (int64_t)b * a.q_bs / ldq * a.lddq + (int64_t)h * DH;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = ty + 16 * i;
    if (r >= nq) continue;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      *reinterpret_cast<float4*>(dQg + (int64_t)(q0 + r - a.qoff) * a.lddq + tx * 4 + 64 * c) =
          make_float4(a.scale * dq[i][c][0], a.scale * dq[i][c][1], a.scale * dq[i][c][2], a.scale * dq[i][c][3]);
  }
}

double pairs_of(int s, int e) { return 0.5 * ((double)e * (e + 1) - (double)s * (s + 1)); }

}  // namespace

sbp_status attn_fwd_f32(const AttnArgs& a, int dh, int B, hipStream_t st) {
  const int Tc = a.e - a.s;
  dim3 grid((unsigned)cdiv(Tc, 64), (unsigned)a.Hq, (unsigned)B);
  ProfScope prof("attn_f32_fwd", st, 4.0 * dh * a.Hq * B * pairs_of(a.s, a.e), 0.0);
  if (dh == 128)
    hipLaunchKernelGGL(attn_f32_fwd_kernel<128>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(attn_f32_fwd_kernel<64>, grid, dim3(256), 0, st, a);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

sbp_status attn_delta_f32(const AttnArgs& a, const void* O, const float* lse_src, int64_t lsb,
                          int64_t lst, int dh, int B, hipStream_t st) {
  const int64_t rows = (int64_t)(a.e - a.s) * a.Hq;
  dim3 grid((unsigned)cdiv(rows, 4), (unsigned)B);
  ProfScope prof("attn_f32_delta", st, 0.0, 8.0 * rows * B * dh);
  if (dh == 128)
    hipLaunchKernelGGL(attn_f32_delta_kernel<128>, grid, dim3(256), 0, st, a, (const float*)O, lse_src, lsb, lst);
  else
    hipLaunchKernelGGL(attn_f32_delta_kernel<64>, grid, dim3(256), 0, st, a, (const float*)O, lse_src, lsb, lst);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

sbp_status attn_bwd_chunk_f32(const AttnArgs& a, int dh, int B, hipStream_t st) {
  const double pairs = pairs_of(a.s, a.e) * a.Hq * B;
  {
    dim3 grid((unsigned)cdiv(a.e, 64), (unsigned)a.Hkv, (unsigned)B);
    ProfScope prof("attn_f32_dkdv", st, 8.0 * dh * pairs, 0.0);
    if (dh == 128)
      hipLaunchKernelGGL(attn_f32_dkdv_kernel<128>, grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(attn_f32_dkdv_kernel<64>, grid, dim3(256), 0, st, a);
    SBP_LAUNCH_CHECK();
  }
  {
    dim3 grid((unsigned)cdiv(a.e - a.s, 32), (unsigned)a.Hq, (unsigned)B);
    ProfScope prof("attn_f32_dq", st, 6.0 * dh * pairs, 0.0);
    if (dh == 128)
      hipLaunchKernelGGL(attn_f32_dq_kernel<128>, grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(attn_f32_dq_kernel<64>, grid, dim3(256), 0, st, a);
    SBP_LAUNCH_CHECK();
  }
  return SBP_OK;
}

}  // namespace sbp
