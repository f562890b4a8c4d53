// NT GEMM on CDNA4 matrix cores:  C[M,N] (op)= alpha * A[M,K] . B[N,K]^T
//
// Every chunk GEMM of the StreamBP path is put in this one form (both
// operands K-contiguous), so one kernel serves them all:
//   logits      Z_c   = H_c  . W^T      A = H_c  [T_c, d],  B = W   [V, d]
//   input grad  dH_c  = dZ_c . W        A = dZ_c [T_c, V],  B = W^T [d, V]
//   weight grad dW   += dZ_c^T . H_c    A = dZ_c^T [V, T_c], B = H_c^T [d, T_c]
// (the transposed operands are written by the producing kernels or by a
// transpose kernel; see transpose.hip / ce.hip).
//
// Tiling: a 256-thread block (4 waves of 64) owns a BM x BN output tile and
// walks K in steps of 128 bytes per row (64 bf16 or 32 fp32).  Global loads
// are 16-byte vectors staged through registers into a double-buffered LDS
// tile; LDS rows are 8 x 16-byte chunks with chunk c of row r stored at
// c ^ (r & 7) so the fragment reads of 8 consecutive rows hit distinct banks.
// Each wave computes a (BM/WGM) x (BN/WGN) sub-tile from 16x16 MFMA blocks:
// bf16 uses v_mfma_f32_16x16x32_bf16 (one 16-byte fragment per lane per
// instruction), fp32 uses v_mfma_f32_16x16x4_f32 four times per fragment.
// The lane that holds k-chunk g of an A row also holds k-chunk g of the B
// column, so the k order inside an instruction never matters.
// Output layout of a 16x16 block: lane l, element i -> row 4*(l/16)+i,
// column l%16.
//
// Block -> tile mapping is XCD-aware: consecutive block ids go round-robin
// to the 8 XCDs, so block b is given the (b/8)-th tile of a contiguous range
// owned by XCD b%8.  Blocks that share an L2 then share operand panels, and
// with split-K the splits fall on whole XCDs.
#include "common.h"
#include "kernels.h"

namespace sbp {

template <typename T> struct Mfma;
template <> struct Mfma<bf16_t> {
  static constexpr int EPC = 8;  // elements per 16-byte chunk
  __device__ __forceinline__ static void mma(f32x4_t& c, const uint4& a, const uint4& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  static constexpr int EPC = 4;
  __device__ __forceinline__ static void mma(f32x4_t& c, const uint4& a, const uint4& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  }
};

template <typename T, int BM, int BN, int WGM, int WGN, int EPI>
__global__ __launch_bounds__(256) void gemm_nt_kernel(GemmParams p) {
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int EPC = Mfma<T>::EPC;
  constexpr int BK = 8 * EPC;
  constexpr int AP = BM / 32, BP = BN / 32;
  static_assert(WGM * WGN == 4, "4 waves per block");
  static_assert(BM % 32 == 0 && BN % 32 == 0 && WTM % 16 == 0 && WTN % 16 == 0, "tile");
  __shared__ uint4 lds[2][(BM + BN) * 8];

  if (p.active && *p.active == 0) return;

  const int ntile = p.tiles_m * p.tiles_n;
  const int total = ntile * p.k_split;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, idx = bid >> 3;
  const int base = total >> 3, rem = total & 7;
  const int lin = xcd * base + (xcd < rem ? xcd : rem) + idx;
  const int split = lin / ntile;
  const int t = lin - split * ntile;
  int tm, tn;
  if (p.m_fastest) {
    tm = t % p.tiles_m;
    tn = t / p.tiles_m;
  } else {
    tn = t % p.tiles_n;
    tm = t / p.tiles_n;
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int kb = split * p.k_per_split;
  const int ke = min(p.K, kb + p.k_per_split);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int lr = tid >> 3, lc = tid & 7;
  const T* __restrict__ A = reinterpret_cast<const T*>(p.A);
  const T* __restrict__ B = reinterpret_cast<const T*>(p.B);

  uint4 ra[AP], rb[BP];
  auto gload = [&](int k0) {
    const int kk = k0 + lc * EPC;
#pragma unroll
    for (int i = 0; i < AP; ++i) {
      const int row = m0 + lr + 32 * i;
      if (row < p.M && kk < ke)
        ra[i] = *reinterpret_cast<const uint4*>(A + (int64_t)row * p.lda + kk);
      else
        ra[i] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < BP; ++i) {
      const int row = n0 + lr + 32 * i;
      if (row < p.N && kk < ke)
        rb[i] = *reinterpret_cast<const uint4*>(B + (int64_t)row * p.ldb + kk);
      else
        rb[i] = make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int s) {
#pragma unroll
    for (int i = 0; i < AP; ++i) {
      const int r = lr + 32 * i;
      lds[s][r * 8 + (lc ^ (r & 7))] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < BP; ++i) {
      const int r = lr + 32 * i;
      lds[s][(BM + r) * 8 + (lc ^ (r & 7))] = rb[i];
    }
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = ke > kb ? (ke - kb + BK - 1) / BK : 0;
  if (nk > 0) {
    gload(kb);
    lstore(0);
  }
  __syncthreads();
  for (int it = 0; it < nk; ++it) {
    const int s = it & 1;
    if (it + 1 < nk) gload(kb + (it + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ch = ks * 4 + (lane >> 4);
      uint4 af[FM], bfr[FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int r = wm * WTM + fm * 16 + (lane & 15);
        af[fm] = lds[s][r * 8 + (ch ^ (r & 7))];
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int r = wn * WTN + fn * 16 + (lane & 15);
        bfr[fn] = lds[s][(BM + r) * 8 + (ch ^ (r & 7))];
      }
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) Mfma<T>::mma(acc[fm][fn], af[fm], bfr[fn]);
    }
    if (it + 1 < nk) lstore(s ^ 1);
    __syncthreads();
  }

  // ---- epilogue ----
  float beta = (float)p.beta;
  if (EPI == EPI_F32_ACC && p.beta_zero && *p.beta_zero) beta = 0.f;
  const int rbase = m0 + wm * WTM + 4 * (lane >> 4);
  const int cbase = n0 + wn * WTN + (lane & 15);
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int col = cbase + fn * 16;
      if (col >= p.N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rbase + fm * 16 + i;
        if (row >= p.M) continue;
        const float v = p.alpha * acc[fm][fn][i];
        if constexpr (EPI == EPI_F32) {
          reinterpret_cast<float*>(p.C)[(int64_t)row * p.ldc + col] = v;
        } else if constexpr (EPI == EPI_F32_ACC) {
          float* c = reinterpret_cast<float*>(p.C) + (int64_t)row * p.ldc + col;
          *c = (beta != 0.f) ? (v + beta * *c) : v;
        } else if constexpr (EPI == EPI_OUT) {
          Elem<T>::store(reinterpret_cast<T*>(p.C), (int64_t)row * p.ldc + col, v);
        } else if constexpr (EPI == EPI_OUT_RESID) {
          const float r = Elem<T>::load(reinterpret_cast<const T*>(p.R), (int64_t)row * p.ldr + col);
          Elem<T>::store(reinterpret_cast<T*>(p.C), (int64_t)row * p.ldc + col, v + r);
        } else {  // EPI_PARTIAL
          reinterpret_cast<float*>(p.C)[(int64_t)split * p.split_stride + (int64_t)row * p.ldc + col] = v;
        }
      }
    }
  }
}

template <typename T, int BM, int BN, int WGM, int WGN>
static void launch_cfg(int epi, GemmParams p, hipStream_t st) {
  p.tiles_m = (int)cdiv(p.M, BM);
  p.tiles_n = (int)cdiv(p.N, BN);
  const int grid = p.tiles_m * p.tiles_n * p.k_split;
  switch (epi) {
    case EPI_F32: hipLaunchKernelGGL((gemm_nt_kernel<T, BM, BN, WGM, WGN, EPI_F32>), dim3(grid), dim3(256), 0, st, p); break;
    case EPI_F32_ACC: hipLaunchKernelGGL((gemm_nt_kernel<T, BM, BN, WGM, WGN, EPI_F32_ACC>), dim3(grid), dim3(256), 0, st, p); break;
    case EPI_OUT: hipLaunchKernelGGL((gemm_nt_kernel<T, BM, BN, WGM, WGN, EPI_OUT>), dim3(grid), dim3(256), 0, st, p); break;
    case EPI_OUT_RESID: hipLaunchKernelGGL((gemm_nt_kernel<T, BM, BN, WGM, WGN, EPI_OUT_RESID>), dim3(grid), dim3(256), 0, st, p); break;
    default: hipLaunchKernelGGL((gemm_nt_kernel<T, BM, BN, WGM, WGN, EPI_PARTIAL>), dim3(grid), dim3(256), 0, st, p); break;
  }
}

int gemm_k_granule(int dtype) { return dtype == SBP_BF16 ? 64 : 32; }

sbp_status gemm_nt(int dtype, int epi, GemmParams p, int tile, hipStream_t st, const char* name) {
  if (p.M <= 0 || p.N <= 0) return SBP_OK;
  if (p.k_split < 1) p.k_split = 1;
  const int gran = gemm_k_granule(dtype);
  if (p.k_per_split <= 0) p.k_per_split = (int)round_up(cdiv(p.K, p.k_split), gran);
  const double flops = 2.0 * p.M * p.N * (double)p.K;
  const size_t esz = dtype == SBP_BF16 ? 2 : 4;
  const double bytes = ((double)p.M * p.K + (double)p.N * p.K) * esz +
                       (double)p.M * p.N * (epi == EPI_F32_ACC ? 8.0 : epi == EPI_OUT || epi == EPI_OUT_RESID ? (double)esz : 4.0 * p.k_split);
  ProfScope prof(name, st, flops, bytes);
  if (dtype == SBP_BF16) {
    if (tile == GEMM_TILE_256)
      launch_cfg<bf16_t, 256, 256, 2, 2>(epi, p, st);
    else
      launch_cfg<bf16_t, 128, 128, 2, 2>(epi, p, st);
  } else {
    launch_cfg<float, 128, 128, 2, 2>(epi, p, st);
  }
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

}  // namespace sbp
