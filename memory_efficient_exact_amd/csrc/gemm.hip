// GEMM on CDNA4 matrix cores:  C[M,N] (op)= alpha * A[M,K] . B[N,K]^T, where
// the bf16 kernel also takes both operands stored K-major (A as [K, M], B as
// [K, N]), so that weight gradients, which contract over tokens, read the
// activations in place:
//   logits      Z_c   = H_c  . W^T      A = H_c  [T_c, d],  B = W   [V, d]
//   input grad  dH_c  = dZ_c . W        A = dZ_c [T_c, V],  B = W^T [d, V]
//   weight grad dW   += dZ_g^T . H_g    A = dZ_g [K_g, V],  B = H_g [K_g, d], both K-major
// (W^T is formed once per call; the fp32 path also forms dZ^T and H^T; see
// misc.hip / ce.hip).
//
// Two kernels:
//  * gemm_nt_bf16_ring_kernel (bf16, the default): a 256 x 256 tile, 4
//    waves of 128 x 128 as 4 x 4 v_mfma_f32_32x32x16_bf16 blocks, operands
//    fed global -> LDS by DMA through two 64 KB stages (its section below
//    has the details);
//  * gemm_nt_kernel (fp32, and bf16 the ring cannot take): a 128 x 128 tile, 4 waves
//    of 64 x 64 as 16x16 MFMA blocks (v_mfma_f32_16x16x32_bf16, or
//    v_mfma_f32_16x16x4_f32 four times per fragment), 16-byte global loads
//    staged through registers into a double-buffered LDS tile whose rows are
//    8 x 16-byte chunks, chunk c of row r at c ^ (r & 7).  The lane that
//    holds k-chunk g of an A row also holds k-chunk g of the B column, so the
//    k order inside an instruction never matters.  Output layout of a 16x16
//    block: lane l, element i -> row 4*(l/16)+i, column l%16.
//
// Block -> tile mapping is XCD-aware: consecutive block ids go round-robin
// to the 8 XCDs, so block b is given the (b/8)-th tile of a contiguous range
// owned by XCD b%8.  Blocks that share an L2 then share operand panels, and
// with split-K the splits fall on whole XCDs.
#include "common.h"
#include <type_traits>
#include "kernels.h"

namespace sbp {

// Native vectors for the nontemporal loads and stores of the epilogues
// (the builtins take no struct types).
typedef float ntf4_t __attribute__((ext_vector_type(4)));
typedef unsigned int ntu2_t __attribute__((ext_vector_type(2)));

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

#define SBP_AS1 __attribute__((address_space(1)))
#define SBP_AS3 __attribute__((address_space(3)))

__device__ __forceinline__ void tile_coords(const GemmParams& p, int& tm, int& tn, int& split) {
  const int ntile = p.tiles_m * p.tiles_n;
  const int total = ntile * p.k_split;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, idx = bid >> 3;
  const int base = total >> 3, rem = total & 7;
  const int lin = xcd * base + (xcd < rem ? xcd : rem) + idx;
  split = lin / ntile;
  const int t = lin - split * ntile;
  // Grouped order: 4 tile rows at a time, m fastest inside the group, so an
  // XCD's ~32 concurrent blocks cover about 4 x 8 tiles and share their A
  // and B panels through its L2 (operand panels of long-K products are
  // megabytes, so reuse has to be concurrent rather than over time).  Same-box
  // A/B over groups of 1, 2, 4, 8 and 16 rows: 4 is fastest on the LM-head,
  // layer and model workloads (1-3% over 8; 1 and 16 are the slowest).
  constexpr int GM = 4;
  const int g = t / (GM * p.tiles_n);
  const int rows = min(GM, p.tiles_m - g * GM);
  const int tl = t - g * GM * p.tiles_n;
  tm = g * GM + tl % rows;
  tn = tl / rows;
}

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// two fp32 -> packed fp16 (round to nearest even)
__device__ __forceinline__ uint32_t pk_f16(float lo, float hi) {
  const f16x2_t h = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, h);
}

// ---------------------------------------------------------------------------
// Pipelined variant (the default for bf16): the same 256 x 256 tile and
// 32x32x16 MFMA with two 64-wide K stages (64 KB each) in two distinct LDS
// arrays.  Every DMA instruction fetches 8 rows x 128 bytes -- whole cache
// lines; fetching half lines (16 rows x 64 bytes) was measured on the box to
// move ~40% less data per second.  Rows are 8 x 16-byte chunks, chunk c of
// row r at c ^ ((r >> 1) & 7): gfx950's LDS serves 256 bytes (64 banks) per
// clock, 16 lanes of a 16-byte fragment read, and rows r .. r+15 then fill
// the 16 chunk positions of the two 128-byte halves of a bank line.  Per
// stage t (4 k16 steps):
//   read step 1 | MFMAs step 0 | read step 2 | MFMAs step 1 | read step 3 |
//   MFMAs step 2 | wait for stage t+1, bare barrier | fetch stage t+2 into
//   stage t's buffer | read step 0 of stage t+1 | MFMAs step 3
// so fragment reads always run under 16 MFMAs, and the barrier only waits
// for stage t+1 (issued one stage earlier), never for t+2.
// ---------------------------------------------------------------------------
struct RingFrag {
  uint4 a[4], b[4];
};

// LDS DMA as inline assembly (global_load_lds: lane l's bytes land at M0 +
// size * l).  Issued this way the compiler neither tracks the LDS writes nor
// adds waits for them -- its alias tracking cannot tell the transposed LDS
// reads apart from in-flight fills and would drain every DMA before them --
// so the kernel orders them itself with explicit waits and barriers.  The
// s_nop is the one wait state gfx9 needs between an M0 write and an LDS DMA.
// 16 zero bytes: the source of every DMA lane outside the operands
__device__ uint4 g_ring_zero;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)p;  // low half of a generic LDS address
}
__device__ __forceinline__ void dma_x4(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g),
               "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}
// The same fill with a uniform 64-bit base and a per-lane 32-bit byte offset
// (scalar-base addressing): the per-instruction address step is then a
// scalar add, with no vector instructions between the DMAs and the MFMAs.
__device__ __forceinline__ void dma_x4_s(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base),
               "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}
__device__ __forceinline__ void dma_x1(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g),
               "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// A K-major operand ([K, P] in memory, P contiguous) is staged as four
// 8 KB segments, segment s holding p in [64 s, 64 s + 64) of the stage's 64
// k-rows: 128 bytes per k-row, 16-byte chunk c of k-row r at c ^ 4 ((r >> 1)
// & 1).  One DMA instruction then fetches 8 k-rows x 128 bytes, the shape of
// a row-major fetch (contiguous 512-byte runs per instruction were measured
// slower).  Fragments (lane l: p = l % 32 of the fragment, k = 8 (l/32) ..
// + 8 of the k16 step) are read transposed with two ds_read_b64_tr_b16:
// within each 16-lane group, lane j fetches 4 p of k-row 8 (l/32) + (j >> 2)
// (+ 4 for the second read) and receives one p of 4 consecutive k-rows, so
// the k order matches a row-major fragment's.  A 32-lane half reads 4 k-rows
// x 64 bytes, which the XOR spreads over the 4 64-byte quarters of a 256-byte
// bank line (conflict-free).
// Per-lane part of a transposed fragment read: k-row 8 (l/32) + q with q =
// (l >> 2) & 3, chunk x = 2 ((l >> 4) & 1) + ((l & 3) >> 1), 8-byte half l & 1.
__device__ __forceinline__ int kmaj_lane_off(int lane) {
  const int q = (lane >> 2) & 3, x = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  return (8 * (lane >> 5) + q) * 128 + x * 16 + 8 * (lane & 1);
}
// Fragment i of the sub-tile starting at p_base (a multiple of 128) of the
// K-major region at byte offset rbyte of L, k16 step ks.
__device__ __forceinline__ uint4 kmaj_frag(const uint4* L, int rbyte, int lo, int p_base, int i, int ks,
                                          int lane) {
  const int q = (lane >> 2) & 3;
  const SBP_AS3 char* b = (const SBP_AS3 char*)L + rbyte + lo + ks * 16 * 128 +
                          (p_base / 64 + (i >> 1)) * 8192 + 64 * ((i & 1) ^ (q >> 1));
  i16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SBP_AS3 i16x4_t*)b);
  i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SBP_AS3 i16x4_t*)(b + 4 * 128));
  uint4 u;
  u.x = (uint32_t)(uint16_t)v0[0] | ((uint32_t)(uint16_t)v0[1] << 16);
  u.y = (uint32_t)(uint16_t)v0[2] | ((uint32_t)(uint16_t)v0[3] << 16);
  u.z = (uint32_t)(uint16_t)v1[0] | ((uint32_t)(uint16_t)v1[1] << 16);
  u.w = (uint32_t)(uint16_t)v1[2] | ((uint32_t)(uint16_t)v1[3] << 16);
  return u;
}

// Fragments of k16 step ks (0..3) of a 64-wide stage in LDS tile L (A in
// bytes [0, 32K), B in [32K, 64K)).
template <bool AKM, bool BKM>
__device__ __forceinline__ void ring_load(const uint4* __restrict__ L, int ks, int wm, int wn, int lane,
                                          int klo, RingFrag& f) {
  constexpr int BM = 256, WT = 128;
  const int ch = ks * 2 + (lane >> 5);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (AKM) {
      f.a[i] = kmaj_frag(L, 0, klo, wm * WT, i, ks, lane);
    } else {
      const int r = wm * WT + i * 32 + (lane & 31);
      f.a[i] = L[r * 8 + (ch ^ ((r >> 1) & 7))];
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (BKM) {
      f.b[i] = kmaj_frag(L, BM * 128, klo, wn * WT, i, ks, lane);
    } else {
      const int r = BM + wn * WT + i * 32 + (lane & 31);
      f.b[i] = L[r * 8 + (ch ^ ((r >> 1) & 7))];
    }
  }
}

// Reads of the next fragments spread over the first MFMAs of a group (two
// reads per MFMA), for the K-major tiles' 16 transposed reads per k16 step.
template <int NR>
__device__ __forceinline__ void interleave_reads() {
#pragma unroll
  for (int i = 0; i < NR / 2; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS reads
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 16 - NR / 2, 0);
}

__device__ __forceinline__ void ring_mma(const RingFrag& f, f32x16_t (&acc)[4][4]) {
#pragma unroll
  for (int fm = 0; fm < 4; ++fm)
#pragma unroll
    for (int fn = 0; fn < 4; ++fn)
      acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8_t, f.a[fm]), __builtin_bit_cast(bf16x8_t, f.b[fn]), acc[fm][fn],
          0, 0, 0);
}

template <int EPI, bool AKM, bool BKM>
__global__ __launch_bounds__(256, 1) void gemm_nt_bf16_ring_kernel(GemmParams p) {
  constexpr int BM = 256, BN = 256, BK = 64, WT = 128;
  __shared__ uint4 L0[(BM + BN) * 8];
  __shared__ uint4 L1[(BM + BN) * 8];
  __shared__ uint32_t PF[4][64];  // sink of the L2 prefetches (never read)
  __shared__ float MQ[EPI == EPI_REL16_LSE ? 4 * 64 : 1];  // quarter maxima of a 32-row block
  if (p.active && *p.active == 0) return;
  int tm, tn, split;
  tile_coords(p, tm, tn, split);
  const int m0 = tm * BM, n0 = tn * BN;
  // K runs to a multiple of 128: chunks at k >= K read zeros (so K itself
  // need only be a multiple of 8)
  const int Kpad = (p.K + 127) & ~127;
  const int kb = split * p.k_per_split;
  const int ke = min(Kpad, kb + p.k_per_split);
  const bf16_t* zero = reinterpret_cast<const bf16_t*>(&g_ring_zero);

  // B rows past b_split come from the second buffer (tile-aligned split)
  const void* Bsel = p.B;
  if (p.B2 && n0 >= p.b_split)
    Bsel = reinterpret_cast<const bf16_t*>(p.B2) - (int64_t)p.b_split * p.ldb;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  // DMA role: waves 0-1 fetch the A panel, 2-3 the B panel: 128 rows each of
  // a row-major operand, or 32 k-rows each of a K-major one
  const int opnd = wave >> 1;
  static_assert(AKM == BKM, "both operands K-major or neither");
  constexpr bool kmaj = AKM;
  const int klo = kmaj_lane_off(lane);
  const int rbase = (wave & 1) * 128;
  // row-major: instruction j fills LDS rows 256 opnd + rbase + 8j + lane / 8,
  // slot lane % 8, with logical chunk slot ^ ((row >> 1) & 7)
  const int chunk_even = (lane & 7) ^ (lane >> 4), chunk_odd = (lane & 7) ^ (4 + (lane >> 4));
  const bf16_t* X = reinterpret_cast<const bf16_t*>(opnd ? Bsel : p.A);
  const int64_t ld = opnd ? p.ldb : p.lda;
  const int lim = opnd ? p.N : p.M;
  const int r0 = (opnd ? n0 : m0) + rbase + (lane >> 3);

  // Per-lane parts of the fetch addresses.  Instruction j of a stage reads
  // row rb + ro(j), column c(j) + co(j) -- k0 goes to the row of a K-major
  // operand and to the column of a row-major one -- and zeros outside
  // [0, rlim) x [0, clim):
  //   row-major: rows r0 + 8j, column k0 + 8 (chunk slot ^ ((row >> 1) & 7)),
  //              filling the 1 KB at 32768 opnd + 16384 (wave & 1) + 1024 j;
  //   K-major:   k-rows k0 + 32 (wave & 1) + 8 (j & 3) + lane / 8 of segment
  //              s = j >> 2, p = 64 s + 8 (slot ^ 4 ((lane >> 4) & 1)),
  //              filling the 1 KB at 32768 opnd + 8192 s + 4096 (wave & 1)
  //              + 1024 (j & 3).
  const int p0 = opnd ? n0 : m0;
  const int kl = (wave & 1) * 32 + (lane >> 3);
  const int rlim = kmaj ? p.K : lim, clim = kmaj ? lim : p.K;
  const int c_km = p0 + 8 * ((lane & 7) ^ (4 * ((lane >> 4) & 1)));
  const int c_even = kmaj ? c_km : chunk_even * 8;
  const int c_odd = kmaj ? c_km : chunk_odd * 8;
  const uint32_t dst0 = (uint32_t)(opnd * 32768 + (wave & 1) * (kmaj ? 4096 : 16384));
  // Interior tiles (every row of the tile below lim, every stage below K)
  // take the scalar-base path: a uniform stage base
  // X + p0 ld + k0 (row-major) or X + k0 ld + p0 (K-major) plus per-lane byte
  // offsets that are the same for every stage; other stages the general path
  // with the zero redirect.  The 32-bit offsets need ld < 2^22.
  // (decided per wave, for the whole loop: the operand's rows of this tile
  // all below lim, and K a multiple of 128 so that no stage -- the padded
  // ones included -- reaches past K)
  const bool fast_tile = ld < (1 << 22) && p0 + 256 <= lim && p.K % 128 == 0;
  const uint32_t off_e = kmaj ? (uint32_t)((int64_t)kl * ld + (c_km - p0)) * 2u
                              : (uint32_t)((int64_t)(rbase + (lane >> 3)) * ld + c_even) * 2u;
  const uint32_t off_o = kmaj ? off_e : (uint32_t)((int64_t)(rbase + (lane >> 3)) * ld + c_odd) * 2u;
  // the stage's two base addresses (even / odd j) are computed once and
  // kept opaque, so that each instruction adds a uniform offset to one
  struct StageSrc {
    const bf16_t *e, *o;
    int rb, ce, co;
    const char* sb;  // uniform stage base (scalar-base path)
    bool fast;
  };
  auto stage_src = [&](int k0) __attribute__((always_inline)) {
    StageSrc q;
    q.fast = fast_tile;
    q.sb = reinterpret_cast<const char*>(kmaj ? X + (int64_t)k0 * ld + p0 : X + (int64_t)p0 * ld + k0);
    q.rb = kmaj ? k0 + kl : r0;
    q.ce = c_even + (kmaj ? 0 : k0);
    q.co = c_odd + (kmaj ? 0 : k0);
    const bf16_t* row = X + (int64_t)q.rb * ld;
    q.e = row + q.ce;
    q.o = row + q.co;
    asm volatile("" : "+v"(q.e), "+v"(q.o));
    return q;
  };
  // uniform byte step of instruction j from the stage base (instruction j
  // reads what the general path's src_addr(q, j) reads when all lanes are in
  // range)
  auto step_of = [&](int j) __attribute__((always_inline)) {
    return kmaj ? ((int64_t)8 * (j & 3) * ld + 64 * (j >> 2)) * 2 : (int64_t)8 * j * ld * 2;
  };
  auto src_addr = [&](const StageSrc& q, int j) __attribute__((always_inline)) {
    const int ro = kmaj ? 8 * (j & 3) : 8 * j, co = kmaj ? 64 * (j >> 2) : 0;
    const bool ok = q.rb + ro < rlim && ((j & 1) ? q.co : q.ce) + co < clim;
    const bf16_t* g = ((j & 1) ? q.o : q.e) + (int64_t)ro * ld + co;
    return ok ? g : zero;
  };
  auto dst_of = [&](int j) __attribute__((always_inline)) {
    return dst0 + (kmaj ? 8192u * (j >> 2) + 1024u * (j & 3) : 1024u * j);
  };
  // four DMAs whose addresses are all formed first (in distinct registers, so
  // that no address register is rewritten right after its load issues)
  auto issue_one = [&](uint4* L, const StageSrc& q, int j) __attribute__((always_inline)) {
    dma_x4(src_addr(q, j), lds_addr(L) + dst_of(j));
  };
  auto issue_one_s = [&](uint4* L, const StageSrc& q, int j) __attribute__((always_inline)) {
    dma_x4_s(q.sb + step_of(j), (j & 1) ? off_o : off_e, lds_addr(L) + dst_of(j));
  };
  auto issue_four = [&](uint4* L, const StageSrc& q, int j0) __attribute__((always_inline)) {
    const bf16_t* g0 = src_addr(q, j0);
    const bf16_t* g1 = src_addr(q, j0 + 1);
    const bf16_t* g2 = src_addr(q, j0 + 2);
    const bf16_t* g3 = src_addr(q, j0 + 3);
    asm volatile("" ::"v"(g0), "v"(g1), "v"(g2), "v"(g3));
    const uint32_t l = lds_addr(L);
    dma_x4(g0, l + dst_of(j0));
    dma_x4(g1, l + dst_of(j0 + 1));
    dma_x4(g2, l + dst_of(j0 + 2));
    dma_x4(g3, l + dst_of(j0 + 3));
  };
  auto issue = [&](uint4* L, int k0) __attribute__((always_inline)) {
    const StageSrc q = stage_src(k0);
#pragma unroll
    for (int j = 0; j < 16; j += 4) issue_four(L, q, j);
  };
  // L2 prefetch of the stage after the one being fetched: one 4-byte DMA per
  // row touches the row's cache line of that K slice (2 instructions per
  // wave), so that its real fetch a stage later finds the line in L2 (or
  // already on its way).  The ring thus hides two stages of memory latency
  // with two LDS buffers.
  auto prefetch = [&](int k0) __attribute__((always_inline)) {
    // row-major: rows p0 + rbase + 64h + lane at column k0; K-major: k-rows
    // k0 + 32 (wave & 1) + 16h + lane / 4, 128-byte line lane % 4 of the
    // tile's 512 bytes
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = kmaj ? min(k0 + (wave & 1) * 32 + 16 * h + (lane >> 2), p.K - 1)
                           : min(p0 + rbase + 64 * h + lane, lim - 1);
      const int col = max(0, kmaj ? min(p0 + 64 * (lane & 3), lim - 8) : min(k0, p.K - 8));
      dma_x1(X + (int64_t)row * ld + col, lds_addr(&PF[wave][0]));
    }
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};

  // nk is 0 or even.  The refill past the end re-fetches the last stage into
  // a buffer nobody reads, so every step has the same shape.  The compiler
  // does not see the DMAs (inline assembly), so every wait for them is
  // explicit (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4,
  // lgkmcnt 11:8); vmcnt retires loads in issue order.
  //
  // A stage's 16 DMA instructions per wave are issued in two halves, each
  // spread over 16 MFMAs: instructions 0-7 of stage t+2 right after the
  // barrier that frees its buffer (under the last k16 step of stage t), and
  // 8-15 under the first k16 step of stage t+1, followed by the L2 prefetch
  // of stage t+3.  The vector-memory pipe moves about 64 bytes per clock per
  // CU, so a whole stage (64 KB) under one 16-MFMA window would stall the
  // MFMA issue; two windows keep it under half busy.  The second half has
  // two k16 steps to land before the barrier that waits for it.
  const int nk = ke > kb ? (ke - kb) / BK : 0;
  RingFrag f0, f1;
  if (nk > 0) {
    issue(L0, kb);
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): stage 0 landed
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    {
      const StageSrc q1 = stage_src(kb + min(1, nk - 1) * BK);
      issue_four(L1, q1, 0);
      issue_four(L1, q1, 4);
    }
    ring_load<AKM, BKM>(L0, 0, wm, wn, lane, klo, f0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  }
  // 16 MFMAs on fragments f with 8 DMA instructions (j0 .. j0 + 7 of the
  // stage qs describes), one before every second MFMA: a DMA holds the
  // wave's in-order issue for longer than one MFMA occupies the matrix pipe,
  // so two MFMAs between DMAs keep the pipe fed
  auto mma_dma = [&](auto fast_tag, const RingFrag& f, uint4* Ldst, const StageSrc& qs, int j0)
                     __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      if (m % 2 == 0) {
        if constexpr (decltype(fast_tag)::value) issue_one_s(Ldst, qs, j0 + m / 2);
        else issue_one(Ldst, qs, j0 + m / 2);
        __builtin_amdgcn_sched_barrier(0);
      }
      acc[m >> 2][m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8_t, f.a[m >> 2]), __builtin_bit_cast(bf16x8_t, f.b[m & 3]), acc[m >> 2][m & 3], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto step = [&](auto fast_tag, const uint4* Lc, uint4* Ln, uint4* Lrefill, int t) __attribute__((always_inline)) {
    // lgkmcnt(0) after each MFMA group: the reads issued before it have long
    // landed, and saying so keeps at most 8 reads outstanding (the counter
    // cannot express waits with more than 15 in flight).
    ring_load<AKM, BKM>(Lc, 1, wm, wn, lane, klo, f1);
    __builtin_amdgcn_sched_barrier(0);
    // second half of stage t+1's fill, then the L2 prefetch of stage t+3
    mma_dma(fast_tag, f0, Ln, stage_src(kb + min(t + 1, nk - 1) * BK), 8);
    prefetch(kb + min(t + 3, nk - 1) * BK);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    ring_load<AKM, BKM>(Lc, 2, wm, wn, lane, klo, f0);
    if constexpr (!kmaj) __builtin_amdgcn_sched_barrier(0);
    ring_mma(f1, acc);
    if constexpr (kmaj) interleave_reads<16>();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    ring_load<AKM, BKM>(Lc, 3, wm, wn, lane, klo, f1);
    if constexpr (!kmaj) __builtin_amdgcn_sched_barrier(0);
    ring_mma(f0, acc);
    if constexpr (kmaj) interleave_reads<16>();
    __builtin_amdgcn_sched_barrier(0);
    // stage t+1 landed (only the 2 prefetches issued after it may still be
    // in flight), step 3 read
    __builtin_amdgcn_s_waitcnt(0x0072);  // vmcnt(2) lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // the next stage's first fragments, then the first half of stage t+2's
    // fill (into the buffer the barrier just freed) under step 3's MFMAs
    ring_load<AKM, BKM>(Ln, 0, wm, wn, lane, klo, f0);
    __builtin_amdgcn_sched_barrier(0);
    mma_dma(fast_tag, f1, Lrefill, stage_src(kb + min(t + 2, nk - 1) * BK), 0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  };
  // wave-uniform choice of the fill path for the whole loop (both loops run
  // the same barriers)
  if (fast_tile) {
    for (int it = 0; it < nk; it += 2) {
      step(std::true_type{}, L0, L1, L0, it);
      step(std::true_type{}, L1, L0, L1, it + 1);
    }
  } else {
    for (int it = 0; it < nk; it += 2) {
      step(std::false_type{}, L0, L1, L0, it);
      step(std::false_type{}, L1, L0, L1, it + 1);
    }
  }

  // Epilogue through LDS: each wave parks 32 rows x 128 columns of fp32 (16 KB)
  // in its own quarter of L0|L1, then writes row-contiguous 4-wide vectors
  // (after the trailing refill and prefetch DMAs have landed).
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  __syncthreads();
  // output tiles past a split go to that split's buffer (whole tiles: the
  // splits are multiples of 256)
  if constexpr (EPI == EPI_OUT || EPI == EPI_F32 || EPI == EPI_F32_ACC) {
    constexpr int64_t es = EPI == EPI_OUT ? 2 : 4;
    const int at = p.c_split_cols ? n0 : m0;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (p.Cx[i] && at >= p.c_split[i])
        p.C = reinterpret_cast<char*>(p.Cx[i]) -
              (int64_t)p.c_split[i] * (p.c_split_cols ? 1 : p.ldc) * es;
  }
  float* W = reinterpret_cast<float*>((wave < 2 ? L0 : L1)) + (wave & 1) * (32 * 128);
  float beta = (float)p.beta;
  if (EPI == EPI_F32_ACC && p.beta_zero && *p.beta_zero) beta = 0.f;
  const bool vec_ok = (p.ldc % 4 == 0) && (EPI != EPI_OUT_RESID || p.ldr % 4 == 0);
  // tiles wholly inside C (nearly all of them) take straight-line code with
  // no per-vector bounds checks (wave-uniform)
  const bool full = vec_ok && m0 + BM <= p.M && n0 + BN <= p.N;
  // All 16 vector passes of a wave's 32-row block are one batch: its old C
  // (read-modify-write) or residual values are loaded before any of its
  // stores, so the 16 loads are in flight together.
  constexpr int BATCH = 16;
  constexpr bool LOADS = EPI == EPI_F32_ACC || EPI == EPI_OUT_RESID;
  if constexpr (EPI == EPI_F32_ACC) {
    // Full tiles that add into C: the old values of a wave's row block are
    // loaded two row blocks ahead (into two register sets), so that their
    // loads overlap the staging and stores of the blocks before them (1%
    // faster on the LM-head weight gradient than loading each block's own
    // old values after staging it).  C is read once and written once per
    // launch, so both go nontemporal and do not evict the operand panels
    // that other blocks of the launch still stream through L2 (LM-head
    // weight gradient 2% faster).
    if (full && beta != 0.f) {  // wave-uniform
      float4 ob[2][16];
      auto ld = [&](int fm, float4 (&o)[16]) __attribute__((always_inline)) {
        const int64_t rc0 = (int64_t)(m0 + wm * WT + fm * 32 + (lane >> 5));
        const int c0 = n0 + wn * WT + (lane & 31) * 4;
#pragma unroll
        for (int bq = 0; bq < 16; ++bq) {
          const ntf4_t t = __builtin_nontemporal_load(
              reinterpret_cast<const ntf4_t*>(reinterpret_cast<const float*>(p.C) + (rc0 + 2 * bq) * p.ldc + c0));
          o[bq] = make_float4(t.x, t.y, t.z, t.w);
        }
      };
      ld(0, ob[0]);
      ld(1, ob[1]);
#pragma unroll
      for (int fm = 0; fm < 4; ++fm) {
#pragma unroll
        for (int fn = 0; fn < 4; ++fn)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int lr = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
            W[lr * 128 + fn * 32 + (lane & 31)] = acc[fm][fn][e];
          }
        __builtin_amdgcn_wave_barrier();
        const int64_t rc0 = (int64_t)(m0 + wm * WT + fm * 32 + (lane >> 5));
        const int c0 = n0 + wn * WT + (lane & 31) * 4;
#pragma unroll
        for (int bq = 0; bq < 16; ++bq) {
          const int lr = bq * 2 + (lane >> 5);
          const float4 v4 = *reinterpret_cast<const float4*>(&W[lr * 128 + (lane & 31) * 4]);
          const float4 o = ob[fm & 1][bq];
          const ntf4_t r = {p.alpha * v4.x + beta * o.x, p.alpha * v4.y + beta * o.y,
                            p.alpha * v4.z + beta * o.z, p.alpha * v4.w + beta * o.w};
          __builtin_nontemporal_store(r, reinterpret_cast<ntf4_t*>(reinterpret_cast<float*>(p.C) + (rc0 + 2 * bq) * p.ldc + c0));
        }
        if (fm + 2 < 4) ld(fm + 2, ob[fm & 1]);
        __builtin_amdgcn_wave_barrier();
      }
      return;
    }
  }
#pragma unroll
  for (int fm = 0; fm < 4; ++fm) {
#pragma unroll
    for (int fn = 0; fn < 4; ++fn)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int lr = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        W[lr * 128 + fn * 32 + (lane & 31)] = acc[fm][fn][e];
      }
    __builtin_amdgcn_wave_barrier();
    if constexpr (EPI == EPI_LSE_TGT || EPI == EPI_REL16_LSE) {
      // statistics (and target values) first; REL16 stores after them
    } else if (full) {
      // rows m0 + wm 128 + fm 32 + 2 bq + l / 32, columns n0 + wn 128 + 4 (l % 32)
      const int64_t rc0 = (int64_t)(m0 + wm * WT + fm * 32 + (lane >> 5));
      const int c0 = n0 + wn * WT + (lane & 31) * 4;
      float4 old[16];
      if constexpr (EPI == EPI_F32_ACC) {
        if (beta != 0.f) {
#pragma unroll
          for (int bq = 0; bq < 16; ++bq)
            old[bq] = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.C) + (rc0 + 2 * bq) * p.ldc + c0);
        } else {
#pragma unroll
          for (int bq = 0; bq < 16; ++bq) old[bq] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      } else if constexpr (EPI == EPI_OUT_RESID) {
#pragma unroll
        for (int bq = 0; bq < 16; ++bq) {
          const uint2 r = *reinterpret_cast<const uint2*>(reinterpret_cast<const bf16_t*>(p.R) + (rc0 + 2 * bq) * p.ldr + c0);
          old[bq] = make_float4(bf2f((bf16_t)(r.x & 0xffff)), bf2f((bf16_t)(r.x >> 16)),
                                bf2f((bf16_t)(r.y & 0xffff)), bf2f((bf16_t)(r.y >> 16)));
        }
      }
#pragma unroll
      for (int bq = 0; bq < 16; ++bq) {
        const int lr = bq * 2 + (lane >> 5);
        const float4 v4 = *reinterpret_cast<const float4*>(&W[lr * 128 + (lane & 31) * 4]);
        float v[4] = {p.alpha * v4.x, p.alpha * v4.y, p.alpha * v4.z, p.alpha * v4.w};
        const int64_t off = (rc0 + 2 * bq) * p.ldc + c0;
        if constexpr (EPI == EPI_F32) {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.C) + off) = make_float4(v[0], v[1], v[2], v[3]);
        } else if constexpr (EPI == EPI_PARTIAL) {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.C) + (int64_t)split * p.split_stride + off) =
              make_float4(v[0], v[1], v[2], v[3]);
        } else if constexpr (EPI == EPI_F32_ACC) {
          const float4 o = old[bq];
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.C) + off) =
              make_float4(v[0] + beta * o.x, v[1] + beta * o.y, v[2] + beta * o.z, v[3] + beta * o.w);
        } else {
          if constexpr (EPI == EPI_OUT_RESID) {
            v[0] += old[bq].x; v[1] += old[bq].y; v[2] += old[bq].z; v[3] += old[bq].w;
          }
          uint2 u;
          u.x = pk_bf16(v[0], v[1]);
          u.y = pk_bf16(v[2], v[3]);
          *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(p.C) + off) = u;
        }
      }
    } else
#pragma unroll
    for (int it0 = 0; it0 < 16; it0 += BATCH) {
      float4 old[BATCH];
      if constexpr (LOADS) {
#pragma unroll
        for (int bq = 0; bq < BATCH; ++bq) {
          const int lr = (it0 + bq) * 2 + (lane >> 5);
          const int row = m0 + wm * WT + fm * 32 + lr;
          const int col = n0 + wn * WT + (lane & 31) * 4;
          old[bq] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (row >= p.M || !vec_ok || col + 4 > p.N) continue;
          if constexpr (EPI == EPI_F32_ACC) {
            if (beta != 0.f)
              old[bq] = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.C) +
                                                         (int64_t)row * p.ldc + col);
          } else {
            const uint2 r = *reinterpret_cast<const uint2*>(reinterpret_cast<const bf16_t*>(p.R) +
                                                            (int64_t)row * p.ldr + col);
            old[bq] = make_float4(bf2f((bf16_t)(r.x & 0xffff)), bf2f((bf16_t)(r.x >> 16)),
                                  bf2f((bf16_t)(r.y & 0xffff)), bf2f((bf16_t)(r.y >> 16)));
          }
        }
      }
#pragma unroll
      for (int bq = 0; bq < BATCH; ++bq) {
        const int lr = (it0 + bq) * 2 + (lane >> 5);
        const int lc = (lane & 31) * 4;
        const float4 v4 = *reinterpret_cast<const float4*>(&W[lr * 128 + lc]);
        float v[4] = {p.alpha * v4.x, p.alpha * v4.y, p.alpha * v4.z, p.alpha * v4.w};
        const int row = m0 + wm * WT + fm * 32 + lr;
        const int col = n0 + wn * WT + lc;
        if (row >= p.M || col >= p.N) continue;
        const int64_t off = (int64_t)row * p.ldc + col;
        if (vec_ok && col + 4 <= p.N) {
          if constexpr (EPI == EPI_F32) {
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.C) + off) = make_float4(v[0], v[1], v[2], v[3]);
          } else if constexpr (EPI == EPI_PARTIAL) {
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.C) + (int64_t)split * p.split_stride + off) =
                make_float4(v[0], v[1], v[2], v[3]);
          } else if constexpr (EPI == EPI_F32_ACC) {
            const float4 o = old[bq];
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.C) + off) =
                make_float4(v[0] + beta * o.x, v[1] + beta * o.y, v[2] + beta * o.z, v[3] + beta * o.w);
          } else {
            if constexpr (EPI == EPI_OUT_RESID) {
              v[0] += old[bq].x; v[1] += old[bq].y; v[2] += old[bq].z; v[3] += old[bq].w;
            }
            uint2 u;
            u.x = pk_bf16(v[0], v[1]);
            u.y = pk_bf16(v[2], v[3]);
            *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(p.C) + off) = u;
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (col + j >= p.N) break;
            if constexpr (EPI == EPI_F32) {
              reinterpret_cast<float*>(p.C)[off + j] = v[j];
            } else if constexpr (EPI == EPI_PARTIAL) {
              reinterpret_cast<float*>(p.C)[(int64_t)split * p.split_stride + off + j] = v[j];
            } else if constexpr (EPI == EPI_F32_ACC) {
              float* c = reinterpret_cast<float*>(p.C) + off + j;
              *c = (beta != 0.f) ? (v[j] + beta * *c) : v[j];
            } else if constexpr (EPI == EPI_OUT) {
              Elem<bf16_t>::store(reinterpret_cast<bf16_t*>(p.C), off + j, v[j]);
            } else {
              const float r = Elem<bf16_t>::load(reinterpret_cast<const bf16_t*>(p.R), (int64_t)row * p.ldr + col + j);
              Elem<bf16_t>::store(reinterpret_cast<bf16_t*>(p.C), off + j, v[j] + r);
            }
          }
        }
      }
    }
    if constexpr (EPI == EPI_REL16_LSE || EPI == EPI_LSE_TGT) {
      // (max, sum-exp) of each row's 64-column quarters of the wave's block,
      // one lane per (row l % 32, quarter l / 32), read from the staged block
      // in a lane-rotated order (conflict-free); no cross-lane traffic.
      const int lr = lane & 31, hq = lane >> 5;
      const int row = m0 + wm * WT + fm * 32 + lr;
      const int cbase = n0 + wn * WT + hq * 64;
      const float* Wr = &W[lr * 128 + hq * 64];
      float m = -INFINITY, sx = 0.f;
      if (full) {
        // two passes over the 64 staged values (max, then the sum of
        // exp(x - max)): no column checks and no data-dependent branches
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float4 q = *reinterpret_cast<const float4*>(Wr + ((j + lane) & 15) * 4);
          m = fmaxf(m, fmaxf(fmaxf(q.x, q.y), fmaxf(q.z, q.w)));
        }
        // exp(x - m) = 2^(x log2 e - m log2 e): one fma and one exp2 each
        constexpr float L2E = 1.4426950408889634f;
        const float ml = m * L2E;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float4 q = *reinterpret_cast<const float4*>(Wr + ((j + lane) & 15) * 4);
          sx += (__builtin_amdgcn_exp2f(__builtin_fmaf(q.x, L2E, -ml)) +
                 __builtin_amdgcn_exp2f(__builtin_fmaf(q.y, L2E, -ml))) +
                (__builtin_amdgcn_exp2f(__builtin_fmaf(q.z, L2E, -ml)) +
                 __builtin_amdgcn_exp2f(__builtin_fmaf(q.w, L2E, -ml)));
        }
      } else
      // one pass, online: the running sum is rescaled when a float4 raises
      // the running max
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int c4 = (j + lane) & 15;
        const float4 q = *reinterpret_cast<const float4*>(Wr + c4 * 4);
        const int c = cbase + c4 * 4;
        const float x0 = c + 0 < p.N ? q.x : -INFINITY, x1 = c + 1 < p.N ? q.y : -INFINITY;
        const float x2 = c + 2 < p.N ? q.z : -INFINITY, x3 = c + 3 < p.N ? q.w : -INFINITY;
        const float m4 = fmaxf(fmaxf(x0, x1), fmaxf(x2, x3));
        if (m4 > m) {
          sx = (m == -INFINITY) ? 0.f : sx * __expf(m - m4);
          m = m4;
        }
        if (m != -INFINITY) sx += __expf(x0 - m) + __expf(x1 - m) + __expf(x2 - m) + __expf(x3 - m);
      }
      if (row < p.M) p.row_stats[(int64_t)row * p.ld_stats + 4 * tn + 2 * wn + hq] = make_float2(m, sx);
      if constexpr (EPI == EPI_REL16_LSE) MQ[wave * 64 + lane] = m;
      if constexpr (EPI == EPI_LSE_TGT || EPI == EPI_REL16_LSE) {
        // the one lane whose quarter holds the row's target column
        if (row < p.M && p.target_out) {
          const int y = p.row_target[row];
          if (y >= cbase && y < cbase + 64 && y < p.N) p.target_out[row] = Wr[y - cbase];
        }
      }
    }
    if constexpr (EPI == EPI_REL16_LSE) {
      // every value minus the max of its 64-column quarter, as fp16, in
      // row-contiguous 8-byte stores (quarter maxima from the pass above);
      // nontemporal: the chunk's logits are read back by the row kernel
      // only after the whole launch
      __builtin_amdgcn_wave_barrier();
      const int q = (lane & 31) >> 4;  // the lane's quarter of the wave's 128 columns
      const int c0 = n0 + wn * WT + (lane & 31) * 4;
      uint16_t* C16 = reinterpret_cast<uint16_t*>(p.C);
#pragma unroll
      for (int bq = 0; bq < 16; ++bq) {
        const int lr = bq * 2 + (lane >> 5);
        const int row = m0 + wm * WT + fm * 32 + lr;
        const float mq = MQ[wave * 64 + q * 32 + lr];
        const float4 v4 = *reinterpret_cast<const float4*>(&W[lr * 128 + (lane & 31) * 4]);
        const float v[4] = {v4.x - mq, v4.y - mq, v4.z - mq, v4.w - mq};
        if (full || (row < p.M && vec_ok && c0 + 4 <= p.N)) {
          const ntu2_t u = {pk_f16(v[0], v[1]), pk_f16(v[2], v[3])};
          __builtin_nontemporal_store(u, reinterpret_cast<ntu2_t*>(C16 + (int64_t)row * p.ldc + c0));
        } else if (row < p.M) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (c0 + j < p.N) C16[(int64_t)row * p.ldc + c0 + j] = __builtin_bit_cast(uint16_t, (_Float16)v[j]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <bool AKM, bool BKM>
static void launch_bf16_ring_layout(int epi, const GemmParams& p, int grid, hipStream_t st) {
  switch (epi) {
    case EPI_F32: hipLaunchKernelGGL((gemm_nt_bf16_ring_kernel<EPI_F32, AKM, BKM>), dim3(grid), dim3(256), 0, st, p); break;
    case EPI_REL16_LSE: hipLaunchKernelGGL((gemm_nt_bf16_ring_kernel<EPI_REL16_LSE, AKM, BKM>), dim3(grid), dim3(256), 0, st, p); break;
    case EPI_LSE_TGT:
      if constexpr (!AKM) hipLaunchKernelGGL((gemm_nt_bf16_ring_kernel<EPI_LSE_TGT, false, false>), dim3(grid), dim3(256), 0, st, p);
      break;
    case EPI_F32_ACC: hipLaunchKernelGGL((gemm_nt_bf16_ring_kernel<EPI_F32_ACC, AKM, BKM>), dim3(grid), dim3(256), 0, st, p); break;
    case EPI_OUT: hipLaunchKernelGGL((gemm_nt_bf16_ring_kernel<EPI_OUT, AKM, BKM>), dim3(grid), dim3(256), 0, st, p); break;
    case EPI_OUT_RESID: hipLaunchKernelGGL((gemm_nt_bf16_ring_kernel<EPI_OUT_RESID, AKM, BKM>), dim3(grid), dim3(256), 0, st, p); break;
    default: hipLaunchKernelGGL((gemm_nt_bf16_ring_kernel<EPI_PARTIAL, AKM, BKM>), dim3(grid), dim3(256), 0, st, p); break;
  }
}

static void launch_bf16_ring(int epi, GemmParams p, hipStream_t st) {
  p.tiles_m = (int)cdiv(p.M, 256);
  p.tiles_n = (int)cdiv(p.N, 256);
  const int grid = p.tiles_m * p.tiles_n * p.k_split;
  if (p.a_kmajor)
    launch_bf16_ring_layout<true, true>(epi, p, grid, st);
  else
    launch_bf16_ring_layout<false, false>(epi, p, grid, st);
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

int gemm_k_granule(int dtype) { return dtype == SBP_BF16 ? 128 : 32; }

sbp_status gemm_nt(int dtype, int epi, GemmParams p, int tile, hipStream_t st, const char* name) {
  if (p.M <= 0 || p.N <= 0) return SBP_OK;
  if (p.k_split < 1) p.k_split = 1;
  const int gran = gemm_k_granule(dtype);
  if (p.k_per_split <= 0) p.k_per_split = (int)round_up(cdiv(p.K, p.k_split), gran);
  const double flops = 2.0 * p.M * p.N * (double)p.K;
  const size_t esz = dtype == SBP_BF16 ? 2 : 4;
  const double bytes = ((double)p.M * p.K + (double)p.N * p.K) * esz +
                       (double)p.M * p.N * (epi == EPI_F32_ACC ? 8.0 : epi == EPI_OUT || epi == EPI_OUT_RESID ? (double)esz : epi == EPI_LSE_TGT ? 0.0 : epi == EPI_REL16_LSE ? 2.0 : 4.0 * p.k_split);
  // (the row statistics of EPI_REL16_LSE / EPI_LSE_TGT add 8 bytes per 64 output columns)
  ProfScope prof(name, st, flops, bytes);
  const bool ring_ok = dtype == SBP_BF16 && (p.K % 8 == 0 || p.a_kmajor) &&
                       p.k_per_split % 128 == 0 && p.lda % 8 == 0 && p.ldb % 8 == 0 &&
                       (!p.a_kmajor || p.lda >= round_up(p.M, 8)) &&
                       (!p.b_kmajor || p.ldb >= round_up(p.N, 8));
  if ((epi == EPI_REL16_LSE || epi == EPI_LSE_TGT) &&
      !(tile == GEMM_TILE_RING && ring_ok && p.k_split == 1 && p.row_stats))
    return set_error(SBP_ERR_UNSUPPORTED, "row-statistics epilogue needs the bf16 ring GEMM without split-K");
  if (epi == EPI_REL16_LSE && p.target_out && !p.row_target)
    return set_error(SBP_ERR_INVALID_ARG, "target-value output needs the row target array");
  if (epi == EPI_LSE_TGT && (p.a_kmajor || !p.row_target || !p.target_out))
    return set_error(SBP_ERR_UNSUPPORTED, "target-value epilogue needs row-major operands and its row arrays");
  if ((p.a_kmajor || p.b_kmajor) && !(tile == GEMM_TILE_RING && ring_ok && p.a_kmajor == p.b_kmajor))
    return set_error(SBP_ERR_UNSUPPORTED, "K-major GEMM operands need the bf16 ring GEMM, both K-major");
  if (p.B2 || p.Cx[0] || p.Cx[1]) {
    const bool ok = tile == GEMM_TILE_RING && ring_ok && p.k_split == 1 &&
                    (epi == EPI_OUT || epi == EPI_F32 || epi == EPI_F32_ACC) &&
                    (!p.B2 || (!p.b_kmajor && p.b_split > 0 && p.b_split % 256 == 0)) &&
                    (!p.Cx[0] || (p.c_split[0] > 0 && p.c_split[0] % 256 == 0)) &&
                    (!p.Cx[1] || (p.Cx[0] && p.c_split[1] > p.c_split[0] && p.c_split[1] % 256 == 0));
    if (!ok) return set_error(SBP_ERR_UNSUPPORTED, "GEMM operand/output splits need the bf16 ring GEMM and tile-aligned splits");
  }
  if (dtype == SBP_BF16) {
    if (tile == GEMM_TILE_RING && ring_ok)
      launch_bf16_ring(epi, p, st);
    else
      launch_cfg<bf16_t, 128, 128, 2, 2>(epi, p, st);
  } else {
    launch_cfg<float, 128, 128, 2, 2>(epi, p, st);
  }
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

}  // namespace sbp
