// sbp_attn_bwd_chunked: causal GQA attention backward, chunked over queries.
//
// StreamBP skill page, "Architecture Overview" (causal structure
// exploitation) and "Practical Guidance" (masks across chunk boundaries,
// causal masking): query chunk c = [s, e) reads keys/values [0, e) only, and
// inside it no key block above the diagonal is visited.  Per chunk, in
// reverse order:
//   attn_fwd_kernel   per (128-query tile, q head): S^T = K Q^T over the
//                     causal prefix, online softmax per query, O^T += V^T P^T;
//                     writes LSE and Delta = rowsum(dO * O) (and O if asked).
//   attn_dkdv_kernel  per (128-key tile, kv head): for every q head of the
//                     group and every query tile of the chunk that sees the
//                     keys: S = Q K^T, P, dP = dO V^T, dS = P (dP - Delta),
//                     dV += P^T dO, dK += dS^T Q; fp32 read-modify-write.
//   attn_dq_kernel    per (128-query tile, q head): S^T, dP^T over key tiles
//                     up to the diagonal, dQ += dS K.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, wave64): the A operand of
// lane l holds row l%32 and 8 consecutive k of group l/32; B likewise by
// column; the 32x32 fp32 result has lane l holding column l%32 and rows
// 8*(e/4) + 4*(l/32) + e%4, e = 0..15.  Because that result column is the
// lane, a score block computed in one orientation is already, element by
// element, the A (or B) operand of the next product in the other
// orientation: elements 8i..8i+7 of a lane form the k16 step i, whose k
// index e maps to the block row above.  The matching operand of that product
// (dO, Q, K or V with the contraction over its rows) is read transposed from
// LDS with ds_read_b64_tr_b16: within each 16-lane group, lane i returns
// element i%4 of the 8-byte chunks fetched by lanes i/4 + 4m (m = 0..3), so
// 16 lanes that fetch 4 rows x 16 columns receive one column each, 4 rows
// deep.  LDS tiles are rows of dh bf16 with 16-byte chunk c of row r stored
// at c ^ f(r).  gfx950's LDS serves 256 bytes (64 four-byte banks) per
// clock: 16 lanes of a 16-byte row read, 32 lanes of an 8-byte transposed
// read.  f is chosen so that both are conflict-free: the row read's 16 rows
// r..r+15 land on 16 distinct chunks of the 256-byte bank line, and the
// transposed read's 4 rows x 64 bytes on 4 distinct 64-byte quarters.
//   dh 128 (rows of 256 B):  f(r) = 4 (r & 3) + ((r >> 2) & 3)
//   dh  64 (rows of 128 B):  f(r) = 4 ((r >> 1) & 1) + ((r >> 2) & 3)
// (f depends on r mod 16 only).
#include "attn.h"
#include "common.h"
#include "kernels.h"

namespace sbp {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
#define SBP_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int DH>
__device__ __forceinline__ int swz(int r) {
  return DH == 128 ? ((r & 3) << 2) | ((r >> 2) & 3) : (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// LDS DMA as inline assembly: global_load_lds_dwordx4, lane l's 16 bytes
// landing at M0 + 16 l.  Issued this way the compiler does not track the
// LDS writes.  Tracked, it could not tell a tile's fragment reads from the
// next tile's fill in flight (one LDS array, computed offsets) and waited for
// that fill before the tile's first read, exposing its whole latency every
// tile; and any fill it tracked made it wait for every outstanding LDS read
// (lgkmcnt(0)) before each MFMA, where a count of the reads still needed
// suffices.  The kernels order fills and reads themselves: dma_barrier before
// a buffer is read, a full wait before LDS is reused for anything else.  s_nop 4: the
// wait states gfx9 needs between an SGPR written by a vector instruction (a
// readfirstlane) and a memory instruction that reads it; they also cover the
// one an M0 write needs before an LDS DMA.
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)p;  // low half of a generic LDS address
}
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g),
               "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}
// uniform 64-bit base plus a per-lane 32-bit byte offset
__device__ __forceinline__ void dma16_s(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base),
               "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// DMA rows [0, 64) of a [rows][DH] bf16 tile (global row pitch ld elements)
// into a swizzled LDS tile: each 1 KB global_load_lds covers 1024 / (2 DH)
// rows, lane i filling 16-byte slot i, so the swizzle is applied to the
// global address (lane i fetches logical chunk (i % CPR) ^ f(row)).  Rows at
// or past nvalid fetch row nvalid - 1 instead (finite data the callers mask).
template <int DH>
__device__ __forceinline__ void dma_tile64(char* lds, const bf16_t* __restrict__ src, int64_t ld,
                                           int nvalid, int wave, int lane) {
  constexpr int ROWB = DH * 2, RPI = 1024 / ROWB, NI = 64 / RPI, CPR = DH / 8;
  const int rr = lane / CPR, pc = lane % CPR;
#pragma unroll
  for (int i = wave; i < NI; i += 4) {
    const int r = i * RPI + rr;
    const int c = pc ^ swz<DH>(r);
    const int gr = r < nvalid ? r : nvalid - 1;
    dma16(src + (int64_t)gr * ld + c * 8, lds_u32(lds + i * 1024));
  }
}

// DMA of quarter q (16 floats) of a row of 64 consecutive fp32 (16-byte
// aligned, in bounds) with lanes 0..3: four waves fetch one row together, so
// that every wave issues the same number of DMAs.
__device__ __forceinline__ void dma_f32x16(float* lds, const float* __restrict__ src, int q, int lane) {
  if (lane < 4) dma16(src + q * 16 + lane * 4, lds_u32(lds + q * 16));
}

// Double-buffer hand-over.  The DMA writes of a tile are counted by each
// wave's own vmcnt, so every wave first waits for its share of the tile about
// to be read, and the barrier then makes all shares visible (it also ends
// every wave's reads of the buffer about to be refilled).  The wave index is
// made wave-uniform (readfirstlane) so that the DMA issue branches are scalar.
__device__ __forceinline__ void dma_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The DMA of dma_tile64 for tiles whose 64 rows all exist, from per-lane byte
// offsets formed once (dma64_offsets): only the wave-uniform tile base
// changes from tile to tile, so each DMA is a scalar base plus a fixed
// 32-bit lane offset (64 rows of a pitch below 2^25 elements).
template <int DH, int NW>
struct Dma64Off {
  static constexpr int ROWB = DH * 2, RPI = 1024 / ROWB, NI = 64 / RPI, PER = NI / NW;
  uint32_t off[PER];
  __device__ __forceinline__ Dma64Off(int64_t ld, int wave, int lane) {
    constexpr int CPR = DH / 8;
    const int rr = lane / CPR, pc = lane % CPR;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int r = (wave + NW * j) * RPI + rr;
      off[j] = (uint32_t)((int64_t)r * ld + 8 * (pc ^ swz<DH>(r))) * 2u;
    }
  }
};
template <int DH, int NW>
__device__ __forceinline__ void dma_tile64_full(char* lds, const bf16_t* __restrict__ src, const Dma64Off<DH, NW>& o,
                                                int wave) {
#pragma unroll
  for (int j = 0; j < Dma64Off<DH, NW>::PER; ++j) dma16_s(src, o.off[j], lds_u32(lds + (wave + NW * j) * 1024));
}

// Block -> work mapping for the 8 XCDs.  Workgroups are dispatched
// round-robin over the XCDs in linear order (x fastest), so the kv head is
// taken from the low part of the linear id: when Hkv divides 8 every block
// of one kv head runs on the same XCD and the K / V (or Q / dO) it streams
// stays in that XCD's L2.  Query blocks are issued heaviest (most keys)
// first.  A grid that fits the chip in one round at two blocks per CU (512
// blocks or fewer) puts the first half of its blocks one per CU and the
// second half into the CUs' second slots; that half is issued lightest
// first, so that a CU's two blocks sum to about the same work.
struct QBlock {
  int h, qblk;
};
__device__ __forceinline__ QBlock q_block(int Hkv, int G) {
  const int lin = blockIdx.x + gridDim.x * blockIdx.y;
  const int kv = lin % Hkv;
  int r = lin / Hkv;               // rank by work, heaviest first
  const int R = (int)gridDim.x * G;
  if (gridDim.x * gridDim.y * gridDim.z <= 512 && r >= R / 2) r = R / 2 + (R - 1 - r);
  return {kv * G + r % G, (int)gridDim.x - 1 - r / G};
}
struct KBlock {
  int kv, kblk;
};
__device__ __forceinline__ KBlock k_block(int Hkv) {
  const int lin = blockIdx.x + gridDim.x * blockIdx.y;
  return {lin % Hkv, lin / Hkv};
}

// Per-lane LDS byte offsets of the fragment reads of a swizzled tile, so
// that every read is a per-lane register plus a compile-time immediate:
//   row read, rows rbase + l%32 (rbase % 32 == 0), k16 step ks (16-byte
//     chunk 2 ks + l/32):                       row[ks] + rbase * 2DH
//   transposed read of column block nb, rows rbase + 4(l/32) + 0..3 and
//     the same + 8 (rbase % 16 == 0):           tr[nb][0 / 1] + rbase * 2DH
// (checked exhaustively against the DMA placement on the host).
template <int DH>
struct LdsOff {
  static constexpr int KS = DH / 16, NB = DH / 32, ROWB = DH * 2;
  int row[KS], tr[NB][2];
  // rbase (a multiple of 16, wave-uniform): a row offset folded into the
  // lane offsets, so that reads of a wave's fixed rows need no address add
  __device__ __forceinline__ explicit LdsOff(int lane, int rbase = 0) {
    const int g = lane >> 5, r = lane & 31, f = swz<DH>(r);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) row[ks] = (rbase + r) * ROWB + 16 * ((2 * ks + g) ^ f);
    const int G = (lane >> 4) & 3, j = lane & 15;
    const int rr = 4 * (G >> 1) + (j >> 2), colc = 2 * (G & 1) + ((j & 3) >> 1);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int rw = rr + 8 * h;
        tr[nb][h] = (rbase + rw) * ROWB + 16 * ((4 * nb + colc) ^ swz<DH>(rw)) + 8 * (j & 1);
      }
  }
  // 16-byte row read: row rbase + l%32, columns 16 ks + 8 (l/32) .. + 8
  __device__ __forceinline__ uint4 row_frag(const char* t, int rbase, int ks) const {
    return *reinterpret_cast<const uint4*>(t + row[ks] + rbase * ROWB);
  }
  // Transposed read: 8 bf16 of column 32 nb + l%32 at rows rbase + 4(l/32) +
  // {0..3} and rbase + 8 + 4(l/32) + {0..3}.
  __device__ __forceinline__ uint4 tr_frag(const char* t, int rbase, int nb) const {
    const SBP_LDS char* p = (const SBP_LDS char*)t + rbase * ROWB;
    i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SBP_LDS i16x4_t*)(p + tr[nb][0]));
    i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SBP_LDS i16x4_t*)(p + tr[nb][1]));
    uint4 u;
    u.x = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
    u.y = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
    u.z = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
    u.w = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
    return u;
  }
};

// Elements 8i..8i+7 of a result block as a bf16 operand (k16 step i).
__device__ __forceinline__ uint4 pack_frag(const f32x16_t& a, int i) {
  uint4 u;
  u.x = pk_bf16(a[8 * i + 0], a[8 * i + 1]);
  u.y = pk_bf16(a[8 * i + 2], a[8 * i + 3]);
  u.z = pk_bf16(a[8 * i + 4], a[8 * i + 5]);
  u.w = pk_bf16(a[8 * i + 6], a[8 * i + 7]);
  return u;
}

__device__ __forceinline__ f32x16_t mma(const uint4& a, const uint4& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Row of element e of a result block for this lane.
__device__ __forceinline__ int crow(int e, int lane) { return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }

// 16-byte global fragment of a [rows][DH] matrix (row pitch ld): row r,
// k16 step ks, group g: columns 16 ks + 8 g .. +8; zero past nrows.
template <int DH>
__device__ __forceinline__ uint4 glb_frag(const bf16_t* __restrict__ p, int64_t ld, int r, int nrows,
                                          int ks, int g) {
  if (r >= nrows) return make_uint4(0, 0, 0, 0);
  return *reinterpret_cast<const uint4*>(p + (int64_t)r * ld + ks * 16 + g * 8);
}

// Key range of a wave of 32 queries [qw, qw + 32) (forward and dQ):
// kfirst is the first key any query of the block sees, klo this lane's own
// first key, [wlo, whi] the first keys of the wave's first and last query.
// kind(k0) classifies the 64-key tile [k0, k0 + 64) for the wave: 0 none of
// its keys is seen, 1 every query sees every key, 2 a mask is needed.
struct SeqRange {
  int kfirst, klo, wlo, whi, qw;
  __device__ __forceinline__ int kind(int k0) const {
    if (k0 > qw + 31 || k0 + 63 < wlo) return 0;
    return (k0 + 63 <= qw && k0 >= whi) ? 1 : 2;
  }
};
__device__ __forceinline__ SeqRange seq_range(const AttnArgs& a, int q0, int qw, int qcol) {
  SeqRange r{0, 0, 0, 0, qw};
  if (a.seq_lo) {
    const int last = a.e - 1;  // rows past the chunk take its last query's bounds
    r.kfirst = a.seq_lo[min(q0, last)];
    r.klo = a.seq_lo[min(qcol, last)];
    r.wlo = a.seq_lo[min(qw, last)];
    r.whi = a.seq_lo[min(qw + 31, last)];
  }
  return r;
}

// ---------------------------------------------------------------------------
// Forward statistics.  Block: 4 waves, 128 queries (32 per wave), one q head.
// Key/value tiles of 64 rows are double-buffered in two LDS arrays: tile t+1
// is fetched while tile t is used.
// ---------------------------------------------------------------------------
template <int DH, bool MASK>
__device__ __forceinline__ void fwd_tile(const LdsOff<DH>& lo, const char* kt, const char* vt, int k0, int qcol,
                                         int klo, int lane, float c2, const uint4 (&qf)[DH / 16], float& m,
                                         float& l, f32x16_t (&ot)[DH / 32]) {
  constexpr int NB = DH / 32, KS = DH / 16;
  f32x16_t st[2];
  // The two MFMA phases run at raised wave priority: of the two waves on a
  // SIMD, the one with matrix work issues first while the other is in its
  // softmax.  (Measured 4-5% faster here; the dQ and dK/dV kernels ran 1-3%
  // slower with the same change, so they keep the default.)
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    st[kb] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) st[kb] = mma(lo.row_frag(kt, kb * 32, ks), qf[ks], st[kb]);
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
  // mask (key > query, or key before the query's sequence start klo), online
  // softmax along the keys (rows).  The scores stay unscaled: the scale c2 is
  // positive, so the scaled maximum is c2 times the raw one (rounding is
  // monotonic), and it enters the exponent through one fma per score.
  float mt = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if constexpr (MASK) {
        const int key = k0 + kb * 32 + crow(e, lane);
        if (!(key <= qcol && key >= klo)) st[kb][e] = -INFINITY;
      }
      mt = fmaxf(mt, st[kb][e]);
    }
  mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * c2;
  // Lazy rescale: the running max m only moves (and O, l are rescaled) when
  // some lane's tile max exceeds it by more than 8 (base 2); otherwise P is
  // taken against the stale m and stays <= 2^8 (exact in the fp32 sums, the
  // same relative precision in bf16).  LSE = m + log2 l either way.  m starts
  // finite (-1e30), so a query none of whose keys a tile shows (packed
  // sequences) gets p = exp2(-inf) = 0, not NaN.
  const bool raise = __ballot(mt > m + 8.f) != 0;
  float ls = 0.f;
  if (raise) {  // wave-uniform
    const float mn = fmaxf(m, mt);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    l *= alpha;
    m = mn;
#pragma unroll
    for (int i = 0; i < NB; ++i) ot[i] *= alpha;
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][e], c2, -m));
      st[kb][e] = p;
      ls += p;
    }
  ls += __shfl_xor(ls, 32, 64);
  l += ls;
  // O^T[dh, q] += V^T[dh, key] P^T[key, q]
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 pb = pack_frag(st[kb], i);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        ot[nb] = mma(lo.tr_frag(vt, kb * 32 + 16 * i, nb), pb, ot[nb]);
    }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
}

template <int DH>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(AttnArgs a) {
  constexpr int NB = DH / 32;   // 32-wide dh blocks
  constexpr int KS = DH / 16;   // k16 steps over dh
  __shared__ __attribute__((aligned(16))) char K0[64 * DH * 2];
  __shared__ __attribute__((aligned(16))) char V0[64 * DH * 2];
  __shared__ __attribute__((aligned(16))) char K1[64 * DH * 2];
  __shared__ __attribute__((aligned(16))) char V1[64 * DH * 2];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const QBlock qbk = q_block(a.Hkv, a.G);
  const int h = qbk.h, b = blockIdx.z, kv = h / a.G;
  const LdsOff<DH> lo(lane);
  const int q0 = a.s + qbk.qblk * 128;              // first query of the block
  const int qw = q0 + wave * 32;                    // first query of the wave
  const int qcol = qw + (lane & 31);                // this lane's query
  const int64_t ldq = a.ldq, ldk = (int64_t)a.Hkv * DH;
  const bf16_t* Qb = a.Q + (int64_t)b * a.q_bs + (int64_t)h * DH;  // row t at (t - qoff)
  const bf16_t* Kb = a.K + ((int64_t)b * a.T) * ldk + (int64_t)kv * DH;
  const bf16_t* Vb = a.V + ((int64_t)b * a.T) * ldk + (int64_t)kv * DH;
  const int qrel = qcol - a.qoff, qend = a.e - a.qoff;

  // Q^T as the B operand of S^T = K Q^T: column = query, k = dh
  uint4 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = glb_frag<DH>(Qb, ldq, qrel, qend, ks, lane >> 5);

  f32x16_t ot[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) ot[i] = f32x16_t{};
  float m = -1e30f, l = 0.f;
  const float c2 = a.scale * kLog2e;

  // keys [kfirst, kend): packed sequences start at the sequence of the
  // block's first query; klo is this lane's own lower key bound, [wlo, whi]
  // the range of the wave's (seq_lo is non-decreasing)
  const SeqRange sr = seq_range(a, q0, qw, qcol);
  const int kend = min(q0 + 128, a.e);
  const int ntiles = (kend + 63) / 64, t0 = sr.kfirst / 64;
  const Dma64Off<DH, 4> kvoff(ldk, wave, lane);
  auto issue = [&](char* kd, char* vd, int t) {
    const int k0 = t * 64;
    if (kend - k0 >= 64) {  // wave-uniform
      dma_tile64_full<DH, 4>(kd, Kb + (int64_t)k0 * ldk, kvoff, wave);
      dma_tile64_full<DH, 4>(vd, Vb + (int64_t)k0 * ldk, kvoff, wave);
    } else {
      dma_tile64<DH>(kd, Kb + (int64_t)k0 * ldk, ldk, kend - k0, wave, lane);
      dma_tile64<DH>(vd, Vb + (int64_t)k0 * ldk, ldk, kend - k0, wave, lane);
    }
  };
  issue(K0, V0, t0);
  for (int t = t0; t < ntiles; t += 2) {
    dma_barrier();  // tile t landed; everyone is done with the other buffer
    issue(K1, V1, min(t + 1, ntiles - 1));
    // only tiles that reach past the wave's first query (or, packed, start
    // before its last query's sequence) need the mask
    switch (sr.kind(t * 64)) {
      case 1: fwd_tile<DH, false>(lo, K0, V0, t * 64, qcol, sr.klo, lane, c2, qf, m, l, ot); break;
      case 2: fwd_tile<DH, true>(lo, K0, V0, t * 64, qcol, sr.klo, lane, c2, qf, m, l, ot); break;
      default: break;
    }
    dma_barrier();
    issue(K0, V0, min(t + 2, ntiles - 1));
    if (t + 1 < ntiles) switch (sr.kind((t + 1) * 64)) {
      case 1: fwd_tile<DH, false>(lo, K1, V1, (t + 1) * 64, qcol, sr.klo, lane, c2, qf, m, l, ot); break;
      case 2: fwd_tile<DH, true>(lo, K1, V1, (t + 1) * 64, qcol, sr.klo, lane, c2, qf, m, l, ot); break;
      default: break;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // no DMA may still target LDS at exit
  if (qcol >= a.e) return;
  const float inv = 1.f / l;
  const float lse = m + log2f(l);  // base-2 units (scores were scaled by log2 e)
  const int64_t row = (int64_t)b * a.q_bs + (int64_t)qrel * ldq + (int64_t)h * DH;
  // Delta = sum_dh dO * O, O from the fp32 accumulator; O written if asked
  float dsum = 0.f;
  const bf16_t* dorow = a.dO ? a.dO + row : nullptr;
  bf16_t* orow = a.O ? a.O + row : nullptr;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = nb * 32 + 8 * q4 + 4 * (lane >> 5);  // rows of elements 4q4 .. 4q4+3
      float o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = ot[nb][4 * q4 + j] * inv;
      if (dorow) {
        const uint2 u = *reinterpret_cast<const uint2*>(dorow + d0);
        dsum += o[0] * bf2f((bf16_t)(u.x & 0xffff)) + o[1] * bf2f((bf16_t)(u.x >> 16)) +
                o[2] * bf2f((bf16_t)(u.y & 0xffff)) + o[3] * bf2f((bf16_t)(u.y >> 16));
      }
      if (orow) {
        uint2 w;
        w.x = pk_bf16(o[0], o[1]);
        w.y = pk_bf16(o[2], o[3]);
        *reinterpret_cast<uint2*>(orow + d0) = w;
      }
    }
  dsum += __shfl_xor(dsum, 32, 64);
  if (lane < 32) {
    a.lse[(int64_t)b * a.lse_sb + (int64_t)h * a.lse_sh + (int64_t)(qcol - a.s) * a.lse_st] = lse;
    if (a.dO) a.delta[(int64_t)b * a.dl_sb + (int64_t)h * a.dl_sh + (int64_t)(qcol - a.s) * a.dl_st] = dsum;
  }
}

// ---------------------------------------------------------------------------
// Delta = rowsum(dO * O) from a given O (dtype), one wave per (row, head);
// optionally also copies a caller's LSE ([B, T, Hq], rows of the chunk) into
// the statistics layout.
// ---------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(256) void attn_delta_kernel(AttnArgs a, const bf16_t* __restrict__ O,
                                                         const float* __restrict__ lse_src,
                                                         int64_t lsb, int64_t lst) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t idx = (int64_t)blockIdx.x * 4 + wave;  // over Tc * Hq rows of batch row b
  const int Tc = a.e - a.s;
  if (idx >= (int64_t)Tc * a.Hq) return;
  const int b = blockIdx.y;
  const int h = (int)(idx % a.Hq);
  const int t = a.s + (int)(idx / a.Hq);
  const int64_t off = (int64_t)b * a.q_bs + (int64_t)(t - a.qoff) * a.ldq + (int64_t)h * DH;
  float s = 0.f;
  for (int d = lane; d < DH; d += 64) s += bf2f(a.dO[off + d]) * bf2f(O[off + d]);
  s = wave_sum(s);
  if (lane == 0) {
    a.delta[(int64_t)b * a.dl_sb + (int64_t)h * a.dl_sh + (int64_t)(t - a.s) * a.dl_st] = s;
    if (lse_src)
      a.lse[(int64_t)b * a.lse_sb + (int64_t)h * a.lse_sh + (int64_t)(t - a.s) * a.lse_st] =
          lse_src[(int64_t)b * lsb + (int64_t)t * lst + h] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dK, dV.  Block: 8 waves (two per SIMD), 128 keys, one kv head.  Wave w owns
// the 32 keys kbase + 32 (w & 3) and the query half w >> 2 of every 64-query
// tile; the two waves of a key group add their dK / dV partials through LDS
// at the end.  K and V of the block stay in LDS for the whole loop (B
// operands of S = Q K^T and dP = dO V^T, read per step), which keeps a wave
// within 256 registers so that two waves share each SIMD and cover each
// other's latencies.  The block iterates over (q head of the group, 64-query
// tile of the chunk at or after the keys); the Q / dO tiles and their LSE /
// Delta rows are double-buffered by DMA.  Query tiles start at s + 64 j so
// the statistics rows are 16-byte aligned; statistics rows are padded past
// the chunk so every 64-row fetch is in bounds, and queries at or past e are
// masked.
// ---------------------------------------------------------------------------

// DMA of rows [0, 64) of a [rows][DH] tile by the 8 waves of a block (same
// placement as dma_tile64).
template <int DH>
__device__ __forceinline__ void dma_tile64_w8(char* lds, const bf16_t* __restrict__ src, int64_t ld,
                                              int nvalid, int wave, int lane) {
  constexpr int ROWB = DH * 2, RPI = 1024 / ROWB, NI = 64 / RPI, CPR = DH / 8;
  const int rr = lane / CPR, pc = lane % CPR;
#pragma unroll
  for (int i = wave; i < NI; i += 8) {
    const int r = i * RPI + rr;
    const int c = pc ^ swz<DH>(r);
    const int gr = r < nvalid ? r : nvalid - 1;
    dma16(src + (int64_t)gr * ld + c * 8, lds_u32(lds + i * 1024));
  }
}

// Softmax step of a dK/dV tile: P = exp(s S - LSE), dS = P (dP - Delta) in
// place; elements 4j..4j+3 are rows 8j + 4(l/32) + 0..3 of the wave's 32
// queries.  MASK zeroes the pairs a query does not see.  The LSE / Delta rows
// of j = 0, 1 come in registers (read during the last score step), those of
// j = 2, 3 from the LDS rows ls / dl.
template <bool MASK>
__device__ __forceinline__ void dkdv_softmax(f32x16_t& sp, f32x16_t& dp, const float4 (&l4s)[2],
                                             const float4 (&d4s)[2], const float* ls, const float* dl, int qrow,
                                             int q0, int kcol, int qlim, int lane, float c2) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r0 = qrow + 8 * j + 4 * (lane >> 5);
    const float4 l4 = j < 2 ? l4s[j & 1] : *reinterpret_cast<const float4*>(ls + r0);
    const float4 d4 = j < 2 ? d4s[j & 1] : *reinterpret_cast<const float4*>(dl + r0);
    const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv_[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e_ = 4 * j + i;
      float p = __builtin_amdgcn_exp2f(sp[e_] * c2 - lv[i]);
      float g = p * (dp[e_] - dv_[i]);
      if constexpr (MASK) {
        // statistics rows past the chunk are padding (any value): select, do
        // not multiply, so that they cannot leak in.  qlim: the end of the
        // chunk or of the key's sequence, whichever comes first
        const int q = q0 + r0 + i;
        const bool on = kcol <= q && q < qlim;
        p = on ? p : 0.f;
        g = on ? g : 0.f;
      }
      sp[e_] = p;
      dp[e_] = g;
    }
  }
}

// One wave's share of a 64-query tile: its 32 queries (tile rows qrow ..
// qrow + 31) against its 32 keys (K / V tile rows krow .. krow + 31).  The
// matrix phases are shared by masked and unmasked tiles; the softmax between
// them is one straight-line block of either kind (one wave-uniform branch).
// lq / lk: fragment offsets with the wave's query rows (qrow) and key rows
// folded in.
template <int DH>
__device__ __forceinline__ void dkdv_tile(const LdsOff<DH>& lq, const LdsOff<DH>& lk, const char* kt,
                                          const char* vt, const char* qt, const char* ot, const float* ls,
                                          const float* dl, int qrow, int q0, int kcol, int qlim, int lane,
                                          float c2, bool mask, f32x16_t (&dk)[DH / 32],
                                          f32x16_t (&dv)[DH / 32]) {
  constexpr int NB = DH / 32, KS = DH / 16;
  // S = Q K^T and dP = dO V^T: [32 queries x 32 keys], fragments one step ahead
  f32x16_t sp = f32x16_t{}, dp = f32x16_t{};
  // LSE / Delta rows of j = 0, 1, read in the last score step (into the
  // fragment registers it frees) so that the softmax does not start on an LDS
  // wait; reading all four there spills
  float4 l4s[2], d4s[2];
  auto ldle = [&](int j) {
    const int r0 = qrow + 8 * j + 4 * (lane >> 5);
    l4s[j] = *reinterpret_cast<const float4*>(ls + r0);
    d4s[j] = *reinterpret_cast<const float4*>(dl + r0);
  };
  {
    uint4 fq[2], fk[2], fo[2], fv[2];
    auto ld = [&](int ks) {
      fq[ks & 1] = lq.row_frag(qt, 0, ks);
      fk[ks & 1] = lk.row_frag(kt, 0, ks);
      fo[ks & 1] = lq.row_frag(ot, 0, ks);
      fv[ks & 1] = lk.row_frag(vt, 0, ks);
    };
    ld(0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) {
        ld(ks + 1);
      } else {
        ldle(0);
        ldle(1);
      }
      __builtin_amdgcn_sched_barrier(0);
      sp = mma(fq[ks & 1], fk[ks & 1], sp);
      dp = mma(fo[ks & 1], fv[ks & 1], dp);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (mask)  // wave-uniform
    dkdv_softmax<true>(sp, dp, l4s, d4s, ls, dl, qrow, q0, kcol, qlim, lane, c2);
  else
    dkdv_softmax<false>(sp, dp, l4s, d4s, ls, dl, qrow, q0, kcol, qlim, lane, c2);
  // dV[key, dh] += P^T[key, q] dO[q, dh];  dK[key, dh] += dS^T[key, q] Q[q, dh]
  {
    uint4 tq[2], to[2];
    auto ld = [&](int st) {
      const int r = (st / NB) * 16, nb = st % NB;
      to[st & 1] = lq.tr_frag(ot, r, nb);
      tq[st & 1] = lq.tr_frag(qt, r, nb);
    };
    ld(0);
    uint4 pa, da;
#pragma unroll
    for (int st = 0; st < 2 * NB; ++st) {
      if (st + 1 < 2 * NB) ld(st + 1);
      __builtin_amdgcn_sched_barrier(0);
      const int i = st / NB, nb = st % NB;
      if (nb == 0) {
        pa = pack_frag(sp, i);
        da = pack_frag(dp, i);
      }
      dv[nb] = mma(pa, to[st & 1], dv[nb]);
      dk[nb] = mma(da, tq[st & 1], dk[nb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <int DH>
__global__ __launch_bounds__(512) void attn_dkdv_kernel(AttnArgs a) {
  constexpr int NB = DH / 32, TB = 64 * DH * 2;
  // One LDS array, laid out so that every fragment read is a lane register
  // plus an immediate below 64 KB: the Q / dO double buffers first (read
  // 48 times per tile), then K and V of the block's 128 keys (their base is
  // folded into the lane offsets of lk), then the LSE / Delta rows.
  __shared__ __attribute__((aligned(16))) char smem[8 * TB + 4 * 64 * sizeof(float)];
  char* const Q0 = smem;
  char* const O0 = smem + TB;  // dO tile
  char* const Q1 = smem + 2 * TB;
  char* const O1 = smem + 3 * TB;
  char* const Kt = smem + 4 * TB;  // 128 keys
  char* const Vt = smem + 6 * TB;
  float* const L0 = reinterpret_cast<float*>(smem + 8 * TB);
  float* const E0 = L0 + 64;
  float* const L1 = L0 + 128;
  float* const E1 = L0 + 192;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave & 3, qh = wave >> 2;
  const KBlock kbk = k_block(a.Hkv);
  const int kv = kbk.kv, b = blockIdx.z;
  const LdsOff<DH> lq(lane, (wave >> 2) * 32), lk(lane, 4 * TB / (2 * DH) + (wave & 3) * 32);
  const int kbase = kbk.kblk * 128;
  const int kw = kbase + kg * 32;
  const int kcol = kw + (lane & 31);  // this lane's key (result column)
  const int qrow = qh * 32;           // the wave's rows of each query tile
  const int64_t ldq = a.ldq, ldk = (int64_t)a.Hkv * DH;
  const bf16_t* Kb = a.K + ((int64_t)b * a.T + kbase) * ldk + (int64_t)kv * DH;
  const bf16_t* Vb = a.V + ((int64_t)b * a.T + kbase) * ldk + (int64_t)kv * DH;
  f32x16_t dk[NB], dv[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    dk[i] = f32x16_t{};
    dv[i] = f32x16_t{};
  }
  const float c2 = a.scale * kLog2e;
  // Queries that see a key j: [j, qlim(j)), qlim the end of the chunk or,
  // packed, of j's sequence (non-decreasing in j).  qlim of this lane's key,
  // and of the wave's first and last key.
  auto qlim_of = [&](int j) { return a.seq_hi ? min(a.e, a.seq_hi[min(j, a.T - 1)]) : a.e; };
  const int qlim = qlim_of(kcol), wq_lo = qlim_of(kw), wq_hi = qlim_of(kw + 31);
  // query tiles s + 64 j that reach the block's keys (queries >= kbase)
  const int j0 = kbase > a.s ? (kbase - a.s) / 64 : 0;
  const int nqt = (qlim_of(kbase + 127) - a.s + 63) / 64 - j0;
  const int n = nqt > 0 ? nqt * a.G : 0;
  // a block whose keys no query of the chunk sees has nothing to add
  if (n == 0 && a.beta) return;
  // K, V of the block's keys (rows past T fetch row T - 1; those keys are
  // masked and never written)
  const int kvalid = a.T - kbase;
  dma_tile64_w8<DH>(Kt, Kb, ldk, kvalid, wave, lane);
  dma_tile64_w8<DH>(Kt + TB, Kb + 64 * ldk, ldk, kvalid - 64, wave, lane);
  dma_tile64_w8<DH>(Vt, Vb, ldk, kvalid, wave, lane);
  dma_tile64_w8<DH>(Vt + TB, Vb + 64 * ldk, ldk, kvalid - 64, wave, lane);
  // each wave: 2 x (64 rows of Q and dO) / 8 waves, plus one quarter row of
  // LSE (waves 0-3) or Delta (waves 4-7)
  // Iteration it = hh nqt + jq: q head kv G + hh, query tile s + 64 (j0 +
  // jq).  Two cursors walk it without divisions: the next tile to fetch
  // (which stays on the last tile once there, so the trailing fetch repeats
  // it into a buffer nobody reads) and the next tile to compute.
  struct Cur {
    int hh, jq;
  };
  auto advance = [&](Cur& c) {
    if (++c.jq == nqt) {
      c.jq = 0;
      ++c.hh;
    }
  };
  Cur ct{0, 0};
  const Dma64Off<DH, 8> qoff(ldq, wave, lane);
  // The fetch cursor carries its Q / dO offset and its statistics row (LSE
  // for waves 0-3, Delta for 4-7): a tile step adds 64 rows, a head step
  // goes back to the first tile and on by one head.
  int fjq = 0, fq0 = a.s + j0 * 64, fetched = 0;  // fetched: tiles whose fetch has been issued
  int64_t fqo = (int64_t)b * a.q_bs + (int64_t)(fq0 - a.qoff) * ldq + (int64_t)kv * a.G * DH;
  const float* fst = wave < 4 ? a.lse + (int64_t)b * a.lse_sb + (int64_t)kv * a.G * a.lse_sh + j0 * 64
                              : a.delta + (int64_t)b * a.dl_sb + (int64_t)kv * a.G * a.dl_sh + j0 * 64;
  const int64_t fst_h = (wave < 4 ? a.lse_sh : a.dl_sh) - (int64_t)(nqt - 1) * 64;
  const int64_t fqo_h = (int64_t)DH - (int64_t)(nqt - 1) * 64 * ldq;
  auto issue = [&](char* qd, char* od, float* ld_, float* dd) {
    if (fetched > 0 && fetched < n) {
      if (++fjq == nqt) {
        fjq = 0;
        fq0 = a.s + j0 * 64;
        fqo += fqo_h;
        fst += fst_h;
      } else {
        fq0 += 64;
        fqo += 64 * ldq;
        fst += 64;
      }
    }
    ++fetched;
    if (a.e - fq0 >= 64) {  // wave-uniform
      dma_tile64_full<DH, 8>(qd, a.Q + fqo, qoff, wave);
      dma_tile64_full<DH, 8>(od, a.dO + fqo, qoff, wave);
    } else {
      dma_tile64_w8<DH>(qd, a.Q + fqo, ldq, a.e - fq0, wave, lane);
      dma_tile64_w8<DH>(od, a.dO + fqo, ldq, a.e - fq0, wave, lane);
    }
    dma_f32x16(wave < 4 ? ld_ : dd, fst, wave & 3, lane);
  };
  auto tile = [&](const char* qt, const char* ot, const float* ls, const float* dl) {
    const int q0 = a.s + (j0 + ct.jq) * 64, qw = q0 + qrow;
    advance(ct);
    // only the wave's queries at or after its keys and before the last
    // key's limit; those wholly after the keys and before every key's limit
    // need no mask
    if (qw + 31 >= kw && qw < wq_hi)
      dkdv_tile<DH>(lq, lk, smem, smem + 2 * TB, qt, ot, ls, dl, qrow, q0, kcol, qlim, lane, c2,
                    !(qw >= kw + 31 && qw + 32 <= wq_lo), dk, dv);
  };
  if (n > 0) issue(Q0, O0, L0, E0);
  for (int it = 0; it < n; it += 2) {
    dma_barrier();  // tile it (and K, V) landed; everyone is done with the other buffers
    issue(Q1, O1, L1, E1);  // tile it + 1 (or the last again)
    tile(Q0, O0, L0, E0);
    dma_barrier();
    issue(Q0, O0, L0, E0);  // tile it + 2 (or the last again)
    if (it + 1 < n) tile(Q1, O1, L1, E1);
  }
  __builtin_amdgcn_s_waitcnt(0);  // no DMA may still target LDS
  __syncthreads();                // every wave is done with K, V
  // query half 1 hands its partials to query half 0 through the K / V
  // arrays (one NB x 16 x 64 fp32 block per key group, in register order)
  float* red = reinterpret_cast<float*>((kg < 2 ? Kt : Vt) + (kg & 1) * TB);
#pragma unroll
  for (int round = 0; round < 2; ++round) {
    f32x16_t (&acc)[NB] = round == 0 ? dk : dv;
    if (qh == 1)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int e_ = 0; e_ < 16; ++e_) red[(nb * 16 + e_) * 64 + lane] = acc[nb][e_];
    __syncthreads();
    if (qh == 0)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int e_ = 0; e_ < 16; ++e_) acc[nb][e_] += red[(nb * 16 + e_) * 64 + lane];
    __syncthreads();
  }
  if (qh != 0) return;
  // result blocks [32 keys x 32 dh]: lane = dh column, rows = keys
  float* dKb = a.dK + ((int64_t)b * a.T) * ldk + (int64_t)kv * DH;
  float* dVb = a.dV + ((int64_t)b * a.T) * ldk + (int64_t)kv * DH;
  // beta: all 32 old values of a column block are loaded before any store,
  // so the loads are in flight together
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float ok[16], ov[16];
#pragma unroll
    for (int e_ = 0; e_ < 16; ++e_) {
      const int key = kw + crow(e_, lane);
      const int64_t off = (int64_t)key * ldk + nb * 32 + (lane & 31);
      const bool in = a.beta && key < a.T;
      ok[e_] = in ? dKb[off] : 0.f;
      ov[e_] = in ? dVb[off] : 0.f;
    }
#pragma unroll
    for (int e_ = 0; e_ < 16; ++e_) {
      const int key = kw + crow(e_, lane);
      if (key >= a.T) continue;
      const int64_t off = (int64_t)key * ldk + nb * 32 + (lane & 31);
      dKb[off] = ok[e_] + a.scale * dk[nb][e_];
      dVb[off] = ov[e_] + dv[nb][e_];
    }
  }
}

// ---------------------------------------------------------------------------
// dQ.  Block: 4 waves, 128 queries (32 per wave), one q head; key tiles of
// 64 up to the diagonal, double-buffered by DMA like the forward.
// ---------------------------------------------------------------------------
// s + the sum of the 8 bf16 values of an operand fragment: four bf16 dot
// products with (1, 1), each adding a word's two values (exact products,
// fp32 accumulation).
__device__ __forceinline__ float frag_sum(const uint4& u, float s) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  const bf16x2_t one = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
#pragma unroll
  for (int k = 0; k < 4; ++k) s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[k]), one, s, false);
  return s;
}

template <int DH, bool MASK>
__device__ __forceinline__ void dq_tile(const LdsOff<DH>& lo, const char* kt, const char* vt, int k0, int qcol,
                                        int klo, int lane, float c2, float lse2, float dl, const uint4 (&qf)[DH / 16],
                                        const uint4 (&of)[DH / 16], f32x16_t (&dq)[DH / 32], float& rs) {
  constexpr int NB = DH / 32, KS = DH / 16;
  f32x16_t st[2], dpt[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    st[kb] = f32x16_t{};
    dpt[kb] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      st[kb] = mma(lo.row_frag(kt, kb * 32, ks), qf[ks], st[kb]);
      dpt[kb] = mma(lo.row_frag(vt, kb * 32, ks), of[ks], dpt[kb]);
    }
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = k0 + kb * 32 + crow(e, lane);
      const float p = (!MASK || (key <= qcol && key >= klo)) ? __builtin_amdgcn_exp2f(st[kb][e] * c2 - lse2) : 0.f;
      dpt[kb][e] = p * (dpt[kb][e] - dl);
    }
  // dQ[q, dh] += dS[q, key] K[key, dh]; rs: this lane's share of the row sum
  // of dS as rounded to bf16 for the product
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 da = pack_frag(dpt[kb], i);
      rs = frag_sum(da, rs);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        dq[nb] = mma(da, lo.tr_frag(kt, kb * 32 + 16 * i, nb), dq[nb]);
    }
}

template <int DH>
__global__ __launch_bounds__(256, 2) void attn_dq_kernel(AttnArgs a) {
  constexpr int NB = DH / 32, KS = DH / 16;
  __shared__ __attribute__((aligned(16))) char K0[64 * DH * 2];
  __shared__ __attribute__((aligned(16))) char V0[64 * DH * 2];
  __shared__ __attribute__((aligned(16))) char K1[64 * DH * 2];
  __shared__ __attribute__((aligned(16))) char V1[64 * DH * 2];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const QBlock qbk = q_block(a.Hkv, a.G);
  const int h = qbk.h, b = blockIdx.z, kv = h / a.G;
  const LdsOff<DH> lo(lane);
  const int q0 = a.s + qbk.qblk * 128;
  const int qw = q0 + wave * 32;
  const int qcol = qw + (lane & 31);
  const int64_t ldq = a.ldq, ldk = (int64_t)a.Hkv * DH;
  const bf16_t* Qb = a.Q + (int64_t)b * a.q_bs + (int64_t)h * DH;   // row t at (t - qoff)
  const bf16_t* Ob = a.dO + (int64_t)b * a.q_bs + (int64_t)h * DH;
  const bf16_t* Kb = a.K + ((int64_t)b * a.T) * ldk + (int64_t)kv * DH;
  const bf16_t* Vb = a.V + ((int64_t)b * a.T) * ldk + (int64_t)kv * DH;
  const int qrel = qcol - a.qoff, qend = a.e - a.qoff;
  uint4 qf[KS], of[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = glb_frag<DH>(Qb, ldq, qrel, qend, ks, lane >> 5);
    of[ks] = glb_frag<DH>(Ob, ldq, qrel, qend, ks, lane >> 5);
  }
  const bool qok = qcol < a.e;
  const float c2 = a.scale * kLog2e;
  const float lse2 = qok ? a.lse[(int64_t)b * a.lse_sb + (int64_t)h * a.lse_sh + (int64_t)(qcol - a.s) * a.lse_st] : INFINITY;
  const float dl = qok ? a.delta[(int64_t)b * a.dl_sb + (int64_t)h * a.dl_sh + (int64_t)(qcol - a.s) * a.dl_st] : 0.f;
  f32x16_t dq[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) dq[i] = f32x16_t{};
  float rs = 0.f;

  const SeqRange sr = seq_range(a, q0, qw, qcol);
  const int kend = min(q0 + 128, a.e);
  const int ntiles = (kend + 63) / 64, t0 = sr.kfirst / 64;
  auto issue = [&](char* kd, char* vd, int t) {
    const int k0 = t * 64;
    dma_tile64<DH>(kd, Kb + (int64_t)k0 * ldk, ldk, kend - k0, wave, lane);
    dma_tile64<DH>(vd, Vb + (int64_t)k0 * ldk, ldk, kend - k0, wave, lane);
  };
  issue(K0, V0, t0);
  for (int t = t0; t < ntiles; t += 2) {
    dma_barrier();
    issue(K1, V1, min(t + 1, ntiles - 1));
    switch (sr.kind(t * 64)) {
      case 1: dq_tile<DH, false>(lo, K0, V0, t * 64, qcol, sr.klo, lane, c2, lse2, dl, qf, of, dq, rs); break;
      case 2: dq_tile<DH, true>(lo, K0, V0, t * 64, qcol, sr.klo, lane, c2, lse2, dl, qf, of, dq, rs); break;
      default: break;
    }
    dma_barrier();
    issue(K0, V0, min(t + 2, ntiles - 1));
    if (t + 1 < ntiles) switch (sr.kind((t + 1) * 64)) {
      case 1: dq_tile<DH, false>(lo, K1, V1, (t + 1) * 64, qcol, sr.klo, lane, c2, lse2, dl, qf, of, dq, rs); break;
      case 2: dq_tile<DH, true>(lo, K1, V1, (t + 1) * 64, qcol, sr.klo, lane, c2, lse2, dl, qf, of, dq, rs); break;
      default: break;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // no DMA may still target LDS
  __syncthreads();                // every wave's share of the last tile landed
  // Every row of dS sums to zero (sum_j P_ij dP_ij = rowsum(dO O) = Delta_i),
  // so dQ_i = s sum_j dS_ij (K_j - c) for any vector c.  The product above
  // used dS rounded to bf16, whose row sums rs_i are not zero; where K has a
  // large component shared by the keys a row attends to, that rounding is
  // amplified.  Subtract rs_i c with c the mean of the block's last key tile
  // (the diagonal keys, which the loop leaves in both buffers; rows past the
  // block's last key repeat that key -- any constant c is exact): as an MFMA
  // with A = -rs_i / 64 on every row of the tile.
  rs += __shfl_xor(rs, 32, 64);
  {
    const uint32_t w = pk_bf16(-rs * (1.f / 64.f), -rs * (1.f / 64.f));
    const uint4 ca = make_uint4(w, w, w, w);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) dq[nb] = mma(ca, lo.tr_frag(K0, kb * 32 + 16 * i, nb), dq[nb]);
  }
  // result blocks [32 queries x 32 dh]: lane = dh column, rows = queries
  bf16_t* dQb = a.dQ + (int64_t)b * a.q_bs / ldq * a.lddq + (int64_t)h * DH;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int q = qw + crow(e, lane);
      if (q >= a.e) continue;
      dQb[(int64_t)(q - a.qoff) * a.lddq + nb * 32 + (lane & 31)] = f2bf(a.scale * dq[nb][e]);
    }
}

// ---------------------------------------------------------------------------
// Host launchers (shared with the decoder layer).
// ---------------------------------------------------------------------------
static double attn_pairs(int s, int e) {
  // (query, key) pairs with key <= query for queries [s, e)
  return 0.5 * ((double)e * (e + 1) - (double)s * (s + 1));
}

sbp_status attn_fwd(const AttnArgs& a, int dh, int B, hipStream_t st) {
  const int Tc = a.e - a.s;
  dim3 grid((unsigned)cdiv(Tc, 128), (unsigned)a.Hq, (unsigned)B);
  ProfScope prof("attn_fwd", st, 4.0 * dh * a.Hq * B * attn_pairs(a.s, a.e), 0.0);
  if (dh == 128)
    hipLaunchKernelGGL(attn_fwd_kernel<128>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<64>, grid, dim3(256), 0, st, a);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

sbp_status attn_delta(const AttnArgs& a, const void* O, const float* lse_src, int64_t lsb,
                      int64_t lst, int dh, int B, hipStream_t st) {
  const int Tc = a.e - a.s;
  const int64_t rows = (int64_t)Tc * a.Hq;
  dim3 grid((unsigned)cdiv(rows, 4), (unsigned)B);
  ProfScope prof("attn_delta", st, 0.0, 4.0 * rows * B * dh);
  if (dh == 128)
    hipLaunchKernelGGL(attn_delta_kernel<128>, grid, dim3(256), 0, st, a, (const bf16_t*)O, lse_src, lsb, lst);
  else
    hipLaunchKernelGGL(attn_delta_kernel<64>, grid, dim3(256), 0, st, a, (const bf16_t*)O, lse_src, lsb, lst);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

sbp_status attn_bwd_chunk(const AttnArgs& a, int dh, int B, hipStream_t st) {
  const double pairs = attn_pairs(a.s, a.e) * a.Hq * B;
  {
    dim3 grid((unsigned)cdiv(a.e, 128), (unsigned)a.Hkv, (unsigned)B);
    ProfScope prof("attn_dkdv", st, 8.0 * dh * pairs, 0.0);
    if (dh == 128)
      hipLaunchKernelGGL(attn_dkdv_kernel<128>, grid, dim3(512), 0, st, a);
    else
      hipLaunchKernelGGL(attn_dkdv_kernel<64>, grid, dim3(512), 0, st, a);
    SBP_LAUNCH_CHECK();
  }
  {
    dim3 grid((unsigned)cdiv(a.e - a.s, 128), (unsigned)a.Hq, (unsigned)B);
    ProfScope prof("attn_dq", st, 6.0 * dh * pairs, 0.0);
    if (dh == 128)
      hipLaunchKernelGGL(attn_dq_kernel<128>, grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(attn_dq_kernel<64>, grid, dim3(256), 0, st, a);
    SBP_LAUNCH_CHECK();
  }
  return SBP_OK;
}

// seq_lo[t], seq_hi[t]: bounds of the packed sequence holding token t, the
// last n with cu[n] <= t by bisection over cu[0 .. nseq - 1]; clamped so
// that seq_lo[t] <= t < seq_hi[t] <= T for any cu.
__global__ __launch_bounds__(256) void seq_bounds_kernel(const int32_t* __restrict__ cu, int nseq,
                                                         int64_t T, int* __restrict__ lo,
                                                         int* __restrict__ hi) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  int a = 0, b = nseq;  // the answer lies in [a, b)
  while (b - a > 1) {
    const int m = (a + b) >> 1;
    if (cu[m] <= t) a = m;
    else b = m;
  }
  const int64_t l = cu[a], h = cu[a + 1];
  lo[t] = (int)(l < 0 ? 0 : (l > t ? t : l));
  hi[t] = (int)(h <= t ? t + 1 : (h > T ? T : h));
}

sbp_status attn_seq_bounds(const int32_t* cu, int nseq, int64_t T, int* seq_lo, int* seq_hi,
                           hipStream_t st) {
  ProfScope prof("attn_seq_bounds", st, 0.0, 8.0 * T);
  hipLaunchKernelGGL(seq_bounds_kernel, dim3((unsigned)cdiv(T, 256)), dim3(256), 0, st, cu, nseq, T,
                     seq_lo, seq_hi);
  SBP_LAUNCH_CHECK();
  return SBP_OK;
}

namespace {

inline bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

sbp_status attn_check(int64_t B, int64_t T, int32_t Hq, int32_t Hkv, int32_t dh, int32_t D,
                      int32_t dtype) {
  if (dtype != SBP_F32 && dtype != SBP_BF16) return set_error(SBP_ERR_INVALID_ARG, "dtype %d is not SBP_F32 or SBP_BF16", dtype);
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || dh < 1) return set_error(SBP_ERR_INVALID_ARG, "B, T, Hq, Hkv, dh must be >= 1");
  if (D < 1 || D > T) return set_error(SBP_ERR_INVALID_ARG, "need 1 <= D <= T (D=%d, T=%lld)", D, (long long)T);
  if (Hq % Hkv) return set_error(SBP_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (dh != 64 && dh != 128) return set_error(SBP_ERR_UNSUPPORTED, "head dim %d not supported (64 or 128)", dh);
  if (T > (1ll << 30) || B > 65535 || Hq > 65535) return set_error(SBP_ERR_UNSUPPORTED, "size out of supported range");
  return SBP_OK;
}

size_t attn_ws(int64_t B, int64_t T, int32_t Hq, int32_t dh, int32_t D, int32_t dtype) {
  (void)dh;
  (void)dtype;
  // per query chunk: LSE_c and Delta_c, fp32 [B, Hq, Lp]
  const int64_t Lp = attn_stats_pitch(max_chunk_len(T, D));
  WsPlan P;
  P.take(sizeof(float) * B * Lp * Hq);
  P.take(sizeof(float) * B * Lp * Hq);
  return round_up((int64_t)P.off, 256);
}

// as attn_ws for B = 1, then seq_lo and seq_hi [T] int32, each 256-aligned
size_t packed_ws(int64_t T, int32_t Hq, int32_t dh, int32_t D, int32_t dtype) {
  return attn_ws(1, T, Hq, dh, D, dtype) + 2 * round_up((int64_t)sizeof(int) * T, 256);
}

// Both entry points: argument checks, then per query chunk in reverse order
// the forward statistics (or Delta from a given O) and the backward.
sbp_status attn_run(const void* Q, const void* K, const void* V, const void* dO, const void* O,
                    const float* lse, const int32_t* cu, int32_t nseq, int64_t B, int64_t T,
                    int32_t Hq, int32_t Hkv, int32_t dh, float scale, int32_t D, int32_t dtype,
                    int32_t accumulate, void* dQ, float* dK, float* dV, void* ws, size_t ws_bytes,
                    hipStream_t str) {
  sbp_status st = attn_check(B, T, Hq, Hkv, dh, D, dtype);
  if (st != SBP_OK) return st;
  if (!Q || !K || !V || !dO || !dQ || !dK || !dV)
    return set_error(SBP_ERR_INVALID_ARG, "Q, K, V, dO, dQ, dK and dV must be non-NULL");
  if ((O == nullptr) != (lse == nullptr))
    return set_error(SBP_ERR_INVALID_ARG, "O and lse must be given together or not at all");
  if (misaligned(Q) || misaligned(K) || misaligned(V) || misaligned(dO) || misaligned(O) ||
      misaligned(lse) || misaligned(dQ) || misaligned(dK) || misaligned(dV) || misaligned(ws))
    return set_error(SBP_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  if (!(scale > 0.f) || !(scale < 1e30f)) return set_error(SBP_ERR_INVALID_ARG, "scale must be positive and finite");
  const size_t need = cu ? packed_ws(T, Hq, dh, D, dtype) : attn_ws(B, T, Hq, dh, D, dtype);
  if (!ws || ws_bytes < need)
    return set_error(SBP_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
  const int64_t Lp = attn_stats_pitch(max_chunk_len(T, D));
  WsPlan P;
  P.base = (char*)ws;
  float* w_lse = (float*)P.take(sizeof(float) * B * Lp * Hq);
  float* w_dl = (float*)P.take(sizeof(float) * B * Lp * Hq);
  int* seq_lo = nullptr;
  int* seq_hi = nullptr;
  if (cu) {
    seq_lo = (int*)P.take(sizeof(int) * T);
    seq_hi = (int*)P.take(sizeof(int) * T);
    st = attn_seq_bounds(cu, nseq, T, seq_lo, seq_hi, str);
    if (st != SBP_OK) return st;
  }
  for (int32_t c = D - 1; c >= 0; --c) {
    int64_t s0, e0;
    chunk_bounds(T, D, c, &s0, &e0);
    AttnArgs a;
    a.Q = (const bf16_t*)Q; a.K = (const bf16_t*)K; a.V = (const bf16_t*)V;
    a.dO = (const bf16_t*)dO; a.O = nullptr; a.dQ = (bf16_t*)dQ; a.dK = dK; a.dV = dV;
    a.ldq = (int64_t)Hq * dh; a.lddq = a.ldq; a.q_bs = T * a.ldq; a.qoff = 0;
    a.T = (int)T; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv;
    a.s = (int)s0; a.e = (int)e0;
    a.scale = scale;
    // the last chunk (processed first) reaches every key: it overwrites
    a.beta = (accumulate || c != D - 1) ? 1 : 0;
    a.delta = w_dl; a.dl_sb = (int64_t)Hq * Lp; a.dl_sh = Lp; a.dl_st = 1;
    a.lse = w_lse; a.lse_sb = (int64_t)Hq * Lp; a.lse_sh = Lp; a.lse_st = 1;
    a.seq_lo = seq_lo; a.seq_hi = seq_hi;
    const bool f32 = dtype == SBP_F32;  // the pointers then hold fp32 arrays
    if (lse) {
      // caller's O and LSE ([B, T, Hq]): Delta, and LSE copied into the chunk layout
      st = f32 ? attn_delta_f32(a, O, lse, T * Hq, Hq, dh, (int)B, str)
               : attn_delta(a, O, lse, T * Hq, Hq, dh, (int)B, str);
    } else {
      st = f32 ? attn_fwd_f32(a, dh, (int)B, str) : attn_fwd(a, dh, (int)B, str);
    }
    if (st != SBP_OK) return st;
    st = f32 ? attn_bwd_chunk_f32(a, dh, (int)B, str) : attn_bwd_chunk(a, dh, (int)B, str);
    if (st != SBP_OK) return st;
  }
  return SBP_OK;
}

}  // namespace

sbp_status attn_bwd_ws_size(int64_t B, int64_t T, int32_t Hq, int32_t Hkv, int32_t dh, int32_t D,
                            int32_t dtype, size_t* bytes) {
  sbp_status st = attn_check(B, T, Hq, Hkv, dh, D, dtype);
  if (st == SBP_OK) *bytes = attn_ws(B, T, Hq, dh, D, dtype);
  return st;
}

sbp_status attn_bwd_run(const void* Q, const void* K, const void* V, const void* dO, const void* O,
                        const float* lse, int64_t B, int64_t T, int32_t Hq, int32_t Hkv, int32_t dh,
                        float scale, int32_t D, int32_t dtype, int32_t accumulate, void* dQ,
                        float* dK, float* dV, void* ws, size_t ws_bytes, hipStream_t str) {
  return attn_run(Q, K, V, dO, O, lse, nullptr, 0, B, T, Hq, Hkv, dh, scale, D, dtype, accumulate,
                  dQ, dK, dV, ws, ws_bytes, str);
}

}  // namespace sbp

using namespace sbp;

extern "C" sbp_status sbp_attn_bwd_workspace_size(int64_t B, int64_t T, int32_t Hq, int32_t Hkv,
                                                  int32_t dh, int32_t D, int32_t dtype,
                                                  size_t* bytes) {
  clear_error();
  if (!bytes) return set_error(SBP_ERR_INVALID_ARG, "bytes is NULL");
  sbp_status st = attn_check(B, T, Hq, Hkv, dh, D, dtype);
  if (st != SBP_OK) return st;
  *bytes = attn_ws(B, T, Hq, dh, D, dtype);
  return SBP_OK;
}

extern "C" sbp_status sbp_attn_bwd_chunked(const void* Q, const void* K, const void* V,
                                           const void* dO, const void* O, const float* lse,
                                           int64_t B, int64_t T, int32_t Hq, int32_t Hkv,
                                           int32_t dh, float scale, int32_t D, int32_t dtype,
                                           int32_t accumulate, void* dQ, float* dK, float* dV,
                                           void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  const sbp_status st = attn_run(Q, K, V, dO, O, lse, nullptr, 0, B, T, Hq, Hkv, dh, scale, D,
                                 dtype, accumulate, dQ, dK, dV, ws, ws_bytes, (hipStream_t)stream);
  return st == SBP_OK ? debug_sync((hipStream_t)stream, "sbp_attn_bwd_chunked") : st;
}

extern "C" sbp_status sbp_attn_bwd_packed_workspace_size(int64_t T, int32_t Hq, int32_t Hkv,
                                                         int32_t dh, int32_t D, int32_t dtype,
                                                         size_t* bytes) {
  clear_error();
  if (!bytes) return set_error(SBP_ERR_INVALID_ARG, "bytes is NULL");
  sbp_status st = attn_check(1, T, Hq, Hkv, dh, D, dtype);
  if (st != SBP_OK) return st;
  *bytes = packed_ws(T, Hq, dh, D, dtype);
  return SBP_OK;
}

extern "C" sbp_status sbp_attn_bwd_packed(const void* Q, const void* K, const void* V,
                                          const void* dO, const void* O, const float* lse,
                                          const int32_t* cu_seqlens, int32_t nseq, int64_t T,
                                          int32_t Hq, int32_t Hkv, int32_t dh, float scale,
                                          int32_t D, int32_t dtype, int32_t accumulate, void* dQ,
                                          float* dK, float* dV, void* ws, size_t ws_bytes,
                                          void* stream) {
  clear_error();
  if (!cu_seqlens) return set_error(SBP_ERR_INVALID_ARG, "cu_seqlens must be non-NULL");
  if (nseq < 1) return set_error(SBP_ERR_INVALID_ARG, "nseq must be >= 1 (got %d)", nseq);
  if (misaligned(cu_seqlens)) return set_error(SBP_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  sbp_status st = debug_check_cu(cu_seqlens, nseq, T, (hipStream_t)stream);
  if (st != SBP_OK) return st;
  st = attn_run(Q, K, V, dO, O, lse, cu_seqlens, nseq, 1, T, Hq, Hkv, dh, scale, D, dtype,
                accumulate, dQ, dK, dV, ws, ws_bytes, (hipStream_t)stream);
  return st == SBP_OK ? debug_sync((hipStream_t)stream, "sbp_attn_bwd_packed") : st;
}
