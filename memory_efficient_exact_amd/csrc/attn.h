// Internal interface of the attention kernels (shared by the attention
// entry point and the decoder layer).
#pragma once

#include "common.h"

namespace sbp {

struct AttnArgs {
  // Query-side arrays (Q, dO, O, dQ) hold rows t - qoff of batch row b at
  // p + b * q_bs + (t - qoff) * ld + head * dh: the whole sequence
  // (qoff = 0, q_bs = T * ld) or just the current chunk (qoff = s).
  const bf16_t* Q;   // [B, T, Hq, dh]
  const bf16_t* K;   // [B, T, Hkv, dh]
  const bf16_t* V;
  const bf16_t* dO;  // [B, T, Hq, dh] (may be null for the forward)
  bf16_t* O;         // forward output (optional) [B, T, Hq, dh]
  bf16_t* dQ;        // [B, T, Hq, dh]
  float* dK;         // [B, T, Hkv, dh]
  float* dV;
  // per-row statistics of the chunk: element (b, h, t) at
  // base + b*sb + h*sh + (t - s)*st   (t absolute, s = chunk start).
  // lse holds the log-sum-exp of the scaled scores in base-2 units
  // (natural-log LSE times log2 e), as the kernels evaluate exp2.
  float* lse;
  int64_t lse_sb, lse_sh, lse_st;
  float* delta;
  int64_t dl_sb, dl_sh, dl_st;
  int64_t ldq;       // row pitch of Q, dO, O
  int64_t lddq;      // row pitch of dQ
  int64_t q_bs;      // batch stride of the query-side arrays
  int qoff;
  int T, Hq, Hkv, G;
  int s, e;          // chunk [s, e)
  float scale;
  int beta;          // dK/dV: 1 = add into, 0 = overwrite
  // Packed independent sequences (B = 1 only): token t belongs to the
  // sequence [seq_lo[t], seq_hi[t]) (seq_lo[t] <= t < seq_hi[t] <= T), and
  // query i sees key j iff seq_lo[i] <= j <= i.  NULL: the whole row is one
  // sequence.
  const int* seq_lo = nullptr;
  const int* seq_hi = nullptr;
};

// Per query chunk [a.s, a.e): forward statistics (LSE always; Delta when
// a.dO is set; O when a.O is set), Delta from a given O, and the backward
// (dK/dV accumulate into fp32, dQ overwritten).
sbp_status attn_fwd(const AttnArgs& a, int dh, int B, hipStream_t st);
// Delta from a given O; when lse_src is set also copies LSE (element (b, t, h)
// at lse_src + b * lsb + t * lst + h) into the statistics layout of a.lse.
sbp_status attn_delta(const AttnArgs& a, const void* O, const float* lse_src, int64_t lsb,
                      int64_t lst, int dh, int B, hipStream_t st);

// Row pitch (floats) of per-chunk LSE / Delta rows: the chunk length padded
// so that a 64-row fetch starting at any 64-aligned row stays in bounds.
inline int64_t attn_stats_pitch(int64_t Tcm) { return round_up(Tcm, 64) + 64; }
sbp_status attn_bwd_chunk(const AttnArgs& a, int dh, int B, hipStream_t st);
// seq_lo / seq_hi [T] of packed sequences from their boundaries cu[0..nseq]
// (clamped so that seq_lo[t] <= t < seq_hi[t] <= T whatever cu holds).
sbp_status attn_seq_bounds(const int32_t* cu, int nseq, int64_t T, int* seq_lo, int* seq_hi,
                           hipStream_t st);

// fp32 mode (attn_f32.hip): the same three steps with AttnArgs whose array
// pointers hold fp32 data (Q, K, V, dO, O, dQ), every product an fp32 FMA.
sbp_status attn_fwd_f32(const AttnArgs& a, int dh, int B, hipStream_t st);
sbp_status attn_delta_f32(const AttnArgs& a, const void* O, const float* lse_src, int64_t lsb,
                          int64_t lst, int dh, int B, hipStream_t st);
sbp_status attn_bwd_chunk_f32(const AttnArgs& a, int dh, int B, hipStream_t st);

// The chunked attention backward of sbp_attn_bwd_chunked on a given
// workspace (every argument checked first), and the size that workspace
// needs (SBP_OK and *bytes set, or an argument error).
sbp_status attn_bwd_ws_size(int64_t B, int64_t T, int32_t Hq, int32_t Hkv, int32_t dh, int32_t D,
                            int32_t dtype, size_t* bytes);
sbp_status attn_bwd_run(const void* Q, const void* K, const void* V, const void* dO, const void* O,
                        const float* lse, int64_t B, int64_t T, int32_t Hq, int32_t Hkv, int32_t dh,
                        float scale, int32_t D, int32_t dtype, int32_t accumulate, void* dQ,
                        float* dK, float* dV, void* ws, size_t ws_bytes, hipStream_t str);

}  // namespace sbp
