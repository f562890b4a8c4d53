// fp32 mode of the decoder layer: streamed backward and chunked forward.
//
// The same layer and the same chunk schedule as layer.hip (skill page,
// "Implementation": per chunk, forward recompute, backward, weight gradients
// added, input gradient kept; keys/values of the whole prefix formed once,
// chunks in reverse order so a chunk's dK/dV are final when its projection
// gradients are taken), with every tensor and product in fp32: the fp32
// GEMM (gemm_nt, 128 x 128 tiles of fp32 MFMA), the fp32 attention kernels
// (attn_f32.hip) and the fp32 instances of the token-wise kernels.  Weight
// gradients contract over the chunk's tokens; the fp32 GEMM reads row-major
// operands only, so both activations of such a product are transposed into
// [features, T_c rounded to 32] slots (zero past T_c) first.
#include "attn.h"
#include "common.h"
#include "kernels.h"

namespace sbp {
namespace {

struct F32Shape {
  int64_t T, d, F, qd, kd, qkvd;
  int Hq, Hkv, dh;
  int32_t D;
  int64_t R, Rp;  // longest chunk, and rounded up to the fp32 GEMM's K granule
  int64_t tw;     // rows of the transpose slots
  float eps, rope_theta;
  bool qk_norm;
};

F32Shape f32_shape(const sbp_layer_desc* L, int32_t D) {
  F32Shape s;
  s.T = L->T; s.d = L->d; s.F = L->F;
  s.Hq = L->Hq; s.Hkv = L->Hkv; s.dh = L->dh;
  s.qd = (int64_t)L->Hq * L->dh;
  s.kd = (int64_t)L->Hkv * L->dh;
  s.qkvd = s.qd + 2 * s.kd;
  s.D = D;
  s.R = max_chunk_len(L->T, D);
  s.Rp = round_up(s.R, gemm_k_granule(SBP_F32));
  s.tw = std::max<int64_t>(std::max<int64_t>(2 * s.F, s.qkvd), s.d);
  s.eps = L->eps;
  s.rope_theta = L->rope_theta;
  s.qk_norm = L->qk_norm != 0;
  return s;
}

struct F32Ws {
  float *Kall, *Vall, *dKacc, *dVacc;
  float *W2T, *W13T, *WoT, *WqkvT;
  float *h1, *q, *o, *a, *n2, *ug, *m, *dm, *dudg, *da, *dov, *dqkv, *dn;
  float *tA, *tB;
  float *rinv1, *rinv2, *lse, *delta, *gpart;
  int *seq_lo, *seq_hi;
  float2* rope_tab;
  float *Kraw, *qraw, *hnpart;
};

// bwd: the backward plan; otherwise the forward's (no gradients, no
// weight transposes, no transpose slots)
size_t f32_plan(const F32Shape& s, bool bwd, bool packed, char* base, F32Ws* w) {
  WsPlan P;
  P.base = base;
  F32Ws x = {};
  const size_t f4 = sizeof(float);
  const int64_t R = s.R;
  x.Kall = (float*)P.take(f4 * s.T * s.kd);
  x.Vall = (float*)P.take(f4 * s.T * s.kd);
  if (bwd) {
    x.dKacc = (float*)P.take(f4 * s.T * s.kd);
    x.dVacc = (float*)P.take(f4 * s.T * s.kd);
    x.W2T = (float*)P.take(f4 * s.F * s.d);
    x.W13T = (float*)P.take(f4 * s.d * 2 * s.F);
    x.WoT = (float*)P.take(f4 * s.qd * s.d);
    x.WqkvT = (float*)P.take(f4 * s.d * s.qkvd);
  }
  x.h1 = (float*)P.take(f4 * R * s.d);
  x.q = (float*)P.take(f4 * R * s.qd);
  x.o = (float*)P.take(f4 * R * s.qd);
  x.a = (float*)P.take(f4 * R * s.d);
  x.n2 = (float*)P.take(f4 * R * s.d);
  x.ug = (float*)P.take(f4 * R * 2 * s.F);
  x.m = (float*)P.take(f4 * R * s.F);
  if (bwd) {
    x.dm = (float*)P.take(f4 * R * s.F);
    x.dudg = (float*)P.take(f4 * R * 2 * s.F);
    x.da = (float*)P.take(f4 * R * s.d);
    x.dov = (float*)P.take(f4 * R * s.qd);
    x.dqkv = (float*)P.take(f4 * R * s.qkvd);
    x.dn = (float*)P.take(f4 * R * s.d);
    x.tA = (float*)P.take(f4 * s.tw * s.Rp);
    x.tB = (float*)P.take(f4 * s.tw * s.Rp);
    x.gpart = (float*)P.take(f4 * gain_grad_splits(R) * s.d);
  }
  x.rinv1 = (float*)P.take(f4 * R);
  x.rinv2 = (float*)P.take(f4 * R);
  x.lse = (float*)P.take(f4 * attn_stats_pitch(R) * s.Hq);
  x.delta = (float*)P.take(f4 * attn_stats_pitch(R) * s.Hq);
  x.seq_lo = packed ? (int*)P.take(sizeof(int) * s.T) : nullptr;
  x.seq_hi = packed ? (int*)P.take(sizeof(int) * s.T) : nullptr;
  x.rope_tab = s.rope_theta > 0.f ? (float2*)P.take(sizeof(float2) * s.T * (s.dh / 2)) : nullptr;
  x.Kraw = s.qk_norm ? (float*)P.take(f4 * s.T * s.kd) : nullptr;
  x.qraw = s.qk_norm ? (float*)P.take(f4 * R * s.qd) : nullptr;
  x.hnpart = s.qk_norm && bwd ? (float*)P.take(f4 * HEADNORM_PARTS * s.dh) : nullptr;
  if (w) *w = x;
  return round_up((int64_t)P.off, 256);
}

#define SBP_TRY(e_)                  \
  do {                               \
    sbp_status _s = (e_);            \
    if (_s != SBP_OK) return _s;     \
  } while (0)

// C[M, N] (op)= A[M, K] B[N, K]^T, fp32
sbp_status mm(const float* A, int64_t lda, const float* B, int64_t ldb, float* C, int64_t ldc,
              int64_t M, int64_t N, int64_t K, int epi, int beta, const float* R, int64_t ldr,
              const char* name, hipStream_t st) {
  GemmParams p;
  p.A = A; p.lda = lda; p.B = B; p.ldb = ldb; p.C = C; p.ldc = ldc; p.R = R; p.ldr = ldr;
  p.M = (int)M; p.N = (int)N; p.K = (int)K; p.beta = beta;
  return gemm_nt(SBP_F32, epi, p, GEMM_TILE_128, st, name);
}

// dst[c][r] = src[r][c] for r < rows, zero up to rows_pad
sbp_status tr(const float* src, int64_t ld_src, int64_t rows, int64_t cols, float* dst,
              int64_t ld_dst, int64_t rows_pad, hipStream_t st) {
  return transpose_pad(SBP_F32, src, ld_src, rows, cols, dst, ld_dst, rows_pad, nullptr, st);
}

// rows x cols fp32 block copy between pitched arrays
sbp_status copy_rows(const float* src, int64_t ld_src, int64_t rows, int64_t cols, float* dst,
                     int64_t ld_dst, hipStream_t st) {
  SBP_HIP_CHECK(hipMemcpy2DAsync(dst, ld_dst * sizeof(float), src, ld_src * sizeof(float),
                                 cols * sizeof(float), rows, hipMemcpyDeviceToDevice, st));
  return SBP_OK;
}

// h1 = RMSNorm(x_c); k (before its norm, when QK-norm) and v of the chunk
sbp_status f32_keys(const F32Shape& S, const F32Ws& W, const float* xc, const sbp_layer_weights* w,
                    int64_t s0, int64_t Tc, hipStream_t st) {
  const int64_t d = S.d, kd = S.kd;
  SBP_TRY(rmsnorm_fwd(xc, d, w->g1, Tc, d, S.eps, W.h1, d, W.rinv1, st, SBP_F32));
  float* kdst = (S.qk_norm ? W.Kraw : W.Kall) + s0 * kd;
  SBP_TRY(mm(W.h1, d, (const float*)w->Wk, d, kdst, kd, Tc, kd, d, EPI_OUT, 0, nullptr, 0, "gemm_layer_fwd", st));
  SBP_TRY(mm(W.h1, d, (const float*)w->Wv, d, W.Vall + s0 * kd, kd, Tc, kd, d, EPI_OUT, 0, nullptr, 0, "gemm_layer_fwd", st));
  if (S.qk_norm)
    SBP_TRY(headnorm_fwd(W.Kraw + s0 * kd, kd, W.Kall + s0 * kd, kd, Tc, S.Hkv, S.dh, w->kn, S.eps, st, SBP_F32));
  if (W.rope_tab)
    SBP_TRY(rope_apply(W.Kall + s0 * kd, true, kd, W.Kall + s0 * kd, kd, Tc, S.Hkv, S.dh, s0,
                       W.seq_lo, W.rope_tab, false, st, true));
  return SBP_OK;
}

// the chunk's queries (h1 already formed), attention forward (o, LSE), a,
// n2, [u | g], m
sbp_status f32_chunk_fwd(const F32Shape& S, const F32Ws& W, const float* xc,
                         const sbp_layer_weights* w, int64_t s0, int64_t e0, AttnArgs& at,
                         hipStream_t st) {
  const int64_t d = S.d, F = S.F, qd = S.qd, Tc = e0 - s0;
  float* qdst = S.qk_norm ? W.qraw : W.q;
  SBP_TRY(mm(W.h1, d, (const float*)w->Wq, d, qdst, qd, Tc, qd, d, EPI_OUT, 0, nullptr, 0, "gemm_layer_fwd", st));
  if (S.qk_norm) SBP_TRY(headnorm_fwd(W.qraw, qd, W.q, qd, Tc, S.Hq, S.dh, w->qn, S.eps, st, SBP_F32));
  if (W.rope_tab)
    SBP_TRY(rope_apply(W.q, true, qd, W.q, qd, Tc, S.Hq, S.dh, s0, W.seq_lo, W.rope_tab, false, st, true));
  at.Q = (const bf16_t*)W.q; at.K = (const bf16_t*)W.Kall; at.V = (const bf16_t*)W.Vall;
  at.dO = nullptr; at.O = (bf16_t*)W.o;
  const int64_t Lp = attn_stats_pitch(S.R);
  at.lse = W.lse; at.lse_sb = 0; at.lse_sh = Lp; at.lse_st = 1;
  at.delta = W.delta; at.dl_sb = 0; at.dl_sh = Lp; at.dl_st = 1;
  at.ldq = qd; at.q_bs = 0; at.qoff = (int)s0;
  at.T = (int)S.T; at.Hq = S.Hq; at.Hkv = S.Hkv; at.G = S.Hq / S.Hkv;
  at.s = (int)s0; at.e = (int)e0; at.scale = 1.0f / sqrtf((float)S.dh);
  at.seq_lo = W.seq_lo; at.seq_hi = W.seq_hi;
  SBP_TRY(attn_fwd_f32(at, S.dh, 1, st));
  SBP_TRY(mm(W.o, qd, (const float*)w->Wo, qd, W.a, d, Tc, d, qd, EPI_OUT_RESID, 0, xc, d, "gemm_layer_fwd", st));
  SBP_TRY(rmsnorm_fwd(W.a, d, w->g2, Tc, d, S.eps, W.n2, d, W.rinv2, st, SBP_F32));
  SBP_TRY(mm(W.n2, d, (const float*)w->W1, d, W.ug, 2 * F, Tc, F, d, EPI_OUT, 0, nullptr, 0, "gemm_layer_fwd", st));
  SBP_TRY(mm(W.n2, d, (const float*)w->W3, d, W.ug + F, 2 * F, Tc, F, d, EPI_OUT, 0, nullptr, 0, "gemm_layer_fwd", st));
  SBP_TRY(swiglu_fwd(W.ug, Tc, F, W.m, st, SBP_F32));
  return SBP_OK;
}

}  // namespace

size_t layer_f32_ws(const sbp_layer_desc* L, int32_t D, bool bwd, bool packed) {
  return f32_plan(f32_shape(L, D), bwd, packed, nullptr, nullptr);
}

sbp_status layer_f32_bwd(const sbp_layer_desc* desc, const int32_t* cu, int32_t nseq, const void* x,
                         const void* dy, const sbp_layer_weights* w, int32_t D, int32_t accumulate,
                         void* dx, sbp_layer_grads* g, void* ws, hipStream_t st) {
  const F32Shape S = f32_shape(desc, D);
  F32Ws W;
  f32_plan(S, true, cu != nullptr, (char*)ws, &W);
  const int64_t d = S.d, F = S.F, qd = S.qd, kd = S.kd, qkvd = S.qkvd, Rp = S.Rp;
  const float* X = (const float*)x;
  const float* DY = (const float*)dy;
  float* DX = (float*)dx;

  // G[M, N] (+)= A^T B over Tc tokens, A [Tc, M] (pitch lda), B [Tc, N]
  auto wg = [&](const float* A, int64_t lda, const float* B, int64_t ldb, float* G, int64_t M,
                int64_t N, int64_t Tc, int beta) -> sbp_status {
    SBP_TRY(tr(A, lda, Tc, M, W.tA, Rp, Rp, st));
    SBP_TRY(tr(B, ldb, Tc, N, W.tB, Rp, Rp, st));
    return mm(W.tA, Rp, W.tB, Rp, G, N, M, N, Rp, EPI_F32_ACC, beta, nullptr, 0, "gemm_layer_dW", st);
  };

  // weight transposes for the products that contract over a weight's rows
  SBP_TRY(tr((const float*)w->W2, F, d, F, W.W2T, d, d, st));
  SBP_TRY(tr((const float*)w->W1, d, F, d, W.W13T, 2 * F, F, st));
  SBP_TRY(tr((const float*)w->W3, d, F, d, W.W13T + F, 2 * F, F, st));
  SBP_TRY(tr((const float*)w->Wo, qd, d, qd, W.WoT, d, d, st));
  SBP_TRY(tr((const float*)w->Wq, d, qd, d, W.WqkvT, qkvd, qd, st));
  SBP_TRY(tr((const float*)w->Wk, d, kd, d, W.WqkvT + qd, qkvd, kd, st));
  SBP_TRY(tr((const float*)w->Wv, d, kd, d, W.WqkvT + qd + kd, qkvd, kd, st));
  if (cu) SBP_TRY(attn_seq_bounds(cu, nseq, S.T, W.seq_lo, W.seq_hi, st));
  if (W.rope_tab) SBP_TRY(rope_table(W.rope_tab, S.T, S.dh, (double)S.rope_theta, st));

  // pass F: keys and values of every token
  for (int32_t c = 0; c < D; ++c) {
    int64_t s0, e0;
    chunk_bounds(S.T, D, c, &s0, &e0);
    SBP_TRY(f32_keys(S, W, X + s0 * d, w, s0, e0 - s0, st));
  }

  for (int32_t c = D - 1; c >= 0; --c) {
    int64_t s0, e0;
    chunk_bounds(S.T, D, c, &s0, &e0);
    const int64_t Tc = e0 - s0;
    const int wb = (c == D - 1) ? (accumulate ? 1 : 0) : 1;  // weight-gradient beta
    const float* xc = X + s0 * d;
    const float* dyc = DY + s0 * d;

    // ---- recompute the chunk's forward ----
    SBP_TRY(rmsnorm_fwd(xc, d, w->g1, Tc, d, S.eps, W.h1, d, W.rinv1, st, SBP_F32));
    AttnArgs at;
    SBP_TRY(f32_chunk_fwd(S, W, xc, w, s0, e0, at, st));

    // ---- MLP backward ----
    SBP_TRY(wg(dyc, d, W.m, F, g->W2, d, F, Tc, wb));                                    // dW2 += dy^T m
    SBP_TRY(mm(dyc, d, W.W2T, d, W.dm, F, Tc, F, d, EPI_OUT, 0, nullptr, 0, "gemm_layer_dX", st));  // dm
    SBP_TRY(swiglu_bwd(W.dm, W.ug, Tc, F, W.dudg, st, SBP_F32));
    SBP_TRY(tr(W.n2, d, Tc, d, W.tB, Rp, Rp, st));                                        // n2^T
    SBP_TRY(tr(W.dudg, 2 * F, Tc, 2 * F, W.tA, Rp, Rp, st));                              // [du | dg]^T
    SBP_TRY(mm(W.tA, Rp, W.tB, Rp, g->W1, d, F, d, Rp, EPI_F32_ACC, wb, nullptr, 0, "gemm_layer_dW", st));
    SBP_TRY(mm(W.tA + F * Rp, Rp, W.tB, Rp, g->W3, d, F, d, Rp, EPI_F32_ACC, wb, nullptr, 0, "gemm_layer_dW", st));
    SBP_TRY(mm(W.dudg, 2 * F, W.W13T, 2 * F, W.dn, d, Tc, d, 2 * F, EPI_F32, 0, nullptr, 0, "gemm_layer_dX", st));
    SBP_TRY(rmsnorm_bwd(W.a, d, w->g2, W.dn, d, W.rinv2, dyc, d, Tc, d, W.da, d, st, SBP_F32));
    SBP_TRY(gain_grad(W.dn, d, W.a, d, W.rinv2, Tc, d, g->g2, wb, W.gpart, st, SBP_F32));

    // ---- output projection ----
    SBP_TRY(wg(W.da, d, W.o, qd, g->Wo, d, qd, Tc, wb));                                  // dWo += da^T o
    SBP_TRY(mm(W.da, d, W.WoT, d, W.dov, qd, Tc, qd, d, EPI_OUT, 0, nullptr, 0, "gemm_layer_dX", st));  // do

    // ---- attention over the causal key prefix ----
    at.dO = (const bf16_t*)W.dov;
    at.dQ = (bf16_t*)W.dqkv; at.lddq = qkvd;
    at.dK = W.dKacc; at.dV = W.dVacc;
    at.beta = (c == D - 1) ? 0 : 1;  // dK/dV accumulators start at the last chunk
    SBP_TRY(attn_delta_f32(at, W.o, nullptr, 0, 0, S.dh, 1, st));
    SBP_TRY(attn_bwd_chunk_f32(at, S.dh, 1, st));
    if (W.rope_tab) {  // gradients of the rotated q, k -> of the projections
      SBP_TRY(rope_apply(W.dqkv, true, qkvd, W.dqkv, qkvd, Tc, S.Hq, S.dh, s0, W.seq_lo, W.rope_tab, true, st, true));
      SBP_TRY(rope_apply(W.dKacc + s0 * kd, true, kd, W.dqkv + qd, qkvd, Tc, S.Hkv, S.dh, s0,
                         W.seq_lo, W.rope_tab, true, st, true));
    } else {
      SBP_TRY(copy_rows(W.dKacc + s0 * kd, kd, Tc, kd, W.dqkv + qd, qkvd, st));
    }
    if (S.qk_norm) {
      SBP_TRY(headnorm_bwd(W.qraw, qd, W.dqkv, qkvd, W.dqkv, qkvd, Tc, S.Hq, S.dh, w->qn, S.eps,
                           g->qn, wb, W.hnpart, st, SBP_F32));
      SBP_TRY(headnorm_bwd(W.Kraw + s0 * kd, kd, W.dqkv + qd, qkvd, W.dqkv + qd, qkvd, Tc, S.Hkv,
                           S.dh, w->kn, S.eps, g->kn, wb, W.hnpart, st, SBP_F32));
    }
    SBP_TRY(copy_rows(W.dVacc + s0 * kd, kd, Tc, kd, W.dqkv + qd + kd, qkvd, st));

    // ---- q, k, v projections and the first norm ----
    SBP_TRY(tr(W.h1, d, Tc, d, W.tB, Rp, Rp, st));                                        // h1^T
    SBP_TRY(tr(W.dqkv, qkvd, Tc, qkvd, W.tA, Rp, Rp, st));                                // [dq | dK | dV]^T
    SBP_TRY(mm(W.tA, Rp, W.tB, Rp, g->Wq, d, qd, d, Rp, EPI_F32_ACC, wb, nullptr, 0, "gemm_layer_dW", st));
    SBP_TRY(mm(W.tA + qd * Rp, Rp, W.tB, Rp, g->Wk, d, kd, d, Rp, EPI_F32_ACC, wb, nullptr, 0, "gemm_layer_dW", st));
    SBP_TRY(mm(W.tA + (qd + kd) * Rp, Rp, W.tB, Rp, g->Wv, d, kd, d, Rp, EPI_F32_ACC, wb, nullptr, 0, "gemm_layer_dW", st));
    SBP_TRY(mm(W.dqkv, qkvd, W.WqkvT, qkvd, W.dn, d, Tc, d, qkvd, EPI_F32, 0, nullptr, 0, "gemm_layer_dX", st));
    SBP_TRY(rmsnorm_bwd(xc, d, w->g1, W.dn, d, W.rinv1, W.da, d, Tc, d, DX + s0 * d, d, st, SBP_F32));
    SBP_TRY(gain_grad(W.dn, d, xc, d, W.rinv1, Tc, d, g->g1, wb, W.gpart, st, SBP_F32));
  }
  return SBP_OK;
}

sbp_status layer_f32_fwd(const sbp_layer_desc* desc, const int32_t* cu, int32_t nseq, const void* x,
                         const sbp_layer_weights* w, int32_t D, void* y, void* ws, hipStream_t st) {
  const F32Shape S = f32_shape(desc, D);
  F32Ws W;
  f32_plan(S, false, cu != nullptr, (char*)ws, &W);
  const int64_t d = S.d, F = S.F;
  const float* X = (const float*)x;
  float* Y = (float*)y;
  if (cu) SBP_TRY(attn_seq_bounds(cu, nseq, S.T, W.seq_lo, W.seq_hi, st));
  if (W.rope_tab) SBP_TRY(rope_table(W.rope_tab, S.T, S.dh, (double)S.rope_theta, st));
  for (int32_t c = 0; c < D; ++c) {
    int64_t s0, e0;
    chunk_bounds(S.T, D, c, &s0, &e0);
    const int64_t Tc = e0 - s0;
    const float* xc = X + s0 * d;
    SBP_TRY(f32_keys(S, W, xc, w, s0, Tc, st));  // h1 and the chunk's own keys first
    AttnArgs at;
    at.dQ = nullptr; at.dK = nullptr; at.dV = nullptr; at.beta = 0; at.lddq = S.qd;
    SBP_TRY(f32_chunk_fwd(S, W, xc, w, s0, e0, at, st));
    SBP_TRY(mm(W.m, F, (const float*)w->W2, F, Y + s0 * d, d, Tc, d, F, EPI_OUT_RESID, 0, W.a, d, "gemm_layer_fwd", st));
  }
  return SBP_OK;
}

#undef SBP_TRY

}  // namespace sbp
