// sbp_layer_bwd: streamed backward of one pre-norm decoder layer.
//
// StreamBP skill page, "Implementation" (the streaming layer backward: per
// chunk, run the layer forward on the chunk, back-propagate the chunk's
// upstream gradient, add the weight gradients, keep the chunk's input
// gradient) and "Architecture Overview" (layer-wise application, causal
// structure).  Layer (no bias; optional per-head RMSNorm of q and k and
// rotary embedding, neither on the pages):
//   h1 = RMSNorm(x; g1); q, k, v = h1 Wq^T, h1 Wk^T, h1 Wv^T;
//   q, k = HeadNorm(q, k) (qk_norm); q, k = Rope(q, k) (rope_theta > 0)
//   o = causal GQA attention (packed sequences: inside each sequence only);
//   a = x + o Wo^T
//   n2 = RMSNorm(a; g2); [u | g] = n2 [W1; W3]^T; m = silu(u) g; y = a + m W2^T
//
// Pass F: h1 and k, v for every token, chunk by chunk (the causal prefix
// every later query chunk reads).  Pass B, chunks c = D-1 .. 0:
//   recompute h1, q, attention forward (o, LSE) over keys [0, e), a, n2,
//   u, g, m;  dW2 += dy^T m;  dm = dy W2;  du, dg;  dW1 += du^T n2,
//   dW3 += dg^T n2;  dn2 = [du | dg] [W1; W3];  da = dy + RMSNorm2'(dn2),
//   dg2 +=;  dWo += da^T o;  do = da Wo;  attention backward over the prefix
//   (dK, dV of keys [0, e) accumulate in fp32; after chunk c, rows [s, e) are
//   final because later chunks already added theirs and earlier chunks never
//   reach them);  dq, dK_c turned back by the inverse rotation and through
//   the per-head norms (if any);
//   dWq, dWk, dWv += [dq | dK_c | dV_c]^T h1;
//   dh1 = [dq | dK_c | dV_c] [Wq; Wk; Wv];  dx = da + RMSNorm1'(dh1), dg1 +=.
// Every product is one bf16 ring GEMM (gemm.hip).  Weight gradients contract
// over the chunk's tokens and read both activations K-major, in place (e.g.
// dW2 = dy^T m from dy [T_c, d] and m [T_c, F]).  Products that contract
// over a weight's rows (dm = dy W2, dn2 = [du | dg] [W1; W3], do = da Wo,
// dh1 = [dq | dK | dV] [Wq; Wk; Wv]) read weight transposes formed once per
// call.
#include "attn.h"
#include "common.h"
#include "kernels.h"

namespace sbp {
namespace {

inline bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

struct LayerShape {
  int64_t T, d, F, qd, kd, qkvd;
  int Hq, Hkv, dh;
  int32_t D;
  int64_t Tcm;
  float eps;
  float rope_theta;  // 0: no rotary embedding
  bool qk_norm;      // per-head RMSNorm of q and k
};

LayerShape layer_shape(const sbp_layer_desc* L, int32_t D) {
  LayerShape s;
  s.T = L->T; s.d = L->d; s.F = L->F;
  s.Hq = L->Hq; s.Hkv = L->Hkv; s.dh = L->dh;
  s.qd = (int64_t)L->Hq * L->dh;
  s.kd = (int64_t)L->Hkv * L->dh;
  s.qkvd = s.qd + 2 * s.kd;
  s.D = D;
  s.Tcm = max_chunk_len(L->T, D);
  s.eps = L->eps;
  s.rope_theta = L->rope_theta;
  s.qk_norm = L->qk_norm != 0;
  return s;
}

struct LayerWs {
  bf16_t *Kall, *Vall;
  float *dKacc, *dVacc;
  bf16_t *W2T, *W13T, *WoT, *WqkvT;
  bf16_t *h1, *q, *o, *a, *n2, *ug, *mdm, *dudg, *da, *dov, *dqkv;
  float *dn, *rinv1, *rinv2, *lse, *delta, *gpart;
  int *seq_lo, *seq_hi;  // packed sequences only
  float2* rope_tab;      // rotary embedding only: [T, dh/2] (cos, sin)
  bf16_t *Kraw, *qraw;   // QK-norm only: k before its norm [T, kd], q [Tcm, qd]
  float* hnpart;         // QK-norm only: [HEADNORM_PARTS, dh]
};

size_t layer_plan(const LayerShape& s, bool packed, char* base, LayerWs* w) {
  WsPlan P;
  P.base = base;
  LayerWs x;
  const size_t b2 = sizeof(bf16_t), f4 = sizeof(float);
  x.Kall = (bf16_t*)P.take(b2 * s.T * s.kd);
  x.Vall = (bf16_t*)P.take(b2 * s.T * s.kd);
  x.dKacc = (float*)P.take(f4 * s.T * s.kd);
  x.dVacc = (float*)P.take(f4 * s.T * s.kd);
  x.W2T = (bf16_t*)P.take(b2 * s.F * s.d);
  x.W13T = (bf16_t*)P.take(b2 * s.d * 2 * s.F);
  x.WoT = (bf16_t*)P.take(b2 * s.qd * s.d);
  x.WqkvT = (bf16_t*)P.take(b2 * s.d * s.qkvd);
  const int64_t R = s.Tcm;
  x.h1 = (bf16_t*)P.take(b2 * R * s.d);
  x.q = (bf16_t*)P.take(b2 * R * s.qd);
  x.o = (bf16_t*)P.take(b2 * R * s.qd);
  x.a = (bf16_t*)P.take(b2 * R * s.d);
  x.n2 = (bf16_t*)P.take(b2 * R * s.d);
  x.ug = (bf16_t*)P.take(b2 * R * 2 * s.F);
  x.mdm = (bf16_t*)P.take(b2 * R * s.F);
  x.dudg = (bf16_t*)P.take(b2 * R * 2 * s.F);
  x.da = (bf16_t*)P.take(b2 * R * s.d);
  x.dov = (bf16_t*)P.take(b2 * R * s.qd);
  x.dqkv = (bf16_t*)P.take(b2 * R * s.qkvd);
  x.dn = (float*)P.take(f4 * R * s.d);
  x.rinv1 = (float*)P.take(f4 * R);
  x.rinv2 = (float*)P.take(f4 * R);
  x.lse = (float*)P.take(f4 * attn_stats_pitch(R) * s.Hq);
  x.delta = (float*)P.take(f4 * attn_stats_pitch(R) * s.Hq);
  x.gpart = (float*)P.take(f4 * gain_grad_splits(R) * s.d);
  x.seq_lo = packed ? (int*)P.take(sizeof(int) * s.T) : nullptr;
  x.seq_hi = packed ? (int*)P.take(sizeof(int) * s.T) : nullptr;
  x.rope_tab = s.rope_theta > 0.f ? (float2*)P.take(sizeof(float2) * s.T * (s.dh / 2)) : nullptr;
  x.Kraw = s.qk_norm ? (bf16_t*)P.take(b2 * s.T * s.kd) : nullptr;
  x.qraw = s.qk_norm ? (bf16_t*)P.take(b2 * R * s.qd) : nullptr;
  x.hnpart = s.qk_norm ? (float*)P.take(f4 * HEADNORM_PARTS * s.dh) : nullptr;
  if (w) *w = x;
  return round_up((int64_t)P.off, 256);
}

sbp_status layer_check(const sbp_layer_desc* L, int32_t D) {
  if (!L) return set_error(SBP_ERR_INVALID_ARG, "desc is NULL");
  if (L->dtype != SBP_F32 && L->dtype != SBP_BF16) return set_error(SBP_ERR_INVALID_ARG, "dtype %d is not SBP_F32 or SBP_BF16", L->dtype);
  if (L->T < 1 || L->d < 1 || L->Hq < 1 || L->Hkv < 1 || L->dh < 1 || L->F < 1)
    return set_error(SBP_ERR_INVALID_ARG, "T, d, Hq, Hkv, dh, F must be >= 1");
  if (D < 1 || D > L->T) return set_error(SBP_ERR_INVALID_ARG, "need 1 <= D <= T (D=%d, T=%lld)", D, (long long)L->T);
  if (L->Hq % L->Hkv) return set_error(SBP_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", L->Hq, L->Hkv);
  if (!(L->eps >= 0.f)) return set_error(SBP_ERR_INVALID_ARG, "eps must be >= 0");
  if (!(L->rope_theta >= 0.f) || !(L->rope_theta < INFINITY))
    return set_error(SBP_ERR_INVALID_ARG, "rope_theta must be finite and >= 0 (0 = none)");
  if (L->qk_norm != 0 && L->qk_norm != 1) return set_error(SBP_ERR_INVALID_ARG, "qk_norm must be 0 or 1");
  if (L->dh != 64 && L->dh != 128) return set_error(SBP_ERR_UNSUPPORTED, "head dim %d not supported (64 or 128)", L->dh);
  if (L->d % 8 || L->F % 8) return set_error(SBP_ERR_UNSUPPORTED, "d and F must be multiples of 8");
  if (L->T > (1ll << 30) || L->d > (1ll << 20) || L->F > (1ll << 24)) return set_error(SBP_ERR_UNSUPPORTED, "size out of supported range");
  return SBP_OK;
}

// Both entry points: checks, then pass F and pass B over the chunks.
sbp_status layer_run(const sbp_layer_desc* desc, const int32_t* cu, int32_t nseq, const void* x,
                     const void* dy, const sbp_layer_weights* w, int32_t D, int32_t accumulate,
                     void* dx, sbp_layer_grads* g, void* ws, size_t ws_bytes, hipStream_t str) {
  sbp_status st = layer_check(desc, D);
  if (st != SBP_OK) return st;
  if (!x || !dy || !w || !dx || !g) return set_error(SBP_ERR_INVALID_ARG, "x, dy, weights, dx, grads must be non-NULL");
  const void* wp[9] = {w->g1, w->Wq, w->Wk, w->Wv, w->Wo, w->g2, w->W1, w->W3, w->W2};
  float* gp[9] = {g->g1, g->Wq, g->Wk, g->Wv, g->Wo, g->g2, g->W1, g->W3, g->W2};
  for (int i = 0; i < 9; ++i) {
    if (!wp[i] || !gp[i]) return set_error(SBP_ERR_INVALID_ARG, "weight/grad pointer %d is NULL", i);
    if (misaligned(wp[i]) || misaligned(gp[i])) return set_error(SBP_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  }
  if (desc->qk_norm && (!w->qn || !w->kn || !g->qn || !g->kn || misaligned(w->qn) ||
                        misaligned(w->kn) || misaligned(g->qn) || misaligned(g->kn)))
    return set_error(SBP_ERR_INVALID_ARG, "qk_norm: qn, kn weights and grads must be non-NULL and 16-byte aligned");
  if (misaligned(x) || misaligned(dy) || misaligned(dx) || misaligned(ws))
    return set_error(SBP_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  const LayerShape S = layer_shape(desc, D);
  const bool packed = cu != nullptr;
  const bool f32 = desc->dtype == SBP_F32;
  const size_t need = f32 ? layer_f32_ws(desc, D, true, packed) : layer_plan(S, packed, nullptr, nullptr);
  if (!ws || ws_bytes < need)
    return set_error(SBP_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
  if (f32) return layer_f32_bwd(desc, cu, nseq, x, dy, w, D, accumulate, dx, g, ws, str);
  LayerWs W;
  layer_plan(S, packed, (char*)ws, &W);
  const int64_t d = S.d, F = S.F, qd = S.qd, kd = S.kd, qkvd = S.qkvd;
  const bf16_t* X = (const bf16_t*)x;
  const bf16_t* DY = (const bf16_t*)dy;
  bf16_t* DX = (bf16_t*)dx;

#define SBP_TRY(e_)                  \
  do {                               \
    sbp_status _s = (e_);            \
    if (_s != SBP_OK) return _s;     \
  } while (0)

  // C[M, N] (op)= A B^T with A [M, K] and B [N, K] (kmaj: A [K, M], B [K, N])
  auto gemm = [&](const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                  int64_t M, int64_t N, int64_t K, int epi, int beta, const void* R, int64_t ldr,
                  const char* name, int kmaj = 0) -> sbp_status {
    GemmParams p;
    p.A = A; p.lda = lda; p.B = B; p.ldb = ldb; p.C = C; p.ldc = ldc; p.R = R; p.ldr = ldr;
    p.M = (int)M; p.N = (int)N; p.K = (int)K; p.beta = beta;
    p.a_kmajor = p.b_kmajor = kmaj;
    return gemm_nt(SBP_BF16, epi, p, GEMM_TILE_RING, str, name);
  };
  // weight gradient G[M, N] (+)= A^T B over the chunk's Tc tokens, A [Tc, M]
  // and B [Tc, N] read K-major
  auto gemm_wg = [&](const void* A, int64_t lda, const void* B, int64_t ldb, float* G, int64_t M,
                     int64_t N, int64_t Tc, int beta) -> sbp_status {
    return gemm(A, lda, B, ldb, G, N, M, N, Tc, EPI_F32_ACC, beta, nullptr, 0, "gemm_layer_dW", 1);
  };
  // Merged launches where the shapes allow tile-aligned splits (K and V
  // projections: columns at kd; W1 and W3: B rows at F; their gradients: C
  // rows at F, at qd and qd + kd): one launch instead of two or three that
  // would each leave most of the chip idle.
  const bool merge_kv = kd % 256 == 0, merge_13 = F % 256 == 0;
  const bool merge_qkv = qd % 256 == 0 && kd % 256 == 0;
  // [K | V] (Tc x 2kd) = h1 [Wk; Wv]^T into two row arrays of pitch kd
  auto gemm_kv = [&](const void* h1, void* Kdst, void* Vdst, int64_t Tc) -> sbp_status {
    GemmParams p;
    p.A = h1; p.lda = d; p.B = w->Wk; p.B2 = w->Wv; p.b_split = (int)kd; p.ldb = d;
    p.C = Kdst; p.ldc = kd; p.Cx[0] = Vdst; p.c_split[0] = (int)kd; p.c_split_cols = 1;
    p.M = (int)Tc; p.N = (int)(2 * kd); p.K = (int)d;
    return gemm_nt(SBP_BF16, EPI_OUT, p, GEMM_TILE_RING, str, "gemm_layer_fwd");
  };
  // [u | g] = n2 [W1; W3]^T
  auto gemm_13 = [&](const void* n2, void* ug, int64_t Tc) -> sbp_status {
    GemmParams p;
    p.A = n2; p.lda = d; p.B = w->W1; p.B2 = w->W3; p.b_split = (int)F; p.ldb = d;
    p.C = ug; p.ldc = 2 * F; p.M = (int)Tc; p.N = (int)(2 * F); p.K = (int)d;
    return gemm_nt(SBP_BF16, EPI_OUT, p, GEMM_TILE_RING, str, "gemm_layer_fwd");
  };
  // G (+)= A^T n over the chunk's tokens, with A [Tc, M] K-major and the
  // result rows split over up to three gradient arrays of pitch N
  auto gemm_wg_split = [&](const void* A, int64_t lda, const void* Bm, int64_t ldb, int64_t M,
                           int64_t N, int64_t Tc, int beta, float* G0, float* G1, int s1,
                           float* G2, int s2) -> sbp_status {
    GemmParams p;
    p.A = A; p.lda = lda; p.B = Bm; p.ldb = ldb; p.C = G0; p.ldc = N;
    p.Cx[0] = G1; p.c_split[0] = s1; p.Cx[1] = G2; p.c_split[1] = s2;
    p.M = (int)M; p.N = (int)N; p.K = (int)Tc; p.beta = beta;
    p.a_kmajor = p.b_kmajor = 1;
    return gemm_nt(SBP_BF16, EPI_F32_ACC, p, GEMM_TILE_RING, str, "gemm_layer_dW");
  };
  auto tr = [&](const void* src, int64_t ld_src, int64_t rows, int64_t cols, void* dst,
                int64_t ld_dst, int64_t rows_pad) -> sbp_status {
    return transpose_pad(SBP_BF16, src, ld_src, rows, cols, dst, ld_dst, rows_pad, nullptr, str);
  };

  // weight transposes for the products that contract over a weight's rows
  SBP_TRY(tr(w->W2, F, d, F, W.W2T, d, d));                       // W2 [d, F] -> [F, d]
  SBP_TRY(tr(w->W1, d, F, d, W.W13T, 2 * F, F));                   // W1 [F, d] -> cols 0..F
  SBP_TRY(tr(w->W3, d, F, d, W.W13T + F, 2 * F, F));               // W3 -> cols F..2F
  SBP_TRY(tr(w->Wo, qd, d, qd, W.WoT, d, d));                      // Wo [d, qd] -> [qd, d]
  SBP_TRY(tr(w->Wq, d, qd, d, W.WqkvT, qkvd, qd));                 // Wq [qd, d] -> cols 0..qd
  SBP_TRY(tr(w->Wk, d, kd, d, W.WqkvT + qd, qkvd, kd));
  SBP_TRY(tr(w->Wv, d, kd, d, W.WqkvT + qd + kd, qkvd, kd));

  // packed sequences: per-token sequence bounds for the attention kernels
  // (and the rotary positions, which restart at each sequence)
  if (packed) SBP_TRY(attn_seq_bounds(cu, nseq, S.T, W.seq_lo, W.seq_hi, str));
  const bool rope = W.rope_tab != nullptr;
  if (rope) SBP_TRY(rope_table(W.rope_tab, S.T, S.dh, (double)S.rope_theta, str));
  // pass F: keys and values of every token
  for (int32_t c = 0; c < D; ++c) {
    int64_t s0, e0;
    chunk_bounds(S.T, D, c, &s0, &e0);
    const int64_t Tc = e0 - s0;
    SBP_TRY(rmsnorm_fwd(X + s0 * d, d, w->g1, Tc, d, S.eps, W.h1, d, W.rinv1, str));
    // keys before their norm are kept (QK-norm) for the norm's backward
    bf16_t* kdst = (S.qk_norm ? W.Kraw : W.Kall) + s0 * kd;
    if (merge_kv) {
      SBP_TRY(gemm_kv(W.h1, kdst, W.Vall + s0 * kd, Tc));
    } else {
      SBP_TRY(gemm(W.h1, d, w->Wk, d, kdst, kd, Tc, kd, d, EPI_OUT, 0, nullptr, 0, "gemm_layer_fwd"));
      SBP_TRY(gemm(W.h1, d, w->Wv, d, W.Vall + s0 * kd, kd, Tc, kd, d, EPI_OUT, 0, nullptr, 0, "gemm_layer_fwd"));
    }
    if (S.qk_norm)
      SBP_TRY(headnorm_fwd(W.Kraw + s0 * kd, kd, W.Kall + s0 * kd, kd, Tc, S.Hkv, S.dh, w->kn, S.eps, str));
    if (rope)
      SBP_TRY(rope_apply(W.Kall + s0 * kd, false, kd, W.Kall + s0 * kd, kd, Tc, S.Hkv, S.dh, s0,
                         W.seq_lo, W.rope_tab, false, str));
  }

  const float scale = 1.0f / sqrtf((float)S.dh);
  for (int32_t c = D - 1; c >= 0; --c) {
    int64_t s0, e0;
    chunk_bounds(S.T, D, c, &s0, &e0);
    const int64_t Tc = e0 - s0;
    const int wb = (c == D - 1) ? (accumulate ? 1 : 0) : 1;  // weight-gradient beta
    const bf16_t* xc = X + s0 * d;
    const bf16_t* dyc = DY + s0 * d;

    // ---- recompute the chunk's forward ----
    SBP_TRY(rmsnorm_fwd(xc, d, w->g1, Tc, d, S.eps, W.h1, d, W.rinv1, str));
    if (S.qk_norm) {
      SBP_TRY(gemm(W.h1, d, w->Wq, d, W.qraw, qd, Tc, qd, d, EPI_OUT, 0, nullptr, 0, "gemm_layer_fwd"));
      SBP_TRY(headnorm_fwd(W.qraw, qd, W.q, qd, Tc, S.Hq, S.dh, w->qn, S.eps, str));
    } else {
      SBP_TRY(gemm(W.h1, d, w->Wq, d, W.q, qd, Tc, qd, d, EPI_OUT, 0, nullptr, 0, "gemm_layer_fwd"));
    }
    if (rope)
      SBP_TRY(rope_apply(W.q, false, qd, W.q, qd, Tc, S.Hq, S.dh, s0, W.seq_lo, W.rope_tab, false, str));
    AttnArgs at;
    at.Q = W.q; at.K = W.Kall; at.V = W.Vall; at.dO = nullptr; at.O = W.o;
    at.dQ = W.dqkv; at.dK = W.dKacc; at.dV = W.dVacc;
    const int64_t Lp = attn_stats_pitch(S.Tcm);
    at.lse = W.lse; at.lse_sb = 0; at.lse_sh = Lp; at.lse_st = 1;
    at.delta = W.delta; at.dl_sb = 0; at.dl_sh = Lp; at.dl_st = 1;
    at.ldq = qd; at.lddq = qkvd; at.q_bs = 0; at.qoff = (int)s0;
    at.T = (int)S.T; at.Hq = S.Hq; at.Hkv = S.Hkv; at.G = S.Hq / S.Hkv;
    at.s = (int)s0; at.e = (int)e0; at.scale = scale;
    at.beta = (c == D - 1) ? 0 : 1;  // dK/dV accumulators start at the last chunk
    at.seq_lo = W.seq_lo; at.seq_hi = W.seq_hi;
    SBP_TRY(attn_fwd(at, S.dh, 1, str));
    SBP_TRY(gemm(W.o, qd, w->Wo, qd, W.a, d, Tc, d, qd, EPI_OUT_RESID, 0, xc, d, "gemm_layer_fwd"));
    SBP_TRY(rmsnorm_fwd(W.a, d, w->g2, Tc, d, S.eps, W.n2, d, W.rinv2, str));
    if (merge_13) {
      SBP_TRY(gemm_13(W.n2, W.ug, Tc));
    } else {
      SBP_TRY(gemm(W.n2, d, w->W1, d, W.ug, 2 * F, Tc, F, d, EPI_OUT, 0, nullptr, 0, "gemm_layer_fwd"));
      SBP_TRY(gemm(W.n2, d, w->W3, d, W.ug + F, 2 * F, Tc, F, d, EPI_OUT, 0, nullptr, 0, "gemm_layer_fwd"));
    }
    SBP_TRY(swiglu_fwd(W.ug, Tc, F, W.mdm, str));

    // ---- MLP backward ----
    SBP_TRY(gemm_wg(dyc, d, W.mdm, F, g->W2, d, F, Tc, wb));                    // dW2 += dy^T m
    SBP_TRY(gemm(dyc, d, W.W2T, d, W.mdm, F, Tc, F, d, EPI_OUT, 0, nullptr, 0, "gemm_layer_dX"));  // dm
    SBP_TRY(swiglu_bwd(W.mdm, W.ug, Tc, F, W.dudg, str));
    if (merge_13) {  // [dW1; dW3] += [du | dg]^T n2
      SBP_TRY(gemm_wg_split(W.dudg, 2 * F, W.n2, d, 2 * F, d, Tc, wb, g->W1, g->W3, (int)F, nullptr, 0));
    } else {
      SBP_TRY(gemm_wg(W.dudg, 2 * F, W.n2, d, g->W1, F, d, Tc, wb));             // dW1 += du^T n2
      SBP_TRY(gemm_wg(W.dudg + F, 2 * F, W.n2, d, g->W3, F, d, Tc, wb));         // dW3 += dg^T n2
    }
    SBP_TRY(gemm(W.dudg, 2 * F, W.W13T, 2 * F, W.dn, d, Tc, d, 2 * F, EPI_F32, 0, nullptr, 0, "gemm_layer_dX"));
    SBP_TRY(rmsnorm_bwd(W.a, d, w->g2, W.dn, d, W.rinv2, dyc, d, Tc, d, W.da, d, str));
    SBP_TRY(gain_grad(W.dn, d, W.a, d, W.rinv2, Tc, d, g->g2, wb, W.gpart, str));

    // ---- output projection ----
    SBP_TRY(gemm_wg(W.da, d, W.o, qd, g->Wo, d, qd, Tc, wb));                  // dWo += da^T o
    SBP_TRY(gemm(W.da, d, W.WoT, d, W.dov, qd, Tc, qd, d, EPI_OUT, 0, nullptr, 0, "gemm_layer_dX"));  // do

    // ---- attention over the causal key prefix ----
    at.dO = W.dov;
    SBP_TRY(attn_delta(at, W.o, nullptr, 0, 0, S.dh, 1, str));
    SBP_TRY(attn_bwd_chunk(at, S.dh, 1, str));
    if (rope) {  // gradients of the rotated q, k -> of the projections
      SBP_TRY(rope_apply(W.dqkv, false, qkvd, W.dqkv, qkvd, Tc, S.Hq, S.dh, s0, W.seq_lo,
                         W.rope_tab, true, str));
      SBP_TRY(rope_apply(W.dKacc + s0 * kd, true, kd, W.dqkv + qd, qkvd, Tc, S.Hkv, S.dh, s0,
                         W.seq_lo, W.rope_tab, true, str));
    } else {
      SBP_TRY(rows_to_bf16(W.dKacc + s0 * kd, kd, Tc, kd, W.dqkv + qd, qkvd, str));
    }
    if (S.qk_norm) {  // through the per-head norms, in place; gain gradients
      SBP_TRY(headnorm_bwd(W.qraw, qd, W.dqkv, qkvd, W.dqkv, qkvd, Tc, S.Hq, S.dh, w->qn, S.eps,
                           g->qn, wb, W.hnpart, str));
      SBP_TRY(headnorm_bwd(W.Kraw + s0 * kd, kd, W.dqkv + qd, qkvd, W.dqkv + qd, qkvd, Tc, S.Hkv,
                           S.dh, w->kn, S.eps, g->kn, wb, W.hnpart, str));
    }
    SBP_TRY(rows_to_bf16(W.dVacc + s0 * kd, kd, Tc, kd, W.dqkv + qd + kd, qkvd, str));

    // ---- q, k, v projections and the first norm ----
    if (merge_qkv) {  // [dWq; dWk; dWv] += [dq | dK | dV]^T h1
      SBP_TRY(gemm_wg_split(W.dqkv, qkvd, W.h1, d, qkvd, d, Tc, wb, g->Wq, g->Wk, (int)qd, g->Wv,
                            (int)(qd + kd)));
    } else {
      SBP_TRY(gemm_wg(W.dqkv, qkvd, W.h1, d, g->Wq, qd, d, Tc, wb));             // dWq += dq^T h1
      SBP_TRY(gemm_wg(W.dqkv + qd, qkvd, W.h1, d, g->Wk, kd, d, Tc, wb));        // dWk += dK^T h1
      SBP_TRY(gemm_wg(W.dqkv + qd + kd, qkvd, W.h1, d, g->Wv, kd, d, Tc, wb));   // dWv += dV^T h1
    }
    SBP_TRY(gemm(W.dqkv, qkvd, W.WqkvT, qkvd, W.dn, d, Tc, d, qkvd, EPI_F32, 0, nullptr, 0, "gemm_layer_dX"));
    SBP_TRY(rmsnorm_bwd(xc, d, w->g1, W.dn, d, W.rinv1, W.da, d, Tc, d, DX + s0 * d, d, str));
    SBP_TRY(gain_grad(W.dn, d, xc, d, W.rinv1, Tc, d, g->g1, wb, W.gpart, str));
  }
#undef SBP_TRY
  return SBP_OK;
}

// ---------------------------------------------------------------------------
// Chunked forward y = Layer(x): chunks in order, each forming its own keys and
// values before its queries attend over keys [0, e) (seq_lo bounds them to the
// query's sequence when packed).  Activations exist for one chunk at a time;
// keys and values for all tokens.
struct LayerFwdWs {
  bf16_t *Kall, *Vall, *h1, *q, *o, *a, *n2, *ug, *m;
  float *rinv, *lse;
  int *seq_lo, *seq_hi;
  float2* rope_tab;
};

size_t layer_fwd_plan(const LayerShape& s, char* base, LayerFwdWs* w) {
  WsPlan P;
  P.base = base;
  LayerFwdWs x;
  const size_t b2 = sizeof(bf16_t), f4 = sizeof(float);
  const int64_t R = s.Tcm;
  x.Kall = (bf16_t*)P.take(b2 * s.T * s.kd);
  x.Vall = (bf16_t*)P.take(b2 * s.T * s.kd);
  x.h1 = (bf16_t*)P.take(b2 * R * s.d);
  x.q = (bf16_t*)P.take(b2 * R * s.qd);
  x.o = (bf16_t*)P.take(b2 * R * s.qd);
  x.a = (bf16_t*)P.take(b2 * R * s.d);
  x.n2 = (bf16_t*)P.take(b2 * R * s.d);
  x.ug = (bf16_t*)P.take(b2 * R * 2 * s.F);
  x.m = (bf16_t*)P.take(b2 * R * s.F);
  x.rinv = (float*)P.take(f4 * R);
  x.lse = (float*)P.take(f4 * attn_stats_pitch(R) * s.Hq);
  x.seq_lo = (int*)P.take(sizeof(int) * s.T);
  x.seq_hi = (int*)P.take(sizeof(int) * s.T);
  x.rope_tab = s.rope_theta > 0.f ? (float2*)P.take(sizeof(float2) * s.T * (s.dh / 2)) : nullptr;
  if (w) *w = x;
  return round_up((int64_t)P.off, 256);
}

sbp_status layer_fwd_run(const sbp_layer_desc* desc, const int32_t* cu, int32_t nseq,
                         const void* x, const sbp_layer_weights* w, int32_t D, void* y, void* ws,
                         size_t ws_bytes, hipStream_t str) {
  sbp_status st = layer_check(desc, D);
  if (st != SBP_OK) return st;
  if (!x || !w || !y) return set_error(SBP_ERR_INVALID_ARG, "x, weights, y must be non-NULL");
  const void* wp[9] = {w->g1, w->Wq, w->Wk, w->Wv, w->Wo, w->g2, w->W1, w->W3, w->W2};
  for (int i = 0; i < 9; ++i) {
    if (!wp[i]) return set_error(SBP_ERR_INVALID_ARG, "weight pointer %d is NULL", i);
    if (misaligned(wp[i])) return set_error(SBP_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  }
  if (desc->qk_norm && (!w->qn || !w->kn || misaligned(w->qn) || misaligned(w->kn)))
    return set_error(SBP_ERR_INVALID_ARG, "qk_norm: qn, kn must be non-NULL and 16-byte aligned");
  if (misaligned(x) || misaligned(y) || misaligned(ws) || (cu && misaligned(cu)))
    return set_error(SBP_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  if (cu && nseq < 1) return set_error(SBP_ERR_INVALID_ARG, "nseq must be >= 1 (got %d)", nseq);
  if (x == y) return set_error(SBP_ERR_INVALID_ARG, "y must not alias x");
  const LayerShape S = layer_shape(desc, D);
  const bool f32 = desc->dtype == SBP_F32;
  const size_t need = f32 ? layer_f32_ws(desc, D, false, true) : layer_fwd_plan(S, nullptr, nullptr);
  if (!ws || ws_bytes < need)
    return set_error(SBP_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
  if (f32) return layer_f32_fwd(desc, cu, nseq, x, w, D, y, ws, str);
  LayerFwdWs W;
  layer_fwd_plan(S, (char*)ws, &W);
  const int64_t d = S.d, F = S.F, qd = S.qd, kd = S.kd;
  const bf16_t* X = (const bf16_t*)x;
  bf16_t* Y = (bf16_t*)y;
  const int* seq_lo = cu ? W.seq_lo : nullptr;
  const int* seq_hi = cu ? W.seq_hi : nullptr;

  auto gemm = [&](const void* A, int64_t lda, const void* B, void* C, int64_t ldc, int64_t M,
                  int64_t N, int64_t K, int epi, const void* R, int64_t ldr) -> sbp_status {
    GemmParams p;
    p.A = A; p.lda = lda; p.B = B; p.ldb = K; p.C = C; p.ldc = ldc; p.R = R; p.ldr = ldr;
    p.M = (int)M; p.N = (int)N; p.K = (int)K;
    return gemm_nt(SBP_BF16, epi, p, GEMM_TILE_RING, str, "gemm_layer_fwd");
  };
#define SBP_TRY(e_)                  \
  do {                               \
    sbp_status _s = (e_);            \
    if (_s != SBP_OK) return _s;     \
  } while (0)

  if (cu) SBP_TRY(attn_seq_bounds(cu, nseq, S.T, W.seq_lo, W.seq_hi, str));
  const bool rope = W.rope_tab != nullptr;
  if (rope) SBP_TRY(rope_table(W.rope_tab, S.T, S.dh, (double)S.rope_theta, str));
  const float scale = 1.0f / sqrtf((float)S.dh);
  const int64_t Lp = attn_stats_pitch(S.Tcm);
  for (int32_t c = 0; c < D; ++c) {
    int64_t s0, e0;
    chunk_bounds(S.T, D, c, &s0, &e0);
    const int64_t Tc = e0 - s0;
    const bf16_t* xc = X + s0 * d;
    SBP_TRY(rmsnorm_fwd(xc, d, w->g1, Tc, d, S.eps, W.h1, d, W.rinv, str));
    if (kd % 256 == 0) {  // [K | V] = h1 [Wk; Wv]^T in one launch
      GemmParams p;
      p.A = W.h1; p.lda = d; p.B = w->Wk; p.B2 = w->Wv; p.b_split = (int)kd; p.ldb = d;
      p.C = W.Kall + s0 * kd; p.ldc = kd; p.Cx[0] = W.Vall + s0 * kd; p.c_split[0] = (int)kd;
      p.c_split_cols = 1; p.M = (int)Tc; p.N = (int)(2 * kd); p.K = (int)d;
      SBP_TRY(gemm_nt(SBP_BF16, EPI_OUT, p, GEMM_TILE_RING, str, "gemm_layer_fwd"));
    } else {
      SBP_TRY(gemm(W.h1, d, w->Wk, W.Kall + s0 * kd, kd, Tc, kd, d, EPI_OUT, nullptr, 0));
      SBP_TRY(gemm(W.h1, d, w->Wv, W.Vall + s0 * kd, kd, Tc, kd, d, EPI_OUT, nullptr, 0));
    }
    SBP_TRY(gemm(W.h1, d, w->Wq, W.q, qd, Tc, qd, d, EPI_OUT, nullptr, 0));
    if (S.qk_norm) {  // in place
      SBP_TRY(headnorm_fwd(W.Kall + s0 * kd, kd, W.Kall + s0 * kd, kd, Tc, S.Hkv, S.dh, w->kn, S.eps, str));
      SBP_TRY(headnorm_fwd(W.q, qd, W.q, qd, Tc, S.Hq, S.dh, w->qn, S.eps, str));
    }
    if (rope) {
      SBP_TRY(rope_apply(W.Kall + s0 * kd, false, kd, W.Kall + s0 * kd, kd, Tc, S.Hkv, S.dh, s0,
                         seq_lo, W.rope_tab, false, str));
      SBP_TRY(rope_apply(W.q, false, qd, W.q, qd, Tc, S.Hq, S.dh, s0, seq_lo, W.rope_tab, false, str));
    }
    AttnArgs at;
    at.Q = W.q; at.K = W.Kall; at.V = W.Vall; at.dO = nullptr; at.O = W.o;
    at.dQ = nullptr; at.dK = nullptr; at.dV = nullptr;
    at.lse = W.lse; at.lse_sb = 0; at.lse_sh = Lp; at.lse_st = 1;
    at.delta = nullptr; at.dl_sb = 0; at.dl_sh = Lp; at.dl_st = 1;
    at.ldq = qd; at.lddq = qd; at.q_bs = 0; at.qoff = (int)s0;
    at.T = (int)S.T; at.Hq = S.Hq; at.Hkv = S.Hkv; at.G = S.Hq / S.Hkv;
    at.s = (int)s0; at.e = (int)e0; at.scale = scale; at.beta = 0;
    at.seq_lo = seq_lo; at.seq_hi = seq_hi;
    SBP_TRY(attn_fwd(at, S.dh, 1, str));
    SBP_TRY(gemm(W.o, qd, w->Wo, W.a, d, Tc, d, qd, EPI_OUT_RESID, xc, d));          // a = x + o Wo^T
    SBP_TRY(rmsnorm_fwd(W.a, d, w->g2, Tc, d, S.eps, W.n2, d, W.rinv, str));
    if (F % 256 == 0) {  // [u | g] = n2 [W1; W3]^T in one launch
      GemmParams p;
      p.A = W.n2; p.lda = d; p.B = w->W1; p.B2 = w->W3; p.b_split = (int)F; p.ldb = d;
      p.C = W.ug; p.ldc = 2 * F; p.M = (int)Tc; p.N = (int)(2 * F); p.K = (int)d;
      SBP_TRY(gemm_nt(SBP_BF16, EPI_OUT, p, GEMM_TILE_RING, str, "gemm_layer_fwd"));
    } else {
      SBP_TRY(gemm(W.n2, d, w->W1, W.ug, 2 * F, Tc, F, d, EPI_OUT, nullptr, 0));
      SBP_TRY(gemm(W.n2, d, w->W3, W.ug + F, 2 * F, Tc, F, d, EPI_OUT, nullptr, 0));
    }
    SBP_TRY(swiglu_fwd(W.ug, Tc, F, W.m, str));
    SBP_TRY(gemm(W.m, F, w->W2, Y + s0 * d, d, Tc, d, F, EPI_OUT_RESID, W.a, d));   // y = a + m W2^T
  }
#undef SBP_TRY
  return SBP_OK;
}

}  // namespace
}  // namespace sbp

using namespace sbp;

extern "C" sbp_status sbp_layer_fwd_workspace_size(const sbp_layer_desc* desc, int32_t D,
                                                   size_t* bytes) {
  clear_error();
  if (!bytes) return set_error(SBP_ERR_INVALID_ARG, "bytes is NULL");
  sbp_status st = layer_check(desc, D);
  if (st != SBP_OK) return st;
  *bytes = desc->dtype == SBP_F32 ? layer_f32_ws(desc, D, false, true)
                                  : layer_fwd_plan(layer_shape(desc, D), nullptr, nullptr);
  return SBP_OK;
}

extern "C" sbp_status sbp_layer_fwd(const sbp_layer_desc* desc, const int32_t* cu_seqlens,
                                    int32_t nseq, const void* x, const sbp_layer_weights* w,
                                    int32_t D, void* y, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  sbp_status st = desc && cu_seqlens && nseq >= 1 && !misaligned(cu_seqlens)
                      ? debug_check_cu(cu_seqlens, nseq, desc->T, (hipStream_t)stream)
                      : SBP_OK;
  if (st != SBP_OK) return st;
  st = layer_fwd_run(desc, cu_seqlens, nseq, x, w, D, y, ws, ws_bytes, (hipStream_t)stream);
  return st == SBP_OK ? debug_sync((hipStream_t)stream, "sbp_layer_fwd") : st;
}

extern "C" sbp_status sbp_layer_bwd_workspace_size(const sbp_layer_desc* desc, int32_t D,
                                                   size_t* bytes) {
  clear_error();
  if (!bytes) return set_error(SBP_ERR_INVALID_ARG, "bytes is NULL");
  sbp_status st = layer_check(desc, D);
  if (st != SBP_OK) return st;
  *bytes = desc->dtype == SBP_F32 ? layer_f32_ws(desc, D, true, false)
                                  : layer_plan(layer_shape(desc, D), false, nullptr, nullptr);
  return SBP_OK;
}

extern "C" sbp_status sbp_layer_bwd(const sbp_layer_desc* desc, const void* x, const void* dy,
                                    const sbp_layer_weights* w, int32_t D, int32_t accumulate,
                                    void* dx, sbp_layer_grads* g, void* ws, size_t ws_bytes,
                                    void* stream) {
  clear_error();
  const sbp_status st = layer_run(desc, nullptr, 0, x, dy, w, D, accumulate, dx, g, ws, ws_bytes,
                                  (hipStream_t)stream);
  return st == SBP_OK ? debug_sync((hipStream_t)stream, "sbp_layer_bwd") : st;
}

extern "C" sbp_status sbp_layer_bwd_packed_workspace_size(const sbp_layer_desc* desc, int32_t D,
                                                          size_t* bytes) {
  clear_error();
  if (!bytes) return set_error(SBP_ERR_INVALID_ARG, "bytes is NULL");
  sbp_status st = layer_check(desc, D);
  if (st != SBP_OK) return st;
  *bytes = desc->dtype == SBP_F32 ? layer_f32_ws(desc, D, true, true)
                                  : layer_plan(layer_shape(desc, D), true, nullptr, nullptr);
  return SBP_OK;
}

extern "C" sbp_status sbp_layer_bwd_packed(const sbp_layer_desc* desc, const int32_t* cu_seqlens,
                                           int32_t nseq, const void* x, const void* dy,
                                           const sbp_layer_weights* w, int32_t D,
                                           int32_t accumulate, void* dx, sbp_layer_grads* g,
                                           void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  if (!cu_seqlens) return set_error(SBP_ERR_INVALID_ARG, "cu_seqlens must be non-NULL");
  if (nseq < 1) return set_error(SBP_ERR_INVALID_ARG, "nseq must be >= 1 (got %d)", nseq);
  if (misaligned(cu_seqlens)) return set_error(SBP_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  sbp_status st = desc ? debug_check_cu(cu_seqlens, nseq, desc->T, (hipStream_t)stream) : SBP_OK;
  if (st != SBP_OK) return st;
  st = layer_run(desc, cu_seqlens, nseq, x, dy, w, D, accumulate, dx, g, ws, ws_bytes,
                 (hipStream_t)stream);
  return st == SBP_OK ? debug_sync((hipStream_t)stream, "sbp_layer_bwd_packed") : st;
}
