// sbp_lmhead_ce_fwd_bwd: chunked LM head + softmax cross-entropy.
//
// Per chunk c = [s, e) (skill page "Implementation": the sequence
// decomposition, the logits-gradient routine and the linear-layer chunk
// gradient):
//   Z_c   = H_c W^T                [T_c, V]                (gemm, EPI_REL16_LSE: per-64-
//                                  column row (max, sum-exp) partials in fp32 and every
//                                  logit minus its group's max in fp16; fp32 logits
//                                  where that epilogue does not apply: fp32, d % 128)
//   lse, l_t, c_t l_t              per row                 (ce_merge of the partials;
//                                  ce_stats over the fp32 logits otherwise)
//   dZ_c                           dtype, zero-padded      (ce_grad)
//   dH_c  = dZ_c W                 split-K partials, sum   (gemm EPI_PARTIAL, splitk_reduce)
//   dW   += dZ_g^T H_g             fp32 read-modify-write  (gemm EPI_F32_ACC)
// The weight gradient is taken once per group g of G consecutive chunks, so
// that the fp32 read-modify-write of dW is paid once per G chunks and the
// GEMM's K (the group's tokens) is about 4096 long.
// W^T is formed once per call (dH contracts over W's rows).  bf16: the dW
// GEMM reads dZ_g and H_g ([tokens, .], contracted over tokens) K-major, in
// place: dZ_c is written into a group buffer whose rows are the group's
// tokens in order, and H_g is a row range of H.  With fused statistics the
// logits GEMM writes the chunk's fp16 relative logits into the chunk's rows
// of that buffer and ce_grad turns them into dZ_c in place (same element
// size and layout), so no separate logits buffer exists.  fp32 (NT GEMMs
// only): dZ_c^T and H_c^T side by side in K per group (slots of T_c rounded
// up to the K granule).  Workspace O(G T_c V + V d).
//
// G, the chunks per dW GEMM, is the largest the caller's workspace holds, up
// to a group of about 4096 tokens: sbp_lmhead_ce_workspace_size gives the
// smallest workspace (G = 1, peak memory falling with D), and
// sbp_lmhead_ce_workspace_size_grouped the one for a given G.
#include "common.h"
#include "kernels.h"

namespace sbp {
namespace {

struct LmWs {
  void* Z;    // fp32 logits [T_c, Vp] (no fused statistics); with them, NULL:
              // each chunk's fp16 relative logits sit in its rows of dZ
  float* ztgt;  // fused statistics: each row's target logit, fp32 [T_c]
  void* dZ;   // bf16: the group buffer [G T_c, Vp]; fp32: [T_c, Vp]
  void* dZt;  // fp32 only
  void* Wt;
  void* Ht;   // fp32 only
  float* part;
  float* lse;
  float* loss_part;
  float2* parts;  // [T_c, nparts] row (max, sum-exp) partials of the logits GEMM
  LmPrep prep;
};

struct LmShape {
  int64_t T, d, V;
  int32_t D;
  int dtype;
  int64_t Tcm, Tcp, Vp;
  int S;  // split count of the dH GEMM
  bool fused_stats;  // the logits GEMM writes the row statistics partials
  int nparts;
  int G;  // chunks per dW GEMM
  int Gmax;  // largest group used: about 4096 tokens
  int64_t Kg;  // fp32: K extent of the dW group buffers, G * Tcp
  bool kmajor;  // bf16: GEMM operands read K-major in place
  bool inplace;  // the fused logits live in the dZ group buffer
  size_t esz;
};

LmShape lm_shape(int64_t T, int64_t d, int64_t V, int32_t D, int dtype, int G) {
  LmShape s;
  s.T = T; s.d = d; s.V = V; s.D = D; s.dtype = dtype;
  s.esz = dtype == SBP_BF16 ? 2 : 4;
  s.Tcm = max_chunk_len(T, D);
  s.Tcp = round_up(s.Tcm, 128);  // fp32 dW slot width; also sets the group size
  s.Vp = round_up(V, 128);
  // dH GEMM: few output tiles, long K = V.  Split K so that the launch has
  // ~256 blocks, one per CU (the ring GEMM holds one block per CU, so more
  // splits only add fp32 partials to write and sum: measured, 8 splits cost
  // 7% more GEMM time and 4x the partial traffic); no split once the tiles
  // alone fill three quarters of the CUs (224 tiles at T_c = 4096, d = 3584:
  // one round of whole-K tiles was 3.8% faster than two rounds of half-K
  // partials); a function of the shape only.
  const int64_t tiles = cdiv(s.Tcm, 256) * cdiv(d, 256);
  int64_t S = tiles >= 192 ? 1 : cdiv(256, tiles);
  S = std::max<int64_t>(1, std::min<int64_t>(S, 16));
  S = std::min<int64_t>(S, std::max<int64_t>(1, s.Vp / 512));
  s.S = (int)S;
  // dW group: up to about 4096 tokens of K per weight-gradient GEMM (its
  // fp32 read-modify-write of the V x d gradient then costs a quarter byte
  // per flop or less); G itself is chosen from the workspace (lm_group).
  s.Gmax = (int)std::max<int64_t>(1, std::min<int64_t>(D, 4096 / s.Tcp));
  s.G = std::max(1, std::min(G, s.Gmax));
  s.Kg = s.G * s.Tcp;
  s.kmajor = dtype == SBP_BF16;
  s.fused_stats = dtype == SBP_BF16 && d % 128 == 0;
  s.inplace = s.fused_stats && s.kmajor;
  s.nparts = (int)(4 * cdiv(V, 256));
  return s;
}

size_t lm_plan(const LmShape& s, char* base, LmWs* w) {
  WsPlan P;
  P.base = base;
  LmWs x;
  x.Z = s.inplace ? nullptr : P.take((s.fused_stats ? 2 : sizeof(float)) * s.Tcm * s.Vp);
  x.Wt = P.take(s.esz * s.d * s.Vp);
  if (s.kmajor) {
    x.dZ = P.take(s.esz * s.G * s.Tcm * s.Vp);
    x.dZt = x.Ht = nullptr;
  } else {
    x.dZ = P.take(s.esz * s.Tcm * s.Vp);
    x.dZt = P.take(s.esz * s.Vp * s.Kg);
    x.Ht = P.take(s.esz * s.d * s.Kg);
  }
  x.part = (float*)P.take(sizeof(float) * (size_t)s.S * s.Tcm * s.d);
  x.lse = (float*)P.take(sizeof(float) * s.Tcm);
  x.loss_part = (float*)P.take(sizeof(float) * s.T);
  x.parts = s.fused_stats ? (float2*)P.take(sizeof(float2) * s.Tcm * s.nparts) : nullptr;
  x.ztgt = s.fused_stats ? (float*)P.take(sizeof(float) * s.Tcm) : nullptr;
  x.prep.n_valid = (int*)P.take(sizeof(int));
  x.prep.inv_norm = (float*)P.take(sizeof(float));
  x.prep.none_active = (int*)P.take(sizeof(int));
  x.prep.chunk_active = (int*)P.take(sizeof(int) * s.D);
  x.prep.group_active = (int*)P.take(sizeof(int) * cdiv(s.D, s.G));
  x.prep.beta_zero = (int*)P.take(sizeof(int) * cdiv(s.D, s.G));
  if (w) *w = x;
  return round_up((int64_t)P.off, 256);
}

// Forward-only log-probability call: per chunk either the statistics
// partials and target logits of the logits GEMM (no logits written) or, where
// that epilogue does not apply, the fp32 logits of the chunk.
struct LpWs {
  float* Z;       // [T_c, Vp] fp32, unfused path only
  float2* parts;  // [T_c, nparts], fused path only
  float* zt;      // [T_c] target logits, fused path only
  LmPrep prep;
};

size_t lp_plan(const LmShape& s, char* base, LpWs* w) {
  WsPlan P;
  P.base = base;
  LpWs x;
  x.Z = s.fused_stats ? nullptr : (float*)P.take(sizeof(float) * s.Tcm * s.Vp);
  x.parts = s.fused_stats ? (float2*)P.take(sizeof(float2) * s.Tcm * s.nparts) : nullptr;
  x.zt = s.fused_stats ? (float*)P.take(sizeof(float) * s.Tcm) : nullptr;
  x.prep.n_valid = (int*)P.take(sizeof(int));
  x.prep.inv_norm = (float*)P.take(sizeof(float));
  x.prep.none_active = (int*)P.take(sizeof(int));
  x.prep.chunk_active = (int*)P.take(sizeof(int) * s.D);
  x.prep.group_active = (int*)P.take(sizeof(int) * s.D);
  x.prep.beta_zero = (int*)P.take(sizeof(int) * s.D);
  if (w) *w = x;
  return round_up((int64_t)P.off, 256);
}

inline bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

// The largest dW group (<= Gmax) whose workspace fits in ws_bytes; 0 if
// not even G = 1 fits.
int lm_group(int64_t T, int64_t d, int64_t V, int32_t D, int dtype, size_t ws_bytes) {
  const int gmax = lm_shape(T, d, V, D, dtype, 1).Gmax;
  for (int g = gmax; g >= 1; --g)
    if (lm_plan(lm_shape(T, d, V, D, dtype, g), nullptr, nullptr) <= ws_bytes) return g;
  return 0;
}

sbp_status lm_check_sizes(int64_t T, int64_t d, int64_t V, int32_t D, int32_t dtype) {
  if (dtype != SBP_F32 && dtype != SBP_BF16) return set_error(SBP_ERR_INVALID_ARG, "dtype %d is not SBP_F32 or SBP_BF16", dtype);
  if (T < 1 || d < 1 || V < 1) return set_error(SBP_ERR_INVALID_ARG, "T, d, V must be >= 1 (got %lld, %lld, %lld)", (long long)T, (long long)d, (long long)V);
  if (D < 1 || D > T) return set_error(SBP_ERR_INVALID_ARG, "need 1 <= D <= T (D=%d, T=%lld)", D, (long long)T);
  const int64_t vec = dtype == SBP_BF16 ? 8 : 4;
  if (d % vec) return set_error(SBP_ERR_UNSUPPORTED, "d=%lld must be a multiple of %lld for this dtype", (long long)d, (long long)vec);
  if (T > (1ll << 30) || V > (1ll << 30) || d > (1ll << 20)) return set_error(SBP_ERR_UNSUPPORTED, "size out of supported range");
  return SBP_OK;
}

}  // namespace
}  // namespace sbp

using namespace sbp;

extern "C" sbp_status sbp_lmhead_ce_workspace_size(int64_t T, int64_t d, int64_t V, int32_t D,
                                                   int32_t dtype, size_t* bytes) {
  clear_error();
  if (!bytes) return set_error(SBP_ERR_INVALID_ARG, "bytes is NULL");
  sbp_status st = lm_check_sizes(T, d, V, D, dtype);
  if (st != SBP_OK) return st;
  *bytes = lm_plan(lm_shape(T, d, V, D, dtype, 1), nullptr, nullptr);
  return SBP_OK;
}

extern "C" sbp_status sbp_lmhead_ce_workspace_size_grouped(int64_t T, int64_t d, int64_t V,
                                                           int32_t D, int32_t dtype, int32_t G,
                                                           size_t* bytes) {
  clear_error();
  if (!bytes) return set_error(SBP_ERR_INVALID_ARG, "bytes is NULL");
  sbp_status st = lm_check_sizes(T, d, V, D, dtype);
  if (st != SBP_OK) return st;
  if (G < 1) return set_error(SBP_ERR_INVALID_ARG, "G must be >= 1 (got %d)", G);
  *bytes = lm_plan(lm_shape(T, d, V, D, dtype, G), nullptr, nullptr);
  return SBP_OK;
}

static sbp_status lmhead_ce_impl(const void* H, const void* W, const int32_t* targets,
                                 const float* weights, int64_t T, int64_t d, int64_t V,
                                 int32_t D, int32_t dtype, int32_t reduction,
                                 int32_t accumulate, float* loss, float* token_loss,
                                 void* dH, float* dW, void* ws, size_t ws_bytes,
                                 void* stream) {
  sbp_status st = lm_check_sizes(T, d, V, D, dtype);
  if (st != SBP_OK) return st;
  if (reduction != SBP_MEAN_VALID && reduction != SBP_SUM)
    return set_error(SBP_ERR_INVALID_ARG, "reduction %d is not SBP_MEAN_VALID or SBP_SUM", reduction);
  if (!H || !W || !targets || !loss || !dH || !dW)
    return set_error(SBP_ERR_INVALID_ARG, "H, W, targets, loss, dH and dW must be non-NULL");
  if (misaligned(H) || misaligned(W) || misaligned(targets) || misaligned(loss) || misaligned(dH) ||
      misaligned(dW) || misaligned(weights) || misaligned(token_loss) || misaligned(ws))
    return set_error(SBP_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  const int G = ws ? lm_group(T, d, V, D, dtype, ws_bytes) : 0;
  if (G == 0) {
    const size_t need = lm_plan(lm_shape(T, d, V, D, dtype, 1), nullptr, nullptr);
    return set_error(SBP_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
  }
  const LmShape s = lm_shape(T, d, V, D, dtype, G);
  LmWs w;
  lm_plan(s, (char*)ws, &w);
  hipStream_t str = (hipStream_t)stream;
  const char* Hb = (const char*)H;

#define SBP_TRY(x)                   \
  do {                               \
    sbp_status _s = (x);             \
    if (_s != SBP_OK) return _s;     \
  } while (0)

  SBP_TRY(lm_prep(targets, T, V, D, s.G, reduction, accumulate, w.prep, str));
  // W^T [d, Vp], zero columns V..Vp (they meet the zero pad of dZ in the dH
  // GEMM)
  SBP_TRY(transpose_pad(dtype, W, d, V, d, w.Wt, s.Vp, s.Vp, nullptr, str));
  int64_t s_group = 0;  // first token of the current dW group
  for (int32_t c = 0; c < D; ++c) {
    int64_t s0, e0;
    chunk_bounds(T, D, c, &s0, &e0);
    const int64_t Tc = e0 - s0;
    const int* act = w.prep.chunk_active + c;
    // chunk c is slot j of dW group g.  bf16: its dZ rows are rows
    // [s0 - s_group, e0 - s_group) of the group buffer; fp32: columns
    // [j Tcp, (j + 1) Tcp) of dZ^T and H^T, zero past the chunk's T_c.  In a
    // group of several chunks an inactive chunk still writes its slot (zeros:
    // every row has c_t = 0).
    const int g = c / s.G, j = c % s.G;
    if (j == 0) s_group = s0;
    const bool last_in_group = j == s.G - 1 || c == D - 1;
    const int* slot_act = s.G == 1 ? act : nullptr;
    char* dZc = (char*)w.dZ + (s.kmajor ? (s0 - s_group) * s.Vp * s.esz : 0);

    // the chunk's logits: in its own rows of the dZ group buffer when the
    // statistics are fused (turned into dZ_c in place by ce_grad)
    void* Zc = s.inplace ? (void*)dZc : w.Z;
    GemmParams g1;
    g1.A = Hb + s0 * d * s.esz; g1.lda = d;
    g1.B = W; g1.ldb = d;
    g1.C = Zc; g1.ldc = s.Vp;
    g1.M = (int)Tc; g1.N = (int)V; g1.K = (int)d;
    g1.active = act;
    g1.m_fastest = 1;
    if (s.fused_stats) {
      g1.row_stats = w.parts;
      g1.ld_stats = s.nparts;
      g1.row_target = targets + s0;
      g1.target_out = w.ztgt;
      SBP_TRY(gemm_nt(dtype, EPI_REL16_LSE, g1, GEMM_TILE_RING, str, "gemm_logits"));
      SBP_TRY(ce_merge(w.parts, s.nparts, s.nparts, w.ztgt, targets, weights, s0, Tc, V, w.lse,
                       w.loss_part, token_loss, str));
    } else {
      SBP_TRY(gemm_nt(dtype, EPI_F32, g1, GEMM_TILE_RING, str, "gemm_logits"));
      SBP_TRY(ce_stats((const float*)w.Z, s.Vp, targets, weights, s0, Tc, V, w.lse, w.loss_part,
                       token_loss, str));
    }
    if (s.kmajor) {
      SBP_TRY(ce_grad(dtype, Zc, s.fused_stats ? w.parts : nullptr, s.nparts, s.Vp, targets,
                      weights, w.prep.inv_norm, w.lse, s0, Tc, V, s.Vp, dZc, s.Vp, nullptr, 0, 0,
                      slot_act, str));
    } else {
      SBP_TRY(ce_grad(dtype, w.Z, nullptr, 0, s.Vp, targets, weights, w.prep.inv_norm, w.lse, s0,
                      Tc, V, s.Vp, dZc, s.Vp, (char*)w.dZt + j * s.Tcp * s.esz, s.Kg, s.Tcp,
                      slot_act, str));
      SBP_TRY(transpose_pad(dtype, Hb + s0 * d * s.esz, d, Tc, d, (char*)w.Ht + j * s.Tcp * s.esz, s.Kg,
                            s.Tcp, slot_act, str));
    }

    // dH_c = dZ_c (W^T)^T over K = Vp: the zero pad of dZ_c (columns V ..
    // Vp) meets the zero columns of W^T
    GemmParams g2;
    g2.A = dZc; g2.lda = s.Vp;
    g2.B = w.Wt; g2.ldb = s.Vp;
    g2.C = w.part; g2.ldc = d;
    g2.M = (int)Tc; g2.N = (int)d; g2.K = (int)s.Vp;
    g2.k_split = s.S;
    g2.split_stride = s.Tcm * d;
    g2.active = act;
    g2.m_fastest = 1;
    SBP_TRY(gemm_nt(dtype, EPI_PARTIAL, g2, GEMM_TILE_RING, str, "gemm_dH"));
    SBP_TRY(splitk_reduce(dtype, w.part, s.Tcm * d, s.S, Tc, d, d, (char*)dH + s0 * d * s.esz, d,
                          act, str));

    if (!last_in_group) continue;
    // dW += dZ_g^T H_g over the group's tokens [s_group, e0)
    GemmParams g3;
    if (s.kmajor) {
      g3.A = w.dZ; g3.lda = s.Vp; g3.a_kmajor = 1;
      g3.B = Hb + s_group * d * s.esz; g3.ldb = d; g3.b_kmajor = 1;
      g3.K = (int)(e0 - s_group);
    } else {
      g3.A = w.dZt; g3.lda = s.Kg;
      g3.B = w.Ht; g3.ldb = s.Kg;
      g3.K = (int)((j + 1) * s.Tcp);
    }
    g3.C = dW; g3.ldc = d;
    g3.M = (int)V; g3.N = (int)d;
    g3.beta = 1;
    g3.beta_zero = w.prep.beta_zero + g;
    g3.active = w.prep.group_active + g;
    g3.m_fastest = 0;
    SBP_TRY(gemm_nt(dtype, EPI_F32_ACC, g3, GEMM_TILE_RING, str, "gemm_dW"));
  }
  if (!accumulate) SBP_TRY(fill_zero_f32(dW, V * d, w.prep.none_active, str));
  SBP_TRY(loss_reduce(w.loss_part, T, w.prep.inv_norm, loss, str));
#undef SBP_TRY
  return SBP_OK;
}

extern "C" sbp_status sbp_lmhead_logprob_workspace_size(int64_t T, int64_t d, int64_t V, int32_t D,
                                                       int32_t dtype, size_t* bytes) {
  clear_error();
  if (!bytes) return set_error(SBP_ERR_INVALID_ARG, "bytes is NULL");
  sbp_status st = lm_check_sizes(T, d, V, D, dtype);
  if (st != SBP_OK) return st;
  *bytes = lp_plan(lm_shape(T, d, V, D, dtype, 1), nullptr, nullptr);
  return SBP_OK;
}

// Per chunk c = [s, e): the logits Z_c = H_c W^T are formed by the GEMM and
// reduced on the fly -- bf16 with d % 128 == 0: the GEMM epilogue writes only
// the per-64-column (max, sum-exp) partials and each row's target logit, and
// lp_rows merges them; otherwise Z_c is written in fp32 and lp_rows passes
// over it.  Chunks without a valid token are skipped (their rows are zeros).
static sbp_status lmhead_logprob_impl(const void* H, const void* W, const int32_t* targets,
                                      int64_t T, int64_t d, int64_t V, int32_t D,
                                      int32_t dtype, float* logprob, float* lse, void* ws,
                                      size_t ws_bytes, void* stream) {
  sbp_status st = lm_check_sizes(T, d, V, D, dtype);
  if (st != SBP_OK) return st;
  if (!H || !W || !targets || !logprob)
    return set_error(SBP_ERR_INVALID_ARG, "H, W, targets and logprob must be non-NULL");
  if (misaligned(H) || misaligned(W) || misaligned(targets) || misaligned(logprob) || misaligned(lse) ||
      misaligned(ws))
    return set_error(SBP_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  const LmShape s = lm_shape(T, d, V, D, dtype, 1);
  const size_t need = lp_plan(s, nullptr, nullptr);
  if (!ws || ws_bytes < need)
    return set_error(SBP_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
  LpWs w;
  lp_plan(s, (char*)ws, &w);
  hipStream_t str = (hipStream_t)stream;
  const char* Hb = (const char*)H;
  sbp_status r = lm_prep(targets, T, V, D, 1, SBP_SUM, 0, w.prep, str);
  for (int32_t c = 0; c < D && r == SBP_OK; ++c) {
    int64_t s0, e0;
    chunk_bounds(T, D, c, &s0, &e0);
    const int64_t Tc = e0 - s0;
    GemmParams g;
    g.A = Hb + s0 * d * s.esz; g.lda = d;
    g.B = W; g.ldb = d;
    g.M = (int)Tc; g.N = (int)V; g.K = (int)d;
    g.active = w.prep.chunk_active + c;
    g.m_fastest = 1;
    if (s.fused_stats) {
      g.row_stats = w.parts;
      g.ld_stats = s.nparts;
      g.row_target = targets + s0;
      g.target_out = w.zt;
      r = gemm_nt(dtype, EPI_LSE_TGT, g, GEMM_TILE_RING, str, "gemm_logits_lp");
      if (r == SBP_OK)
        r = lp_rows(w.parts, s.nparts, s.nparts, w.zt, nullptr, 0, V, targets, s0, Tc, logprob, lse, str);
    } else {
      g.C = w.Z; g.ldc = s.Vp;
      r = gemm_nt(dtype, EPI_F32, g, GEMM_TILE_RING, str, "gemm_logits_lp");
      if (r == SBP_OK)
        r = lp_rows(nullptr, 0, 0, nullptr, w.Z, s.Vp, V, targets, s0, Tc, logprob, lse, str);
    }
  }
  return r;
}

extern "C" sbp_status sbp_lmhead_ce_fwd_bwd(const void* H, const void* W, const int32_t* targets,
                                            const float* weights, int64_t T, int64_t d, int64_t V,
                                            int32_t D, int32_t dtype, int32_t reduction,
                                            int32_t accumulate, float* loss, float* token_loss,
                                            void* dH, float* dW, void* ws, size_t ws_bytes,
                                            void* stream) {
  clear_error();
  sbp_status st = debug_check_targets(targets, T, V, (hipStream_t)stream);
  if (st != SBP_OK) return st;
  st = lmhead_ce_impl(H, W, targets, weights, T, d, V, D, dtype, reduction, accumulate, loss,
                      token_loss, dH, dW, ws, ws_bytes, stream);
  return st == SBP_OK ? debug_sync((hipStream_t)stream, "sbp_lmhead_ce_fwd_bwd") : st;
}

extern "C" sbp_status sbp_lmhead_logprob_fwd(const void* H, const void* W, const int32_t* targets,
                                             int64_t T, int64_t d, int64_t V, int32_t D,
                                             int32_t dtype, float* logprob, float* lse, void* ws,
                                             size_t ws_bytes, void* stream) {
  clear_error();
  sbp_status st = debug_check_targets(targets, T, V, (hipStream_t)stream);
  if (st != SBP_OK) return st;
  st = lmhead_logprob_impl(H, W, targets, T, d, V, D, dtype, logprob, lse, ws, ws_bytes, stream);
  return st == SBP_OK ? debug_sync((hipStream_t)stream, "sbp_lmhead_logprob_fwd") : st;
}
