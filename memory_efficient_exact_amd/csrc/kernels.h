// Internal kernel launchers of libstreambp (not part of the C ABI).
#pragma once

#include "common.h"

namespace sbp {

// ---------------------------------------------------------------- GEMM ----
// EPI_REL16_LSE: the (max, sum-exp) of every 64-column quarter of a tile row
// (columns < N) into row_stats, and into C (fp16, pitch ldc) each value minus
// the max of its quarter (so <= 0: the values near 0 that dominate a softmax
// keep ~11 bits; the quarter's max, kept in fp32 in row_stats, restores the
// value), and, when target_out is set, the fp32 value at each row's target
// column as for EPI_LSE_TGT (ring kernel only, k_split 1).
// EPI_LSE_TGT: the row statistics of EPI_REL16_LSE and, for each row m with
// 0 <= row_target[m] < N, its value at that column into target_out[m]; C is
// not written (ring kernel only, k_split 1).
enum { EPI_F32 = 0, EPI_F32_ACC = 1, EPI_OUT = 2, EPI_OUT_RESID = 3, EPI_PARTIAL = 4, EPI_REL16_LSE = 5,
       EPI_LSE_TGT = 6 };
enum { GEMM_TILE_128 = 0, GEMM_TILE_RING = 3 };

struct GemmParams {
  const void* A = nullptr;  // [M, K] row-major, K contiguous, pitch lda elements ([K, M] if a_kmajor)
  const void* B = nullptr;  // [N, K] row-major, pitch ldb ([K, N] if b_kmajor)
  void* C = nullptr;        // [M, N] pitch ldc (fp32 for F32/F32_ACC/PARTIAL, else dtype)
  const void* R = nullptr;  // residual [M, N] pitch ldr (EPI_OUT_RESID)
  int64_t lda = 0, ldb = 0, ldc = 0, ldr = 0;
  // K % 8 == 0 (bf16) / K % 4 == 0 (fp32); lda/ldb likewise.  The bf16 ring
  // GEMM with K-major operands takes any K.
  int M = 0, N = 0, K = 0;
  float alpha = 1.f;
  int beta = 0;                    // EPI_F32_ACC: C = acc + beta * C
  const int* beta_zero = nullptr;  // EPI_F32_ACC: device flag, non-zero forces beta = 0
  const int* active = nullptr;     // device flag, 0 -> the whole launch is a no-op
  int k_split = 1;                 // EPI_PARTIAL: number of K ranges
  int k_per_split = 0;             // multiple of the K step (0 = even split)
  int64_t split_stride = 0;        // EPI_PARTIAL: elements between partial outputs
  int m_fastest = 1;               // tile order inside an XCD's range (register-staged kernel only)
  // bf16 ring GEMM only: both operands stored K-major, A as [K, M] and B as
  // [K, N], with pitches lda >= round_up(M, 8) and ldb >= round_up(N, 8)
  // between k-rows (rows are read in 8-element chunks up to that bound);
  // the two flags must be equal
  int a_kmajor = 0, b_kmajor = 0;
  float2* row_stats = nullptr;     // EPI_REL16_LSE, EPI_LSE_TGT: [M, ld_stats], entry 4 tn + quarter
  int64_t ld_stats = 0;
  const int32_t* row_target = nullptr;  // EPI_LSE_TGT: [M] column of each row (< 0: none)
  float* target_out = nullptr;          // EPI_LSE_TGT: [M]
  // bf16 ring GEMM only (k_split 1): tile-aligned splits (multiples of 256)
  // that let one launch cover products whose operands or results live in
  // separate buffers.  Rows n >= b_split of a row-major B come from B2 (row n
  // at B2 + (n - b_split) ldb).  Output tiles at or past c_split[i] (rows, or
  // columns if c_split_cols) go to Cx[i]: element (r, c) at Cx[i] +
  // (r - c_split[i]) ldc + c, or r ldc + (c - c_split[i]); c_split[0] <
  // c_split[1], the last one reached wins.  EPI_OUT, EPI_F32, EPI_F32_ACC.
  const void* B2 = nullptr;
  int b_split = 0;
  void* Cx[2] = {nullptr, nullptr};
  int c_split[2] = {0, 0};
  int c_split_cols = 0;
  int tiles_m = 0, tiles_n = 0;    // filled by the launcher
};

int gemm_k_granule(int dtype);
sbp_status gemm_nt(int dtype, int epi, GemmParams p, int tile, hipStream_t st, const char* name);

// ------------------------------------------------------- LM head + CE ----
struct LmPrep {   // device-side scalars written by lm_prep
  int* n_valid;       // [1]
  float* inv_norm;    // [1]  1/N (mean_valid, N>0), 1 (sum), 0 (N == 0), NaN (a target >= V)
  int* chunk_active;  // [D]
  int* group_active;  // [ceil(D/G)]  1 if a chunk of dW group g (chunks gG .. gG+G-1) is active
  int* beta_zero;     // [ceil(D/G)]  1 for the group whose dW GEMM must overwrite
  int* none_active;   // [1]  1 if no chunk has a valid token
};
// A target id >= V (a caller error) sets inv_norm to NaN.
sbp_status lm_prep(const int32_t* targets, int64_t T, int64_t V, int32_t D, int32_t G,
                   int reduction, int accumulate, const LmPrep& pr, hipStream_t st);
// Per-row log-sum-exp and per-token loss for rows [s, s+Tc) of one chunk.
// Row statistics from the logits GEMM's per-64-column partials (nparts per
// row, pitch ldp): lse, l_t = lse - z_t[y_t], c_t l_t, with z_t[y_t] the fp32
// target logit the GEMM wrote into zt [Tc].
sbp_status ce_merge(const float2* parts, int64_t ldp, int nparts, const float* zt,
                    const int32_t* targets, const float* weights, int64_t s, int64_t Tc, int64_t V,
                    float* lse, float* loss_part, float* token_loss, hipStream_t st);
sbp_status ce_stats(const float* Z, int64_t ldz, const int32_t* targets, const float* weights,
                    int64_t s, int64_t Tc, int64_t V, float* lse, float* loss_part,
                    float* token_loss, hipStream_t st);
// dZ (dtype) [Tc, ldg] and, if dZt is not NULL, dZ^T (dtype) [Vp, ldgt] for
// one chunk; zero pads (columns V .. Vp of dZ, columns Tc .. Tcp of dZ^T).
// Z: fp32 logits [Tc, ldz], or, when parts is not NULL, the fp16 relative
// logits of EPI_REL16_LSE with their group maxima in parts [Tc, ldp] (bf16
// output without dZ^T only; dZ may then be Z, ldg == ldz: in place).
sbp_status ce_grad(int dtype, const void* Z, const float2* parts, int64_t ldp, int64_t ldz,
                   const int32_t* targets, const float* weights, const float* inv_norm,
                   const float* lse, int64_t s, int64_t Tc, int64_t V, int64_t Vp, void* dZ,
                   int64_t ldg, void* dZt, int64_t ldgt, int64_t Tcp, const int* active,
                   hipStream_t st);
// Per-token target log-probability of rows [s, s+Tc) of one chunk:
// logprob[s+r] = z_r[y] - lse_r and (if lse_out is not NULL) lse_out[s+r] =
// lse_r, both 0 where y = targets[s+r] < 0 and NaN where y >= V.  From the logits GEMM's
// per-64-column partials and target logits zt[r] when parts is not NULL,
// else from a pass over the fp32 logits Z [Tc, ldz] (V columns).
sbp_status lp_rows(const float2* parts, int64_t ldp, int nparts, const float* zt, const float* Z,
                   int64_t ldz, int64_t V, const int32_t* targets, int64_t s, int64_t Tc,
                   float* logprob, float* lse_out, hipStream_t st);
sbp_status loss_reduce(const float* loss_part, int64_t T, const float* inv_norm, float* loss,
                       hipStream_t st);

// ------------------------------------------------------------ helpers ----
// dst[c][r] = src[r][c] for r < R, 0 for R <= r < Rp; c < C.
sbp_status transpose_pad(int dtype, const void* src, int64_t lds_, int64_t R, int64_t C,
                         void* dst, int64_t ldd, int64_t Rp, const int* active, hipStream_t st);
// out[m][n] = sum_s part[s][m][n] (or 0 where *active == 0), cast to dtype.
sbp_status splitk_reduce(int dtype, const float* part, int64_t split_stride, int S, int64_t M,
                         int64_t N, int64_t ldp, void* out, int64_t ldo, const int* active,
                         hipStream_t st);
// Fill n floats with 0 when *when != 0 (unconditionally when `when` is null).
sbp_status fill_zero_f32(float* p, int64_t n, const int* when, hipStream_t st);
sbp_status fill_zero_bytes(void* p, int64_t nbytes, hipStream_t st);

// ------------------------------------------------------- decoder layer ----
// Token-wise kernels take bf16 rows, or fp32 rows with dtype SBP_F32.
sbp_status rmsnorm_fwd(const void* x, int64_t ldx, const void* g, int64_t rows, int64_t d,
                       float eps, void* out, int64_t ldo, float* rinv, hipStream_t st,
                       int dtype = SBP_BF16);
// out = resid + RMSNorm'(dn) (resid may be NULL)
sbp_status rmsnorm_bwd(const void* x, int64_t ldx, const void* g, const float* dn, int64_t ldn,
                       const float* rinv, const void* resid, int64_t ldr, int64_t rows, int64_t d,
                       void* out, int64_t ldo, hipStream_t st, int dtype = SBP_BF16);
// part: gain_grad_splits(rows) * d floats of scratch
int gain_grad_splits(int64_t rows);
sbp_status gain_grad(const float* dn, int64_t ldn, const void* x, int64_t ldx, const float* rinv,
                     int64_t rows, int64_t d, float* dg, int beta, float* part, hipStream_t st,
                     int dtype = SBP_BF16);
sbp_status swiglu_fwd(const void* ug, int64_t rows, int64_t F, void* m, hipStream_t st,
                      int dtype = SBP_BF16);
sbp_status swiglu_bwd(const void* dm, const void* ug, int64_t rows, int64_t F, void* dudg,
                      hipStream_t st, int dtype = SBP_BF16);
sbp_status rows_to_bf16(const float* src, int64_t lds_, int64_t rows, int64_t cols, void* dst,
                        int64_t ldd, hipStream_t st);
sbp_status rows_to_f32(const void* src, int64_t lds_, int64_t rows, int64_t cols, float* dst,
                       int64_t ldd, hipStream_t st);
// QK-norm: RMSNorm of each head vector (width dh in {64, 128}) of rows x H
// heads, one gain g [dh] for all heads.  headnorm_fwd: out may equal x.
// headnorm_bwd: dx (may equal dy) from x, dy; dg (+)= sum dy * xhat (beta 1
// adds) through part [HEADNORM_PARTS, dh] floats of scratch.
constexpr int HEADNORM_PARTS = 1024;
sbp_status headnorm_fwd(const void* x, int64_t ldx, void* out, int64_t ldo, int64_t rows, int H,
                        int dh, const void* g, float eps, hipStream_t st, int dtype = SBP_BF16);
sbp_status headnorm_bwd(const void* x, int64_t ldx, const void* dy, int64_t ldy, void* dx,
                        int64_t ldd, int64_t rows, int H, int dh, const void* g, float eps,
                        float* dg, int beta, float* part, hipStream_t st, int dtype = SBP_BF16);
// Rotary embedding: tab [P, dh/2] of (cos, sin) for positions 0 .. P-1;
// rope_apply turns rows [0, rows) of src (H heads of width dh, fp32 or bf16,
// pitch lds_) into dst (bf16, or fp32 from fp32 with dst_f32; pitch ldd;
// dst == src allowed when the types match), row r
// at position row0 + r - seq_lo[row0 + r] (seq_lo NULL: row0 + r);
// inverse turns by the negative angle.
sbp_status rope_table(float2* tab, int64_t P, int dh, double theta, hipStream_t st);
sbp_status rope_apply(const void* src, bool src_f32, int64_t lds_, void* dst, int64_t ldd,
                      int64_t rows, int H, int dh, int64_t row0, const int* seq_lo,
                      const float2* tab, bool inverse, hipStream_t st, bool dst_f32 = false);

// ------------------------------------------- decoder layer, fp32 mode ----
// (layer_f32.hip) Workspace bytes and the two runs; the arguments are
// checked by the entry points in layer.hip.
size_t layer_f32_ws(const sbp_layer_desc* desc, int32_t D, bool bwd, bool packed);
sbp_status layer_f32_bwd(const sbp_layer_desc* desc, const int32_t* cu, int32_t nseq, const void* x,
                         const void* dy, const sbp_layer_weights* w, int32_t D, int32_t accumulate,
                         void* dx, sbp_layer_grads* g, void* ws, hipStream_t st);
sbp_status layer_f32_fwd(const sbp_layer_desc* desc, const int32_t* cu, int32_t nseq, const void* x,
                         const sbp_layer_weights* w, int32_t D, void* y, void* ws, hipStream_t st);

// ------------------------------------------------------------ debug mode ----
// SBP_DEBUG set (and not "0"): device-side input checks before a call's
// launches, and a stream synchronisation after them (debug.hip).
bool debug_on();
sbp_status debug_check_targets(const int32_t* targets, int64_t T, int64_t V, hipStream_t st);
sbp_status debug_check_cu(const int32_t* cu, int nseq, int64_t T, hipStream_t st);
sbp_status debug_sync(hipStream_t st, const char* call);

}  // namespace sbp
