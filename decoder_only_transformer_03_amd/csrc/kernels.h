// Host-side launchers of the libgpt2 kernels (internal interface).
#pragma once
#include <hip/hip_runtime.h>
#include "common.h"
#include "epilogue.h"

enum DType : int { DT_F32 = 0, DT_BF16 = 1 };

// LayerNorm backward: rows per workgroup (partials of dw/db/dsum are per workgroup).
// 32 at B*T = 16384, C = 768: two workgroups per CU; 16, 40 and 64 rows measured
// 4%, 7% and 12% slower, 24 the same.
constexpr int LN_BWD_ROWS = 32;
// bias-gradient column sums: row splits (partials of width N each)
constexpr int BIAS_SPLITS = 64;
// floats of partials launch_layernorm_bwd writes for rows x C
inline long ln_bwd_scratch(long rows, int C) {
  return ((rows + LN_BWD_ROWS - 1) / LN_BWD_ROWS) * 3L * C;
}

// One matrix of partial column sums (nparts x ncols, row-major) whose column
// sums go to up to three destinations: dst[k][j] += sum over the parts of
// column k*w + j (null: skipped).  nparts = ceil(M / rows_per_part) for the
// launch's M when rows_per_part > 0, the launch's nblk when rows_per_part < 0,
// else fixed_parts.  chunk0: the problem's
// first 64-column chunk in the launch (problems in order, chunks contiguous).
struct ColsumProblem {
  const float* partial;
  float* dst[3];
  int ncols, w;
  int rows_per_part, fixed_parts;
  int chunk0;
};
// store: dst = sum instead of dst += sum.
hipError_t launch_colsum_grouped(const ColsumProblem* d_probs, int nprobs, int total_chunks, long M,
                                 int nblk, bool store, hipStream_t s);
// grad-norm: workgroups of the sum-of-squares pass (fp64 partials)
constexpr int NORM_PARTS = 1024;

struct AdamChunk {
  long start;  // first element in the flat parameter vector (multiple of 4)
  int len;     // elements (multiple of 4)
  int flags;   // bit 0: weight decay applies (tensor has dim >= 2)
};

// One 64 x 64 tile of a row-major bf16 matrix (rows x cols) at element
// offset `off`, with its first row and column.
struct TTile {
  long off;
  int rows, cols, r0, c0;
};
// dst (same offset) = the transpose, cols x rows, of every listed tile.
hipError_t launch_transpose_tiles(const bf16_t* src, bf16_t* dst, const TTile* tiles, int ntiles,
                                  hipStream_t s);

int ln_bwd_blocks(long rows);

hipError_t launch_embed_fwd(const int32_t* idx_in, int32_t* idx_saved, const float* wte,
                            const float* wpe, float* x, int B, int T, int C, int Vp, int* err,
                            hipStream_t s);
// dwte[idx[r]] += dx[r] over the B*T rows (deterministic; ids in [0, Vp)),
// dwpe[t] += sum_b dx[b,t] (wpe_store: dwpe[t] = ..., rows T.. untouched);
// scratch: embed_bwd_scratch_bytes(B*T, C) bytes.
size_t embed_bwd_scratch_bytes(long rows, int C);
hipError_t launch_embed_bwd(const int32_t* idx, const float* dx, float* dwte, float* dwpe, int B,
                            int T, int C, int Vp, void* scratch, bool wpe_store, hipStream_t s);
hipError_t launch_layernorm_fwd(DType out_t, const float* x, const float* w, const float* b,
                                void* y, float* mean, float* rstd, long rows, int C,
                                hipStream_t s);
// LayerNorm backward into dres; partial (ln_bwd_scratch(rows, C) floats)
// receives per-workgroup rows [dw | db | column sums of the new dres] of width
// 3C each, ceil(rows / LN_BWD_ROWS) of them, for a column-sum launch.
hipError_t launch_layernorm_bwd(DType copy_t, const float* dy, const float* x, const float* mean,
                                const float* rstd, const float* w, float* dres, void* dres_copy,
                                int accumulate, float* partial, long rows, int C, hipStream_t s);
// partial[BIAS_SPLITS][N]: column sums of X (rows x N, row stride ldx) over
// BIAS_SPLITS row slices.
hipError_t launch_colsum_parts(DType in_t, const void* X, long rows, int N, long ldx, float* partial,
                               hipStream_t s);
// Fused softmax cross-entropy; with grad the logits are overwritten by
// d(loss)/d(logits), without only the losses are formed.
hipError_t launch_xent(DType t, void* logits, const int32_t* targets, int* n_valid,
                       float* row_loss, float* loss, long rows, int Vp, int* err, bool grad,
                       hipStream_t s);
// Fused lm_head loss from EPI_LSE partials: counts the rows with a target,
// writes lse and row_loss per row and the mean loss.
hipError_t launch_head_loss(const float* part, int nblk, const float* tlogit,
                           const int32_t* targets, int* n_valid, float* lse, float* row_loss,
                           float* loss, long rows, int Vp, int* err, hipStream_t s);
// One draw per row: temperature, top-k (<= 0: all), inverse CDF of uni[r * u_stride];
// the token goes to out[r * out_stride].  logits 16-byte aligned, ld % 4 == 0.
hipError_t launch_sample(const float* logits, long ld, int rows, int V, float temperature,
                         int top_k, const float* uni, long u_stride, int32_t* out,
                         long out_stride, hipStream_t s);
hipError_t launch_seq_loss(const float* row_loss, const int32_t* targets, int B, int T,
                           float* seq_loss, hipStream_t s);
hipError_t launch_grad_norm(const float* g, long n, double* partial, float max_norm,
                            float* norm_out, float* clip_out, hipStream_t s);
hipError_t launch_adamw(const AdamChunk* chunks, int nchunks, float* p, const float* g, float* m,
                        float* v, bf16_t* shadow, const float* clip, float lr, float b1, float b2,
                        float eps, float wd, float step_size, float inv_sqrt_bc2, hipStream_t s);
// AdamW on the 64 x 64 tiles of decayed matrices, also writing the bf16 copy
// (shadow) and its transpose (shadow_t, same offset, cols x rows).
hipError_t launch_adamw_tiles(const TTile* tiles, int ntiles, float* p, const float* g, float* m,
                              float* v, bf16_t* shadow, bf16_t* shadow_t, const float* clip,
                              float lr, float b1, float b2, float eps, float wd, float step_size,
                              float inv_sqrt_bc2, hipStream_t s);
hipError_t launch_fill(float* p, long n, float val, hipStream_t s);
// p[i] = std * (standard normal number e0 + i of the stream of `seed`), for
// 0 <= i < n (Philox4x32-10 counters, Box-Muller; k_init.hip).
hipError_t launch_init_normal(float* p, long n, long e0, float std, uint64_t seed, hipStream_t s);
hipError_t launch_f32_to_bf16(const float* src, bf16_t* dst, long n, hipStream_t s);

// C[m][n] = sum_k A(m,k) B(n,k) followed by epilogue `epi`, where
// A(m,k) = a_t ? A[k*lda + m] : A[m*lda + k] and B(n,k) = b_t ? B[k*ldb + n] : B[n*ldb + k].
// Operands are `in_t`; the epilogue's TO type is `out_t`.  split_k > 1 is
// only valid with EPI_ATOMIC; 0 lets the launcher choose.
hipError_t launch_gemm(DType in_t, int M, int N, int K, const void* A, long lda, bool a_t,
                       const void* B, long ldb, bool b_t, int epi, DType out_t, const EpiArgs& e,
                       int split_k, hipStream_t s);

// launch_gemm for the forward epilogues (STORE, BIAS, BIAS_GELU, RESID) that,
// when the output has too few tiles to fill the GPU and K is deep enough,
// splits K into fp32 slices of `part` and applies the epilogue to their sum
// in a second pass (same result up to the order of the fp32 additions).
hipError_t launch_gemm_fill(DType in_t, int M, int N, int K, const void* A, long lda, bool a_t,
                            const void* B, long ldb, bool b_t, int epi, DType out_t,
                            const EpiArgs& e, float* part, long part_elems, hipStream_t s);

// Weight gradient out[m][n] += alpha * sum_k A(m,k) B(n,k) for a long
// contraction: split over k into fp32 slices of `part` (part_elems floats of
// scratch), then summed in fixed order into out (deterministic).  store:
// out = instead of out +=.
int gemm_slots();  // workgroup slots of the persistent bf16 GEMM grid
hipError_t launch_gemm_wgrad(DType in_t, int M, int N, int K, const void* A, long lda, bool a_t,
                             const void* B, long ldb, bool b_t, float* out, long ldo, float alpha,
                             float* part, long part_elems, hipStream_t s, bool store = false);
int gemm_partial_splits(DType in_t, int M, int N, int K);

// One product of a grouped weight-gradient launch:
// out[m*ldo + n] += a * sum_k A[k*lda + m] B[k*ldb + n], m < M, n < N, with
// a = alpha, times the launch's scale if `scaled`; its tiles_m x tiles_n
// 256 x 256 tiles are numbered from item0 in the group.
struct GemmProblem {
  const bf16_t* A;
  const bf16_t* B;
  float* out;
  long lda, ldb, ldo;
  int M, N, tiles_m, tiles_n;
  long item0;
  float alpha;
  int scaled;
};
// All products of d_probs (device array, nprobs entries, item0 ascending
// from 0, total_tiles in all) in one persistent launch; bf16 operands, K a
// multiple of 64, whole tiles (no k-slices): deterministic.
// store: out_p = instead of out_p +=.
hipError_t launch_gemm_grouped_wgrad(const GemmProblem* d_probs, int nprobs, long total_tiles,
                                     int K, float scale, bool store, hipStream_t s);
constexpr long SPLITK_PART_ELEMS = 256L * 256 * 256;

// Causal self-attention on the fused qkv activation (B*T, 3C), head h of q,
// k, v at columns h*hd, C + h*hd, 2C + h*hd.  y is (B*T, C) with heads
// re-interleaved; lse is (B, H, T), natural log of the scaled, masked scores.
hipError_t launch_attn_fwd(DType t, const void* qkv, void* y, float* lse, int B, int T, int H,
                           int hd, hipStream_t s);
// Gradients into dqkv (B*T, 3C) given dy (B*T, C); dbuf (B, H, T) fp32 scratch.
// bias_part (bf16 only; null: skipped): row b*ceil(T/128) + j receives the
// column sums of dqkv over rows j*128 .. j*128+127 of sequence b, width 3C.
hipError_t launch_attn_bwd(DType t, const void* qkv, const void* y, const float* lse,
                           const void* dy, void* dqkv, float* dbuf, int B, int T, int H, int hd,
                           float* bias_part, hipStream_t s);

// Few rows (M <= 16) of a linear layer whose input is LayerNorm(x) (x fp32,
// M x K row-major, LayerNorm weight lnw and bias lnb): C = LN(x) B^T with
// the bf16 rounding of LN(x) that layernorm_fwd + the GEMM would give, in
// one launch; the epilogue as for launch_gemm (e.out etc.).  K a multiple of
// 32 and at most LN_SKINNY_MAX_K (the normalised rows are held in LDS).
constexpr int LN_SKINNY_MAX_K = 2048;
hipError_t launch_gemm_ln_skinny(int M, int N, int K, const float* x, const float* lnw,
                                 const float* lnb, const void* B, long ldb, int epi, DType out_t,
                                 const EpiArgs& e, hipStream_t s);

// Key/value cache of the decoding path: per block (B, bs, 2C) [k | v] rows.
// kv_append: the k, v parts of qkv rows (B*T, 3C) into positions pos0 .. pos0+T-1.
hipError_t launch_kv_append(DType t, const void* qkv, void* cache, int B, int Tn, int pos0, int bs,
                            int C, hipStream_t s);
// attention of one new position p per sequence over the cached positions
// 0 .. p: appends position p's key and value (from row b of qkv (B, 3C)) to
// the cache, then attends with q from that row; output row b of y (B, C)
constexpr int ATTN_DECODE_MAX_POS = 8192;  // fp32 path: scores of one (b, h) in LDS (33 KB)
hipError_t launch_attn_decode(DType t, const void* qkv, void* cache, void* y, int B, int p, int bs,
                              int H, int hd, hipStream_t s);
