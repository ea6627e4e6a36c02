/*
 * gpt2_ops.h - single-kernel entry points of libgpt2.so on caller-owned
 * device buffers.  They run the same kernels as the training step and exist
 * for layer-by-layer comparison against a reference (compare every
 * intermediate on the same input; rounding-level differences are expected,
 * larger ones locate a bug - "Reproducing GPT-2: How a Hidden Bug Affected
 * Weight Training", layer-by-layer comparison of activations).
 *
 * All pointers are device pointers; work is enqueued on hip_stream
 * (hipStream_t as void*, NULL = default stream) and the call returns without
 * waiting.  dtype is GPT2_FP32 (operands float) or GPT2_BF16 (operands bf16,
 * stored as uint16, fp32 accumulation).  Nothing is allocated.  Returns
 * GPT2_E_ARG for an unsupported shape/alignment and GPT2_E_HIP if the launch
 * fails.
 */
#ifndef GPT2_OPS_H
#define GPT2_OPS_H
#include "gpt2.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix product of a linear layer ("GPT-2 from Scratch": every nn.Linear):
 *   C[m][n] = alpha * sum_k A(m,k) B(n,k)            mode 0: store
 *   C[m][n] += alpha * sum_k A(m,k) B(n,k)           mode 1: accumulate
 *   same as mode 1, split over k with atomic adds     mode 2 (split_k 0 = auto)
 * A(m,k) = A[m*lda + k], or A[k*lda + m] if a_trans; B(n,k) = B[n*ldb + k], or
 * B[k*ldb + n] if b_trans; C is fp32 row-major with leading dimension ldc.
 * bf16 requires lda, ldb multiples of 8, K a multiple of 8 when an operand is
 * k-contiguous, M (N) a multiple of 8 when A (B) is transposed, N a multiple
 * of 4, and (a_trans, b_trans) != (1, 0). */
gpt2_status gpt2_op_gemm(int dtype, int M, int N, int K, const void* A, long lda, int a_trans,
                         const void* B, long ldb, int b_trans, float* C, long ldc, float alpha,
                         int mode, int split_k, void* hip_stream);

/* A linear layer's forward product with its fused epilogue ("GPT-2 from
 * Scratch": nn.Linear with bias; The MLP and GPT-2's GELU; The Block:
 * pre-LN and residuals), bf16 operands: h[m][n] = sum_k A[m*lda + k] B[n*ldb
 * + k] + bias[n] (bias may be NULL), then
 *   epi 0: C[m][n] = h                                  (bf16)
 *   epi 1: C[m][n] = gelu'(h), C2[m][n] = gelu(h)       (bf16, tanh form)
 *   epi 2: C[m][n] = R[m*ldr + n] + h                   (fp32; R may equal C)
 * out_dtype must name that output type (GPT2_BF16, GPT2_BF16, GPT2_FP32).
 * C and C2 are row-major with leading dimension ldc.  The same kernels the
 * model's forward pass runs: the tiled matrix-core GEMM, or for M <= 16 and K
 * a multiple of 32 the few-rows kernel of a decoding step.  Requires lda,
 * ldb, ldc multiples of 8, K a multiple of 8, N a multiple of 8 (else
 * GPT2_E_ARG, nothing enqueued). */
gpt2_status gpt2_op_gemm_epi(int M, int N, int K, const void* A, long lda, const void* B, long ldb,
                             int epi, const float* bias, const float* R, long ldr, void* C,
                             void* C2, long ldc, int out_dtype, void* hip_stream);

/* Causal self-attention forward ("CausalSelfAttention"): qkv is (B*T, 3C) in
 * dtype with [q | k | v] and head h at columns h*hd of each third; writes y
 * (B*T, C) in dtype with heads re-interleaved and lse (B, H, T) fp32, the
 * natural-log log-sum-exp of the scaled, masked scores of each query.
 * bf16 needs hd == 64; fp32 accepts hd 32 or 64. */
gpt2_status gpt2_op_attention_fwd(int dtype, const void* qkv, void* y, float* lse, int B, int T,
                                  int H, int hd, void* hip_stream);

/* Its backward: given dy (B*T, C) writes dqkv (B*T, 3C) in dtype; dbuf is
 * (B, H, T) fp32 scratch that receives D = rowsum(dy * y). */
gpt2_status gpt2_op_attention_bwd(int dtype, const void* qkv, const void* y, const float* lse,
                                  const void* dy, void* dqkv, float* dbuf, int B, int T, int H,
                                  int hd, void* hip_stream);

/* gpt2_op_attention_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same kernels and the same results, with the scratch for
 * D taken from a fixed array of 1,048,576 floats (4 MiB) that the library
 * keeps on each GPU it runs on, instead of a dbuf argument.  B * H * T may
 * not exceed 1,048,576 (GPT2_E_ARG, nothing enqueued).  Nothing is
 * allocated; the array's address on the current device is looked up on the
 * first call on that device, so hip_stream must belong to the current
 * device.  Every call on one GPU shares that GPU's array: calls that overlap
 * on one GPU (other streams, other threads) race and give wrong results.
 * Nothing in the array needs to start at a particular value: the dQ pass
 * writes every D it uses before the dK/dV pass reads it.  GPT2_E_HIP if the
 * lookup or a launch fails. */
gpt2_status gpt2_op_attention_bwd_noalloc(int dtype, const void* qkv, const void* y,
                                          const float* lse, const void* dy, void* dqkv, int B,
                                          int T, int H, int hd, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* GPT2_OPS_H */
