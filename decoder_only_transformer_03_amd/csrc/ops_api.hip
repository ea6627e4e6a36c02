// Single-kernel entry points (include/gpt2_ops.h).
#include <cstring>

#include "../../include/gpt2_ops.h"
#include "kernels.h"

extern "C" {

gpt2_status gpt2_op_gemm(int dtype, int M, int N, int K, const void* A, long lda, int a_trans,
                         const void* B, long ldb, int b_trans, float* C, long ldc, float alpha,
                         int mode, int split_k, void* hip_stream) {
  if (!A || !B || !C || M < 0 || N < 0 || K < 0 || mode < 0 || mode > 2) return GPT2_E_ARG;
  if (dtype != GPT2_FP32 && dtype != GPT2_BF16) return GPT2_E_ARG;
  if (a_trans && !b_trans && dtype == GPT2_BF16) return GPT2_E_ARG;
  EpiArgs e;
  std::memset(&e, 0, sizeof(e));
  e.out = C;
  e.ldo = ldc;
  e.alpha = alpha;
  int epi = mode == 0 ? EPI_STORE : mode == 1 ? EPI_ACCUM : EPI_ATOMIC;
  hipError_t r = launch_gemm(dtype == GPT2_BF16 ? DT_BF16 : DT_F32, M, N, K, A, lda, a_trans != 0,
                             B, ldb, b_trans != 0, epi, DT_F32, e, mode == 2 ? split_k : 1,
                             reinterpret_cast<hipStream_t>(hip_stream));
  if (r == hipErrorInvalidValue) return GPT2_E_ARG;
  return r == hipSuccess ? GPT2_OK : GPT2_E_HIP;
}

gpt2_status gpt2_op_attention_fwd(int dtype, const void* qkv, void* y, float* lse, int B, int T,
                                  int H, int hd, void* hip_stream) {
  if (!qkv || !y || !lse || B < 1 || T < 1 || H < 1) return GPT2_E_ARG;
  hipError_t r = launch_attn_fwd(dtype == GPT2_BF16 ? DT_BF16 : DT_F32, qkv, y, lse, B, T, H, hd,
                                 reinterpret_cast<hipStream_t>(hip_stream));
  if (r == hipErrorInvalidValue) return GPT2_E_ARG;
  return r == hipSuccess ? GPT2_OK : GPT2_E_HIP;
}

gpt2_status gpt2_op_attention_bwd(int dtype, const void* qkv, const void* y, const float* lse,
                                  const void* dy, void* dqkv, float* dbuf, int B, int T, int H,
                                  int hd, void* hip_stream) {
  if (!qkv || !y || !lse || !dy || !dqkv || !dbuf || B < 1 || T < 1 || H < 1) return GPT2_E_ARG;
  hipError_t r = launch_attn_bwd(dtype == GPT2_BF16 ? DT_BF16 : DT_F32, qkv, y, lse, dy, dqkv,
                                 dbuf, B, T, H, hd, nullptr,
                                 reinterpret_cast<hipStream_t>(hip_stream));
  if (r == hipErrorInvalidValue) return GPT2_E_ARG;
  return r == hipSuccess ? GPT2_OK : GPT2_E_HIP;
}

}  // extern "C"
