// Single-kernel entry points (include/gpt2_ops.h).
#include <cstring>
#include <mutex>

#include "../../include/gpt2_ops.h"
#include "kernels.h"

namespace {

// Device scratch of gpt2_op_attention_bwd_noalloc: the per-(b, h, t) row term
// D = rowsum(dO o O) that the dQ pass writes and the dK/dV pass reads.  Every
// GPU the library runs on holds its own copy of this array until the process
// ends.  In host code `attn_scratch` only names the symbol: kernels get the
// per-device address from hipGetSymbolAddress.
constexpr long ATTN_SCRATCH_FLOATS = 1L << 20;
__device__ __align__(256) float attn_scratch[ATTN_SCRATCH_FLOATS];

constexpr int MAX_DEVICES = 64;
float* scratch_ptr[MAX_DEVICES];
hipError_t scratch_err[MAX_DEVICES];
std::once_flag scratch_once[MAX_DEVICES];

// The address of attn_scratch on the current device, looked up once per
// device with that device current.
hipError_t attn_scratch_on_current_device(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::call_once(scratch_once[dev], [dev] {
    void* p = nullptr;
    scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(attn_scratch));
    scratch_ptr[dev] = static_cast<float*>(p);
  });
  *out = scratch_ptr[dev];
  return scratch_err[dev];
}

}  // namespace

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

gpt2_status gpt2_op_gemm_epi(int M, int N, int K, const void* A, long lda, const void* B, long ldb,
                             int epi, const float* bias, const float* R, long ldr, void* C,
                             void* C2, long ldc, int out_dtype, void* hip_stream) {
  if (!A || !B || !C || M < 0 || N < 0 || K < 0 || epi < 0 || epi > 2) return GPT2_E_ARG;
  if (out_dtype != (epi == 2 ? GPT2_FP32 : GPT2_BF16)) return GPT2_E_ARG;
  if (epi == 1 && !C2) return GPT2_E_ARG;
  if (epi == 2 && (!R || ldr % 4)) return GPT2_E_ARG;
  if (ldc % 8 || K % 8) return GPT2_E_ARG;
  EpiArgs e;
  std::memset(&e, 0, sizeof(e));
  e.out = C;
  e.out2 = C2;
  e.ldo = ldc;
  e.alpha = 1.f;
  e.bias = bias;
  e.resid = R;
  e.ldr = ldr;
  const int kind = epi == 0 ? EPI_BIAS : epi == 1 ? EPI_BIAS_GELU : EPI_RESID;
  hipError_t r = launch_gemm(DT_BF16, M, N, K, A, lda, false, B, ldb, false, kind,
                             out_dtype == GPT2_BF16 ? DT_BF16 : DT_F32, e, 1,
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

gpt2_status gpt2_op_attention_bwd_noalloc(int dtype, const void* qkv, const void* y,
                                          const float* lse, const void* dy, void* dqkv, int B,
                                          int T, int H, int hd, void* hip_stream) {
  if (!qkv || !y || !lse || !dy || !dqkv || B < 1 || T < 1 || H < 1) return GPT2_E_ARG;
  if ((long)B * H * T > ATTN_SCRATCH_FLOATS) return GPT2_E_ARG;
  float* d = nullptr;
  if (attn_scratch_on_current_device(&d) != hipSuccess || !d) return GPT2_E_HIP;
  hipError_t r = launch_attn_bwd(dtype == GPT2_BF16 ? DT_BF16 : DT_F32, qkv, y, lse, dy, dqkv, d,
                                 B, T, H, hd, nullptr, reinterpret_cast<hipStream_t>(hip_stream));
  if (r == hipErrorInvalidValue) return GPT2_E_ARG;
  return r == hipSuccess ? GPT2_OK : GPT2_E_HIP;
}

}  // extern "C"
