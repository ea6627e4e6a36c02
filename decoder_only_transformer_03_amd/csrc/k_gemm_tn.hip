// bf16 MFMA GEMM instantiations for operand layout AT=1, BT=1.
#include "gemm_mfma.h"
GEMM_MFMA_DEFINE_DISPATCH(true, true)

hipError_t launch_gemm_grouped_wgrad(const GemmProblem* d_probs, int nprobs, long total_tiles,
                                     int K, float scale, bool store, hipStream_t s) {
  return gemm_mfma::run_grouped_accum_tt(d_probs, nprobs, total_tiles, K, scale, store, s);
}
