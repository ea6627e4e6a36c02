// bf16 MFMA GEMM instantiations for operand layout AT=0, BT=0.
#include "gemm_mfma.h"
GEMM_MFMA_DEFINE_DISPATCH(false, false)

// Workgroup slots of the persistent GEMM grid (about one per CU).
int gemm_slots() { return gemm_mfma::persistent_slots(); }
