// bf16 MFMA GEMM instantiations for operand layout AT=0, BT=1.
#include "gemm_mfma.h"
GEMM_MFMA_DEFINE_DISPATCH(false, true)
