// MFMA product kernels for bf16 operands and weights (instantiation unit).
#include "gemm_mfma.h"

namespace q3 {

hipError_t gemm_part_bf16(const GemmParams& p, int epi, int nb, hipStream_t s) {
  return launch_epi<OP_BF16, false>(p, epi, nb, s);
}

}  // namespace q3
