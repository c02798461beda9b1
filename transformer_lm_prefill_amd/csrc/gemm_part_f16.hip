// MFMA product kernels for fp16 operands and weights (row-major or tiled) (instantiation unit).
#include "gemm_mfma.h"

namespace q3 {

hipError_t gemm_part_f16(const GemmParams& p, int epi, int nb, hipStream_t s) {
  return launch_epi<OP_F16, false>(p, epi, nb, s);
}

}  // namespace q3
