// MFMA product kernels for fp16 operands, bf16 weights converted on the way to the MFMA (instantiation unit).
#include "gemm_mfma.h"

namespace q3 {

hipError_t gemm_part_f16_cvt(const GemmParams& p, int epi, int nb, hipStream_t s) {
  return launch_epi<OP_F16, true>(p, epi, nb, s);
}

}  // namespace q3
