// MFMA product kernels for Q4_0 weights decoded in the weight-tile path (instantiation unit).
#include "gemm_mfma.h"

namespace q3 {

hipError_t gemm_part_q4(const GemmParams& p, int epi, int op, int nb, hipStream_t s) {
  if (op == OP_F16) {
    switch (epi) {
      case EPI_STORE_16: return launch_q4_nb<EPI_STORE_16, OP_F16>(p, nb, s);
      case EPI_STORE_F32: return launch_q4_nb<EPI_STORE_F32, OP_F16>(p, nb, s);
      case EPI_SWIGLU_16: return launch_q4_nb<EPI_SWIGLU_16, OP_F16>(p, nb, s);
    }
  } else if (op == OP_BF16) {
    switch (epi) {
      case EPI_STORE_16: return launch_q4_nb<EPI_STORE_16, OP_BF16>(p, nb, s);
      case EPI_STORE_F32: return launch_q4_nb<EPI_STORE_F32, OP_BF16>(p, nb, s);
      case EPI_SWIGLU_16: return launch_q4_nb<EPI_SWIGLU_16, OP_BF16>(p, nb, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace q3
