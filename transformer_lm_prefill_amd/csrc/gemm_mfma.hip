// Entry points of the 16-bit MFMA products: shape checks, tile-width choice, and dispatch to
// the instantiation units (kernel design in gemm_mfma.h).
#include "gemm_mfma.h"

namespace q3 {

int gemm_pick_nb(int M, int N, int epi) {
  if (epi == EPI_SWIGLU_16) return 4;
  // Relative per-tile efficiency of the wider tiles (operand reuse), weighed against how
  // evenly the tile count fills whole rounds of 256 CUs.
  const double rel[5] = {0, 0, 0.85, 0.95, 1.0};
  const int tiles_m = (M + kBM - 1) / kBM;
  int best = 0;
  double best_score = -1;
  for (int nb = 4; nb >= 2; --nb) {
    if (N % (64 * nb) != 0) continue;
    const int64_t tiles = static_cast<int64_t>(tiles_m) * (N / (64 * nb));
    const int64_t rounds = (tiles + 255) / 256;
    const double score = rel[nb] * static_cast<double>(tiles) / static_cast<double>(rounds * 256);
    if (score > best_score + 1e-9) {
      best_score = score;
      best = nb;
    }
  }
  return best;
}

hipError_t launch_gemm_mfma_q4(const GemmParams& p, int epi, int op, int nb, hipStream_t s) {
  if (p.M <= 0) return hipSuccess;
  if (nb == 0) nb = gemm_pick_nb(p.M, p.N, epi);
  if (nb < 2 || nb > 4 || p.N % (64 * nb) != 0 || p.K % kBK != 0 || p.K <= 0) return hipErrorInvalidValue;
  if (2 * a_rows(p) * p.lda > 0x7fffffff || p.b_tiled || !tiled_ok(p, epi)) return hipErrorInvalidValue;
  if (epi != EPI_SWIGLU_16 && (p.nseg0 % 16 != 0 || p.nseg1 % 16 != 0)) return hipErrorInvalidValue;
  return gemm_part_q4(p, epi, op, nb, s);
}

hipError_t launch_gemm_mfma(const GemmParams& p, int epi, int op, bool b_bf16, int nb, hipStream_t s) {
  if (p.M <= 0) return hipSuccess;
  if (nb == 0) nb = gemm_pick_nb(p.M, p.N, epi);
  if (nb < 2 || nb > 4 || p.N % (64 * nb) != 0 || p.K % kBK != 0 || p.K <= 0)
    return hipErrorInvalidValue;
  // A tile offsets are 32-bit element offsets
  if (a_rows(p) * p.lda >= (int64_t(1) << 32)) return hipErrorInvalidValue;
  if (!tiled_ok(p, epi) || (p.b_tiled && (b_bf16 || op != OP_F16))) return hipErrorInvalidValue;
  if (op == OP_BF16) {
    if (!b_bf16) return hipErrorInvalidValue;  // bf16 products take bf16 weights
    return gemm_part_bf16(p, epi, nb, s);
  }
  if (op == OP_F16) {
    return b_bf16 ? gemm_part_f16_cvt(p, epi, nb, s) : gemm_part_f16(p, epi, nb, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace q3
