// fp32 path: the same layer arithmetic with true single-precision FMA on the vector ALUs and
// no reduced-precision operand anywhere. A tf32-class product would move the residual by
// about 2e-4 (cortiq-engine 0.8.21, qwen3te.rs, `mm`, note on the device f32 GEMM), which is
// above the 1e-4 budget an fp32 layer is held to, so these kernels never round operands.
// They serve small fp32 layers (the correctness workload); the bf16 kernels carry the
// throughput.
#include "common.h"
#include "kernels.h"

namespace q3 {

// ------------------------------------------------------------------------------------------
// C[m, n] = sum_k A[m, k] B[n, k]  (+ R[m, n]), 64 x 64 tile, 256 threads, 4 x 4 per thread.
// DUAL: a second weight matrix B1 is multiplied alongside B0 and the store is
// silu(A B0^T) * (A B1^T) (SwiGLU gate and up).
template <bool DUAL>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const GemmF32Params p) {
  constexpr int T = 64, KT = 16;
  __shared__ float As[KT][T + 4];
  __shared__ float Bs[KT][T + 4];
  __shared__ float Us[DUAL ? KT : 1][T + 4];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m0 = blockIdx.y * T, n0 = blockIdx.x * T;
  float acc[4][4] = {}, accu[4][4] = {};
  for (int k0 = 0; k0 < p.K; k0 += KT) {
    // 64 rows x 16 k per operand: each thread loads 4 elements of each
    for (int i = threadIdx.x; i < T * KT; i += 256) {
      const int r = i / KT, kk = i % KT;
      const int m = m0 + r, n = n0 + r, k = k0 + kk;
      As[kk][r] = (m < p.M && k < p.K) ? p.A[static_cast<int64_t>(m) * p.lda + k] : 0.f;
      float bv = 0.f, uv = 0.f;
      if (n < p.N && k < p.K) {
        if (DUAL) {
          bv = p.B0[static_cast<int64_t>(n) * p.ldb + k];
          uv = p.B1[static_cast<int64_t>(n) * p.ldb + k];
        } else {
          const float* b = n < p.nseg0 ? p.B0 + static_cast<int64_t>(n) * p.ldb
                           : n < p.nseg1 ? p.B1 + static_cast<int64_t>(n - p.nseg0) * p.ldb
                                         : p.B2 + static_cast<int64_t>(n - p.nseg1) * p.ldb;
          bv = b[k];
        }
      }
      Bs[kk][r] = bv;
      if (DUAL) Us[kk][r] = uv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) {
      float a[4], b[4], u[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[kk][ty * 4 + i];
        b[i] = Bs[kk][tx * 4 + i];
        if (DUAL) u[i] = Us[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
          if (DUAL) accu[i][j] = fmaf(a[i], u[j], accu[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
      if (m < p.M && n < p.N) {
        float v;
        if (DUAL) {
          const float g = acc[i][j];
          v = g / (1.0f + expf(-g)) * accu[i][j];
        } else {
          v = acc[i][j];
          if (p.R) v += p.R[static_cast<int64_t>(m) * p.ldr + n];
        }
        p.C[static_cast<int64_t>(m) * p.ldc + n] = v;
      }
    }
}

hipError_t launch_gemm_f32(const GemmF32Params& p, bool dual, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  dim3 grid((p.N + 63) / 64, (p.M + 63) / 64), block(256);
  if (dual) gemm_f32_kernel<true><<<grid, block, 0, s>>>(p);
  else gemm_f32_kernel<false><<<grid, block, 0, s>>>(p);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Causal GQA attention, fp32: one wave per (query token, head). Keys are taken 64 at a time,
// one per lane (full dot product per lane), then an online-softmax update; the output row is
// spread over the lanes (HD/64 values each).
template <int HD>
__global__ __launch_bounds__(64) void attn_f32_kernel(const AttnF32Params p) {
  constexpr int R = HD / 64;
  __shared__ float qs[HD];
  __shared__ float ps[64];
  const int s = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int g = h / (p.nh / p.nkv);
  const float* q = p.q + static_cast<int64_t>(s) * p.q_stride + static_cast<int64_t>(h) * HD;
  for (int d = lane; d < HD; d += 64) qs[d] = q[d];
  __syncthreads();
  float m = -INFINITY, l = 0.f, o[R];
#pragma unroll
  for (int r = 0; r < R; ++r) o[r] = 0.f;
  const int last = p.causal ? s : p.S - 1;  // last key this query sees
  for (int j0 = 0; j0 <= last; j0 += 64) {
    const int j = j0 + lane;
    float z = -INFINITY;
    if (j <= last) {
      const float* k = p.k + static_cast<int64_t>(j) * p.k_stride + static_cast<int64_t>(g) * HD;
      float dot = 0.f;
      for (int d = 0; d < HD; ++d) dot = fmaf(qs[d], k[d], dot);
      z = dot * p.scale;
    }
    float mt = z;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mt = fmaxf(mt, __shfl_xor(mt, off));
    const float m_new = fmaxf(m, mt);
    const float alpha = expf(m - m_new);
    const float pj = j <= last ? expf(z - m_new) : 0.f;
    l = l * alpha + wave_sum(pj);
    m = m_new;
    __syncthreads();
    ps[lane] = pj;
    __syncthreads();
    const int nj = min(64, last + 1 - j0);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float acc = o[r] * alpha;
      for (int jj = 0; jj < nj; ++jj)
        acc = fmaf(ps[jj], p.v[static_cast<int64_t>(j0 + jj) * p.v_stride + static_cast<int64_t>(g) * HD + lane + 64 * r], acc);
      o[r] = acc;
    }
  }
  float* out = p.o + static_cast<int64_t>(s) * p.o_stride + static_cast<int64_t>(h) * HD;
#pragma unroll
  for (int r = 0; r < R; ++r) out[lane + 64 * r] = o[r] / l;
}

hipError_t launch_attention_f32(const AttnF32Params& p, int head_dim, hipStream_t s) {
  if (p.S <= 0) return hipSuccess;
  if (p.nkv <= 0 || p.nh % p.nkv != 0) return hipErrorInvalidValue;
  dim3 grid(p.S, p.nh), block(64);
  if (head_dim == 64) attn_f32_kernel<64><<<grid, block, 0, s>>>(p);
  else if (head_dim == 128) attn_f32_kernel<128><<<grid, block, 0, s>>>(p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace q3
