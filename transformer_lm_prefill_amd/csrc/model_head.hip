// The steps on either side of the decoder layers in a whole-model text prefill (hf2q 0.1.1,
// qwen3vl_text/forward.rs, `forward_text_prefill_logits_last`): the token embedding lookup
// that starts the residual stream, and the LM head product of the last position's
// normalized hidden state.
//
// Both are HBM-bound streams. The lookup reads S rows of the [vocab, H] table and writes the
// fp32 residual stream; the head reads the whole [vocab, H] matrix once (1.24 GB at a 151936
// vocabulary and H = 4096) for one output row, so it is a matrix-vector product: every wave
// streams four weight rows at once with 16-byte loads, the hidden vector sits in registers,
// and a wave reduction finishes each logit.
#include "common.h"
#include "kernels.h"

namespace q3 {

// x[s, :] = table[tokens[s], :] as fp32; one workgroup per token (tokens already range-checked).
template <int DT>
__global__ __launch_bounds__(256) void embed_gather_kernel(const int32_t* tokens, const void* table,
                                                           float* x, int hidden) {
  const int s = blockIdx.x;
  const int64_t row = static_cast<int64_t>(tokens[s]) * hidden;
  float* out = x + static_cast<int64_t>(s) * hidden;
  for (int i = threadIdx.x * 8; i < hidden; i += 256 * 8) {
    float v[8];
    load8<DT>(table, row + i, v);
    *reinterpret_cast<f32x4*>(out + i) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(out + i + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
}

// y[r] = sum_k W[r, k] x[k] for r < rows; W [rows, hidden] of DT, x, y fp32. A wave owns 4
// consecutive rows; lane l covers the 8-element chunks l, l + 64, ... of each row.
constexpr int kGemvRows = 4;
template <int DT>
__global__ __launch_bounds__(256) void gemv_rows_kernel(const void* W, const float* x, float* y, int rows,
                                                        int hidden) {
  const int lane = threadIdx.x & 63;
  const int r0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * kGemvRows;
  if (r0 >= rows) return;
  float acc[kGemvRows] = {0.f, 0.f, 0.f, 0.f};
  for (int i = lane * 8; i < hidden; i += 64 * 8) {
    const f32x4 xa = *reinterpret_cast<const f32x4*>(x + i);
    const f32x4 xb = *reinterpret_cast<const f32x4*>(x + i + 4);
    const float xv[8] = {xa[0], xa[1], xa[2], xa[3], xb[0], xb[1], xb[2], xb[3]};
#pragma unroll
    for (int j = 0; j < kGemvRows; ++j) {
      const int r = min(r0 + j, rows - 1);  // rows past the end repeat the last (never stored)
      float w[8];
      load8<DT>(W, static_cast<int64_t>(r) * hidden + i, w);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j] = fmaf(w[e], xv[e], acc[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < kGemvRows; ++j) {
    const float v = wave_sum(acc[j]);
    if (lane == 0 && r0 + j < rows) y[r0 + j] = v;
  }
}

hipError_t launch_embed_gather(const int32_t* tokens, const void* table, int dt, float* x, int S, int hidden,
                               hipStream_t s) {
  if (S <= 0) return hipSuccess;
  if (hidden % 8 != 0) return hipErrorInvalidValue;
  if (dt == DT_BF16) embed_gather_kernel<DT_BF16><<<S, 256, 0, s>>>(tokens, table, x, hidden);
  else if (dt == DT_F16) embed_gather_kernel<DT_F16><<<S, 256, 0, s>>>(tokens, table, x, hidden);
  else if (dt == DT_F32) embed_gather_kernel<DT_F32><<<S, 256, 0, s>>>(tokens, table, x, hidden);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// x[:] = one table row as fp32 (the row chosen on the host).
template <int DT>
__global__ __launch_bounds__(256) void embed_row_kernel(const void* row, float* x, int hidden) {
  for (int i = threadIdx.x * 8; i < hidden; i += 256 * 8) {
    float v[8];
    load8<DT>(row, i, v);
    *reinterpret_cast<f32x4*>(x + i) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(x + i + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
}

hipError_t launch_embed_row(const void* table, int dt, int64_t token, float* x, int hidden, hipStream_t s) {
  if (hidden % 8 != 0) return hipErrorInvalidValue;
  const int64_t off = token * hidden;
  if (dt == DT_BF16) embed_row_kernel<DT_BF16><<<1, 256, 0, s>>>(static_cast<const uint16_t*>(table) + off, x, hidden);
  else if (dt == DT_F16) embed_row_kernel<DT_F16><<<1, 256, 0, s>>>(static_cast<const uint16_t*>(table) + off, x, hidden);
  else if (dt == DT_F32) embed_row_kernel<DT_F32><<<1, 256, 0, s>>>(static_cast<const float*>(table) + off, x, hidden);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_gemv_rows(const void* W, int dt, const float* x, float* y, int rows, int hidden, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (hidden % 8 != 0) return hipErrorInvalidValue;
  const int blocks = (rows + 4 * kGemvRows - 1) / (4 * kGemvRows);
  if (dt == DT_BF16) gemv_rows_kernel<DT_BF16><<<blocks, 256, 0, s>>>(W, x, y, rows, hidden);
  else if (dt == DT_F16) gemv_rows_kernel<DT_F16><<<blocks, 256, 0, s>>>(W, x, y, rows, hidden);
  else if (dt == DT_F32) gemv_rows_kernel<DT_F32><<<blocks, 256, 0, s>>>(W, x, y, rows, hidden);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace q3
