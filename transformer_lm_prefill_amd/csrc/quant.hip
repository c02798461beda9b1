// Weight-only quantized projections: GGML Q4_0 blocks (hf2q 0.1.1, qwen3vl_text/forward.rs,
// the dense FFN step: the converted checkpoints' projections are Q4_0) and int8 rows with a
// per-row scale (cortiq-engine 0.8.21, qwen3te.rs, `q8_exact_matmat`).
//
// Q4_0: 32 consecutive weights of a row per 18-byte block, a binary16 scale d then 16 bytes of
// codes; byte j holds weight j's code in its low nibble and weight j + 16's in its high nibble;
// weight = d * (code - 8). Rows are K/32 blocks back to back (18-byte blocks, so a block is only
// 2-byte aligned; two blocks, 36 bytes, start 4-byte aligned when K % 64 == 0 and the matrix
// is 4-byte aligned).
// q8 rows: weight[o, j] = row_scale[o] * q[o, j], q int8 [rows, K].
//
// Prefill (M = S rows of activations) is MFMA-bound: the weights are expanded once per call
// into the operand format (d * (code - 8) is exact in fp32 and rounded once to fp16/bf16;
// row_scale * q likewise) and the dense GEMM runs on them.
// Decode (one activation row) is HBM-bound: the matrix-vector kernels read the quantized bytes
// directly (0.5625 B per weight for Q4_0, 1 B for q8 rows):
//   sum_j w_j x_j = d * (sum_j code_j x_j - 8 * sum_j x_j)   per Q4_0 block, x rounded to
//     binary16, each code pair masked in place into exact binary16 subnormals and multiplied by
//     v_dot2 with fp32 sums (about 1.1 instructions per weight);
//   sum_j w_j x_j = rs * (sum_j (q_j + 128) x_j - 128 * sum_j x_j)   per q8 row, x in fp32,
//     one byte-to-float conversion and one FMA per weight;
// the block sums of x are shared by the four rows a wave computes.
#include "common.h"
#include "kernels.h"

namespace q3 {

typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));

// ---- expansion to the operand format -----------------------------------------------------------
// Workgroup = 256 consecutive blocks: their 4608 bytes come in with coalesced dword loads into
// LDS, thread t expands block t into an LDS tile of 16-bit weights (rows padded against bank
// conflicts), and the 16 KB of weights leave with coalesced 16-byte stores. (Blocks are 18 bytes, so a thread reading its own block from
// global memory would issue nine 2-byte loads at an 18-byte lane stride.)
constexpr int kDqBlocks = 256;

template <int ODT>
__global__ __launch_bounds__(256) void dequant_q4_0_kernel(const uint8_t* blocks, int64_t nblocks, void* out) {
  // tile rows padded from 64 to 80 bytes: 8 consecutive threads' 16-byte stores then start 20
  // words apart, on distinct LDS banks
  constexpr int kRow = 40;  // halfwords per padded tile row
  __shared__ __align__(16) uint32_t raw[kDqBlocks * 18 / 4];
  __shared__ __align__(16) uint16_t tile[kDqBlocks * kRow];
  const int tid = threadIdx.x;
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) * kDqBlocks;
  const int nb = static_cast<int>(min<int64_t>(kDqBlocks, nblocks - b0));
  const uint32_t* src = reinterpret_cast<const uint32_t*>(blocks + b0 * 18);   // 4-byte aligned: b0 % 2 == 0
  for (int i = tid; i < nb * 18 / 4; i += 256) raw[i] = src[i];
  if (nb % 2 != 0 && tid == 0) {   // an odd last block ends on a halfword
    const uint16_t* h = reinterpret_cast<const uint16_t*>(blocks + b0 * 18);
    reinterpret_cast<uint16_t*>(raw)[nb * 9 - 1] = h[nb * 9 - 1];
  }
  __syncthreads();
  if (tid < nb) {
    const uint16_t* h = reinterpret_cast<const uint16_t*>(raw) + tid * 9;
    const float d = h2f(h[0]);
    float lo[16], hi[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t two = h[1 + i];   // code bytes 2i, 2i + 1
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t byte = (two >> (8 * k)) & 0xFF;
        lo[2 * i + k] = d * static_cast<float>(static_cast<int>(byte & 0xF) - 8);
        hi[2 * i + k] = d * static_cast<float>(static_cast<int>(byte >> 4) - 8);
      }
    }
    uint16_t* t = tile + tid * kRow;
    store8<ODT>(t, 0, *reinterpret_cast<const float(*)[8]>(lo));
    store8<ODT>(t, 8, *reinterpret_cast<const float(*)[8]>(lo + 8));
    store8<ODT>(t, 16, *reinterpret_cast<const float(*)[8]>(hi));
    store8<ODT>(t, 24, *reinterpret_cast<const float(*)[8]>(hi + 8));
  }
  __syncthreads();
  u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + b0 * 32);
  const u32x4* from = reinterpret_cast<const u32x4*>(tile);
  for (int i = tid; i < nb * 4; i += 256) dst[i] = from[(i >> 2) * (kRow / 8) + (i & 3)];
}

// Thread = 16 consecutive weights of one row (cols % 16 == 0).
template <int ODT>
__global__ __launch_bounds__(256) void dequant_q8_row_kernel(const int8_t* q, const float* rs, int64_t rows,
                                                             int cols, void* out) {
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int per_row = cols / 16;
  if (c >= rows * per_row) return;
  const int64_t r = c / per_row;
  const float s = rs[r];
  const u32x4 w = *reinterpret_cast<const u32x4*>(q + c * 16);
  float v[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int8_t code = static_cast<int8_t>((w[e >> 2] >> (8 * (e & 3))) & 0xFF);
    v[e] = s * static_cast<float>(code);
  }
  store8<ODT>(out, c * 16, *reinterpret_cast<const float(*)[8]>(v));
  store8<ODT>(out, c * 16 + 8, *reinterpret_cast<const float(*)[8]>(v + 8));
}

hipError_t launch_dequant(int fmt, const void* data, const float* row_scale, int64_t rows, int cols, int out_dt,
                          void* out, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (out_dt != DT_F16 && out_dt != DT_BF16) return hipErrorInvalidValue;
  if (fmt == WF_Q4_0) {
    if (cols % 32 != 0) return hipErrorInvalidValue;
    const int64_t nb = rows * (cols / 32);
    const unsigned grid = static_cast<unsigned>((nb + kDqBlocks - 1) / kDqBlocks);
    const uint8_t* b = static_cast<const uint8_t*>(data);
    if (out_dt == DT_F16) dequant_q4_0_kernel<DT_F16><<<grid, 256, 0, s>>>(b, nb, out);
    else dequant_q4_0_kernel<DT_BF16><<<grid, 256, 0, s>>>(b, nb, out);
  } else if (fmt == WF_Q8_ROW) {
    if (cols % 16 != 0) return hipErrorInvalidValue;
    const int64_t nc = rows * (cols / 16);
    const unsigned grid = static_cast<unsigned>((nc + 255) / 256);
    const int8_t* q = static_cast<const int8_t*>(data);
    if (out_dt == DT_F16) dequant_q8_row_kernel<DT_F16><<<grid, 256, 0, s>>>(q, row_scale, rows, cols, out);
    else dequant_q8_row_kernel<DT_BF16><<<grid, 256, 0, s>>>(q, row_scale, rows, cols, out);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---- matrix-vector products on the quantized bytes (decode) ----------------------------------
constexpr int kQvRows = 4;   // output rows per wave

typedef _Float16 h2x __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2h(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2x, a), __builtin_bit_cast(h2x, b), acc, false);
}

// The activations of one Q4_0 block as 16 binary16 pairs in the order the code pairs below
// take them: for code word i (codes of weights 4i .. 4i+3 in its low nibbles, 16+4i .. 16+4i+3
// in its high nibbles), pairs (x[4i], x[4i+2]), (x[16+4i], x[16+4i+2]), (x[4i+1], x[4i+3]),
// (x[16+4i+1], x[16+4i+3]).
__device__ __forceinline__ void q4_pack_x(const float* x, uint32_t (&xp)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int a = 4 * i;
    xp[4 * i + 0] = Fmt<OP_F16>::pack2(x[a], x[a + 2]);
    xp[4 * i + 1] = Fmt<OP_F16>::pack2(x[16 + a], x[16 + a + 2]);
    xp[4 * i + 2] = Fmt<OP_F16>::pack2(x[a + 1], x[a + 3]);
    xp[4 * i + 3] = Fmt<OP_F16>::pack2(x[16 + a + 1], x[16 + a + 3]);
  }
}

// sum_j code_j * x_j over one block, two codes at a time: a 4-bit code masked in place inside a
// 16-bit half is the binary16 subnormal code * 2^-24 (bits 0-3) or code * 2^-20 (bits 4-7), so
// one AND makes a pair of exact operands for v_dot2 (fp32 sums; binary16 subnormals are kept,
// not flushed); the two scales are undone at the end. q holds the 16 code bytes as 4 words.
__device__ __forceinline__ float q4_codes_dot(const uint32_t (&q)[4], const uint32_t (&xp)[16]) {
  float lo = 0.f, hi = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t q8 = q[i] >> 8;
    lo = dot2h(q[i] & 0x000F000Fu, xp[4 * i + 0], lo);   // codes 4i, 4i+2 (low nibbles of bytes 0, 2)
    hi = dot2h(q[i] & 0x00F000F0u, xp[4 * i + 1], hi);   // codes 16+4i, 16+4i+2 (high nibbles)
    lo = dot2h(q8 & 0x000F000Fu, xp[4 * i + 2], lo);     // codes 4i+1, 4i+3 (bytes 1, 3)
    hi = dot2h(q8 & 0x00F000F0u, xp[4 * i + 3], hi);     // codes 16+4i+1, 16+4i+3
  }
  return fmaf(lo, 16777216.f, hi * 1048576.f);
}

// Lane = one pair of consecutive blocks (64 weights, 36 bytes, 4-byte aligned) of each row.
template <int EPI>
__global__ __launch_bounds__(256) void gemv_q4_0_kernel(GemvParams p) {
  constexpr int NR = EPI == GV_SWIGLU ? 2 * kQvRows : kQvRows;
  const int lane = threadIdx.x & 63;
  const int r0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * kQvRows;
  if (r0 >= p.rows) return;
  const int64_t row_bytes = static_cast<int64_t>(p.K / 32) * 18;
  const uint8_t* rowp[NR];
#pragma unroll
  for (int j = 0; j < kQvRows; ++j) {
    const int r = min(r0 + j, p.rows - 1);  // rows past the end repeat the last (never stored)
    if (EPI == GV_SWIGLU) {
      rowp[j] = static_cast<const uint8_t*>(p.W0) + r * row_bytes;
      rowp[kQvRows + j] = static_cast<const uint8_t*>(p.W1) + r * row_bytes;
    } else {
      const void* W = r < p.nseg0 ? p.W0 : r < p.nseg1 ? p.W1 : p.W2;
      const int rr = r < p.nseg0 ? r : r < p.nseg1 ? r - p.nseg0 : r - p.nseg1;
      rowp[j] = static_cast<const uint8_t*>(W) + rr * row_bytes;
    }
  }
  float acc[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) acc[j] = 0.f;
  const int npairs = p.K / 64;
  for (int pp = lane; pp < npairs; pp += 64) {
    uint32_t w[NR][9];
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const uint8_t* src = rowp[j] + pp * 36;
      const u32x4a4 a = *reinterpret_cast<const u32x4a4*>(src);
      const u32x4a4 b = *reinterpret_cast<const u32x4a4*>(src + 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w[j][e] = a[e];
        w[j][4 + e] = b[e];
      }
      w[j][8] = *reinterpret_cast<const uint32_t*>(src + 32);
    }
    float x[64];
#pragma unroll
    for (int i = 0; i < 8; ++i) load8<DT_F32>(p.x, pp * 64 + 8 * i, *reinterpret_cast<float(*)[8]>(x + 8 * i));
    uint32_t xa[16], xb[16];
    q4_pack_x(x, xa);
    q4_pack_x(x + 32, xb);
    // the code offset 8 goes out against the sums of the same binary16 activations
    float sxa = 0.f, sxb = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      sxa = Fmt<OP_F16>::sum2(xa[e], sxa);
      sxb = Fmt<OP_F16>::sum2(xb[e], sxb);
    }
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const float da = h2f(static_cast<uint16_t>(w[j][0] & 0xFFFF));
      const float db = h2f(static_cast<uint16_t>(w[j][4] >> 16));
      uint32_t qa[4], qb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qa[i] = __builtin_amdgcn_alignbyte(w[j][i + 1], w[j][i], 2);  // bytes 2 .. 17 of block a
        qb[i] = w[j][5 + i];                                           // bytes 20 .. 35: codes of block b
      }
      acc[j] = fmaf(da, fmaf(-8.f, sxa, q4_codes_dot(qa, xa)), acc[j]);
      acc[j] = fmaf(db, fmaf(-8.f, sxb, q4_codes_dot(qb, xb)), acc[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < NR; ++j) acc[j] = wave_sum(acc[j]);
  if (lane < kQvRows && r0 + lane < p.rows) {
    float v = acc[0];
#pragma unroll
    for (int j = 1; j < kQvRows; ++j) v = lane == j ? acc[j] : v;
    const int r = r0 + lane;
    if (EPI == GV_SWIGLU) {
      float u = acc[kQvRows];
#pragma unroll
      for (int j = 1; j < kQvRows; ++j) u = lane == j ? acc[kQvRows + j] : u;
      v = v / (1.f + __expf(-v)) * u;
    } else if (EPI == GV_RESID) {
      v += p.R[r];
    }
    p.y[r] = v;
  }
}

// Lane = 16 consecutive int8 weights of each row per step; U steps loaded together. Codes are
// offset by 128 (flipping the sign bit) so each byte converts as an unsigned value.
template <int EPI>
__global__ __launch_bounds__(256) void gemv_q8_row_kernel(GemvParams p, const float* rs0, const float* rs1,
                                                          const float* rs2) {
  constexpr int NR = EPI == GV_SWIGLU ? 2 * kQvRows : kQvRows;
  constexpr int U = 16 / NR;
  const int lane = threadIdx.x & 63;
  const int r0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * kQvRows;
  if (r0 >= p.rows) return;
  const int8_t* rowp[NR];
  float scale[NR];
#pragma unroll
  for (int j = 0; j < kQvRows; ++j) {
    const int r = min(r0 + j, p.rows - 1);
    if (EPI == GV_SWIGLU) {
      rowp[j] = static_cast<const int8_t*>(p.W0) + static_cast<int64_t>(r) * p.K;
      rowp[kQvRows + j] = static_cast<const int8_t*>(p.W1) + static_cast<int64_t>(r) * p.K;
      scale[j] = rs0[r];
      scale[kQvRows + j] = rs1[r];
    } else {
      const int seg = r < p.nseg0 ? 0 : r < p.nseg1 ? 1 : 2;
      const void* W = seg == 0 ? p.W0 : seg == 1 ? p.W1 : p.W2;
      const float* rs = seg == 0 ? rs0 : seg == 1 ? rs1 : rs2;
      const int rr = seg == 0 ? r : seg == 1 ? r - p.nseg0 : r - p.nseg1;
      rowp[j] = static_cast<const int8_t*>(W) + static_cast<int64_t>(rr) * p.K;
      scale[j] = rs[rr];
    }
  }
  float acc[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) acc[j] = 0.f;
  for (int i0 = lane * 16; i0 < p.K; i0 += 64 * 16 * U) {
    u32x4 w[U][NR];
    float x[U][16];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = min(i0 + u * 1024, p.K - 16);   // steps past the end repeat the last, weighted 0
#pragma unroll
      for (int j = 0; j < NR; ++j) w[u][j] = *reinterpret_cast<const u32x4*>(rowp[j] + i);
      load8<DT_F32>(p.x, i, *reinterpret_cast<float(*)[8]>(x[u]));
      load8<DT_F32>(p.x, i + 8, *reinterpret_cast<float(*)[8]>(x[u] + 8));
      if (i0 + u * 1024 >= p.K) {
#pragma unroll
        for (int e = 0; e < 16; ++e) x[u][e] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float sx = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) sx += x[u][e];
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const uint32_t word = w[u][j][e >> 2] ^ 0x80808080u;
          s = fmaf(static_cast<float>((word >> (8 * (e & 3))) & 0xFF), x[u][e], s);
        }
        acc[j] += fmaf(-128.f, sx, s);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NR; ++j) acc[j] = wave_sum(acc[j]) * scale[j];
  if (lane < kQvRows && r0 + lane < p.rows) {
    float v = acc[0];
#pragma unroll
    for (int j = 1; j < kQvRows; ++j) v = lane == j ? acc[j] : v;
    const int r = r0 + lane;
    if (EPI == GV_SWIGLU) {
      float u = acc[kQvRows];
#pragma unroll
      for (int j = 1; j < kQvRows; ++j) u = lane == j ? acc[kQvRows + j] : u;
      v = v / (1.f + __expf(-v)) * u;
    } else if (EPI == GV_RESID) {
      v += p.R[r];
    }
    p.y[r] = v;
  }
}

hipError_t launch_gemv_quant(const GemvParams& p, int epi, int fmt, const float* rs0, const float* rs1,
                             const float* rs2, hipStream_t s) {
  if (p.norm_w != nullptr) return hipErrorInvalidValue;  // the folded RMSNorm is dense-only
  if (p.rows <= 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>((p.rows + 4 * kQvRows - 1) / (4 * kQvRows));
  if (fmt == WF_Q4_0) {
    if (p.K % 64 != 0) return hipErrorInvalidValue;
    if (epi == GV_STORE) gemv_q4_0_kernel<GV_STORE><<<blocks, 256, 0, s>>>(p);
    else if (epi == GV_RESID) gemv_q4_0_kernel<GV_RESID><<<blocks, 256, 0, s>>>(p);
    else if (epi == GV_SWIGLU) gemv_q4_0_kernel<GV_SWIGLU><<<blocks, 256, 0, s>>>(p);
    else return hipErrorInvalidValue;
  } else if (fmt == WF_Q8_ROW) {
    if (p.K % 16 != 0) return hipErrorInvalidValue;
    if (epi == GV_STORE) gemv_q8_row_kernel<GV_STORE><<<blocks, 256, 0, s>>>(p, rs0, rs1, rs2);
    else if (epi == GV_RESID) gemv_q8_row_kernel<GV_RESID><<<blocks, 256, 0, s>>>(p, rs0, rs1, rs2);
    else if (epi == GV_SWIGLU) gemv_q8_row_kernel<GV_SWIGLU><<<blocks, 256, 0, s>>>(p, rs0, rs1, rs2);
    else return hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace q3
