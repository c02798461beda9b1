// Host-side launchers of the gfx950 kernels. Each returns the HIP error of its launch.
// Shapes are validated by the C-ABI layer (capi.hip) before any launcher is called; the
// launchers only re-check the preconditions that the kernels' index arithmetic relies on.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q3 {

// Element storage types; the values match qwen3_dtype in the public header.
enum DType : int { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

// Tiled 16-bit matrix layout: a [R, C] matrix (R a multiple of 16, C of 32) as 16-row x
// 32-column tiles of 1 KiB each, row-major inside a tile, tiles ordered by row group and then
// by column: element (r, c) sits at ((r / 16) * (C / 32) + c / 32) * 512 + (r % 16) * 32 + c % 32.
// One 32-wide K step of 16 operand rows is then a single contiguous 1 KiB block.
__host__ __device__ constexpr int64_t tiled_index(int64_t r, int64_t c, int64_t C) {
  return ((r >> 4) * (C >> 5) + (c >> 5)) * 512 + (r & 15) * 32 + (c & 31);
}
// src [rows, cols] row-major (src_dt) -> dst fp16 in the tiled layout, rounded to nearest even.
hipError_t launch_tile_matrix(const void* src, int src_dt, int rows, int cols, uint16_t* dst, hipStream_t s);

// ---- RMSNorm (a row per workgroup) -------------------------------------------------------
// y[r] = x[r] * rsqrt(mean(x[r]^2) + eps) * w; x f32 [rows, H]; w and y of the given types;
// y_tiled: y (16-bit) in the tiled layout over ceil(rows / 16) * 16 rows (padding rows untouched).
hipError_t launch_rmsnorm(const float* x, const void* w, int w_dt, void* y, int y_dt, int rows,
                          int hidden, float eps, hipStream_t s, bool y_tiled = false);

// ---- DeepStack rows add -------------------------------------------------------------------
// y[rows[i], :] += ds[i, :] for i < n; rows is a device copy of a host-checked list (strictly
// increasing, inside [0, S)). y f32 [S, H]; ds [n, H] of ds_dt.
hipError_t launch_deepstack_add(float* y, const int32_t* rows, const void* ds, int ds_dt, int n,
                                int S, int hidden, hipStream_t s);

// ---- whole-model steps around the layers (model_head.hip) ---------------------------------
// x[s, :] = table[tokens[s], :] as fp32 (tokens are device int32, already in range).
hipError_t launch_embed_gather(const int32_t* tokens, const void* table, int dt, float* x, int S, int hidden,
                               hipStream_t s);
// x[:] = table[token, :] as fp32, token already range-checked on the host.
hipError_t launch_embed_row(const void* table, int dt, int64_t token, float* x, int hidden, hipStream_t s);
// y[r] = sum_k W[r, k] x[k], W [rows, hidden] of dt, x and y fp32 (hidden % 8 == 0).
hipError_t launch_gemv_rows(const void* W, int dt, const float* x, float* y, int rows, int hidden, hipStream_t s);

// ---- vision-tower rope tables and their application (vision_rope.hip) ----------------------
// cos / sin fp32 [t*h*w, hd] of a merge-block-ordered patch grid; layout 0: 2-D row | col,
// layout 1: 3-axis 4:6:6.
hipError_t launch_vision_rope_tables(int layout, int t, int h, int w, int merge, int hd, double log2_theta,
                                     float* cosv, float* sinv, hipStream_t s);
// In place on x [n, heads, hd] (row stride in elements) of dt; pairing 0: split halves,
// 1: adjacent lanes.
hipError_t launch_apply_rope_tables(void* x, int dt, int n, int heads, int hd, int64_t row_stride,
                                    const float* cosv, const float* sinv, int pairing, hipStream_t s);

// ---- KV cache and one decode step (decode.hip) ------------------------------------------------
// Caches: K and V each [nkv][capacity][hd] of the cache type.
struct KvWriteParams {
  const void* k; const void* v;   // token t, kv head g at k + t*k_stride + g*hd (same for v)
  int64_t k_stride, v_stride;     // elements between consecutive tokens
  int n, nkv, hd;                 // tokens to write, hd % 8 == 0
  void* kc; void* vc;
  int64_t capacity;               // rows per head in the caches
  int row0;                       // token t goes to row row0 + t (row0 + n <= capacity)
};
hipError_t launch_kv_cache_write(const KvWriteParams& p, int src_dt, int cache_dt, hipStream_t s);

struct DecodeAttnParams {
  const float* q;                 // [nh, hd] fp32: one query row per head
  const void* kc; const void* vc; // caches, rows 0..len-1 live
  int64_t capacity;
  int len, nh, nkv;               // nh / nkv <= 16
  float scale_log2;               // softmax scale * log2(e)
  int tiles_per_split, nsplit;    // decode_tiles_per_split / decode_num_splits(len, nkv)
  float* part_o;                  // [nh, nsplit, hd] fp32 scratch
  float* part_ml;                 // [nh, nsplit, 2] fp32 scratch
};
int decode_tiles_per_split(int len, int nkv);
int decode_num_splits(int len, int nkv);
int decode_max_splits(int len, int nkv);   // >= decode_num_splits(l, nkv) for every l <= len
// out [nh, hd] fp32 = softmax(scale q k^T) v over the len cached keys of each head's group.
hipError_t launch_decode_attention(const DecodeAttnParams& p, int hd, int cache_dt, float* out, hipStream_t s);

// y[r] = epilogue(sum_k W_r[k] x[k]) for r < rows; x, y, R fp32; W of wdt [*, K], K % 8 == 0.
enum GemvEpilogue { GV_STORE = 0, GV_RESID = 1, GV_SWIGLU = 2 };
struct GemvParams {
  // GV_STORE / GV_RESID: row r < nseg0 is W0 row r, r < nseg1 is W1 row r - nseg0, else W2 row
  // r - nseg1. GV_SWIGLU: W0 = gate, W1 = up, both [rows, K]; y[r] = silu(g_r) * u_r.
  const void* W0; const void* W1; const void* W2;
  int nseg0, nseg1;
  const float* x;
  float* y;
  const float* R;                 // GV_RESID: y[r] = R[r] + product (R may alias y)
  int rows, K;
  // Optional RMSNorm of x folded in (dense weights only): with norm_w set the product uses
  // x * norm_w / sqrt(mean(x^2) + eps) in place of x (norm_w [K] of norm_dt).
  const void* norm_w = nullptr;
  int norm_dt = 0;
  float eps = 0.f;
  int w_tiled = 0;     // dense 16-bit weights in the tiled layout (rows and K as given)
};
hipError_t launch_gemv(const GemvParams& p, int epi, int wdt, hipStream_t s);

// ---- weight-only quantized projections (quant.hip) -------------------------------------------
// Formats; the values match qwen3_wformat in the public header.
enum WFormat : int { WF_DENSE = 0, WF_Q4_0 = 1, WF_Q8_ROW = 2 };
// out [rows, cols] of out_dt (f16 or bf16) = the dequantized weights (one rounding each).
// Q4_0: data = rows * cols / 32 blocks of 18 bytes (2-byte aligned), cols % 32 == 0.
// Q8 rows: data int8 [rows, cols] (16-byte aligned), row_scale fp32 [rows], cols % 16 == 0.
hipError_t launch_dequant(int fmt, const void* data, const float* row_scale, int64_t rows, int cols, int out_dt,
                          void* out, hipStream_t s);
// launch_gemv on quantized W0..W2 (one format for all); rs0..rs2: the row scales of W0..W2
// (q8 rows only). Q4_0 needs K % 64 == 0 and 4-byte aligned matrices; q8 rows K % 16 == 0
// and 16-byte aligned matrices.
hipError_t launch_gemv_quant(const GemvParams& p, int epi, int fmt, const float* rs0, const float* rs1,
                             const float* rs2, hipStream_t s);

// ---- per-head RMSNorm + interleaved MRoPE, in place ---------------------------------------
struct RopeParams {
  void* q;            // token t, head h at q + t*q_stride + h*hd
  void* k;            // token t, kv head h at k + t*k_stride + h*hd
  int64_t q_stride, k_stride;  // elements between consecutive tokens
  int S, nh, nkv;
  const void* q_norm;
  const void* k_norm;
  int norm_dt;         // storage type of q_norm / k_norm
  const int32_t* pos;  // [3, S]
  float eps;
  double log2_theta;
  int sec_h, sec_w;    // interleave bounds: h pairs i%3==1 && i<3*sec_h, w pairs i%3==2 && i<3*sec_w
  // Optional KV-cache append: with kc set, token t's rotated k rows and its v rows (v + t*v_stride
  // + h*hd) are also written, in cache_dt, to row row0 + t of the head-major caches kc / vc
  // ([nkv][capacity][hd]).
  void* kc = nullptr;
  void* vc = nullptr;
  const void* v = nullptr;
  int64_t v_stride = 0;
  int64_t capacity = 0;
  int row0 = 0;
  int cache_dt = 0;
};
hipError_t launch_qk_norm_mrope(const RopeParams& p, int head_dim, int data_dt, hipStream_t s);

// ---- 16-bit MFMA GEMM:  C[m, n] = sum_k A[m, k] * B[n, k]  --------------------------------
enum GemmEpilogue { EPI_STORE_16 = 0, EPI_STORE_F32 = 1, EPI_SWIGLU_16 = 2 };
enum Op16Host : int { OPH_BF16 = 0, OPH_F16 = 1 };
struct GemmParams {
  const uint16_t* A;   // [M, K] 16-bit, row stride lda
  int64_t lda;
  // B rows come from up to three row-major [*, K] matrices (stride ldb): output column n < nseg0
  // reads B0 row n, n < nseg1 reads B1 row n - nseg0, otherwise B2 row n - nseg1. For
  // EPI_SWIGLU_16, B0 is W_gate and B1 is W_up, both [F, K].
  const uint16_t* B0;
  const uint16_t* B1;
  const uint16_t* B2;
  int nseg0, nseg1;
  int64_t ldb;
  void* C;             // [M, N] (EPI_SWIGLU_16: [M, N/2]) with row stride ldc
  int64_t ldc;
  const float* R;      // EPI_STORE_F32 only: residual added to the product, or nullptr
  int64_t ldr;
  int M, N, K;         // N: product columns (for SwiGLU, 2F: gate and up together)
  // Tiled operands (16-bit, the tiled layout; ld must equal the row length): a_tiled: A over
  // ceil(M / 16) * 16 rows, lda == K (rows past M are read and their products discarded);
  // b_tiled: every B segment, ldb == K; c_tiled: the EPI_SWIGLU_16 output, ldc == N / 2.
  int a_tiled = 0, b_tiled = 0, c_tiled = 0;
  // Exact scales (powers of two; 1 leaves the result as is): EPI_SWIGLU_16 stores
  // act_scale * silu(g) * u; EPI_STORE_F32 and EPI_STORE_16 store out_scale * (A B^T) [+ R].
  float act_scale = 1.f, out_scale = 1.f;
};
// op: OPH_BF16 or OPH_F16, the format of A, of the MFMA and of 16-bit outputs. b_bf16: B is
// stored as bf16 (converted to fp16 on the way to LDS when op is fp16); otherwise B is in op's
// format. nb: 32-column MFMA blocks per wave along N (tile width 64*nb); 0 picks one.
hipError_t launch_gemm_mfma(const GemmParams& p, int epi, int op, bool b_bf16, int nb, hipStream_t s);
// The same product with B0..B2 holding Q4_0 blocks (18 bytes per 32 weights of a row, rows back
// to back, 4-byte aligned; ldb unused) decoded in the weight-tile path into op's format. Needs
// K % 64 == 0, the A operand's byte extent within 32-bit offsets and segment bounds (QKV) at
// multiples of 16 rows; returns hipErrorInvalidValue otherwise.
hipError_t launch_gemm_mfma_q4(const GemmParams& p, int epi, int op, int nb, hipStream_t s);
int gemm_pick_nb(int M, int N, int epi);

// ---- 16-bit GQA flash attention (causal or bidirectional), head_dim 64 or 128 ---------------
struct AttnParams {
  const uint16_t* q; const uint16_t* k; const uint16_t* v; uint16_t* o;
  int64_t q_stride, k_stride, v_stride, o_stride;  // elements between consecutive tokens
  int S, nh, nkv;
  float scale_log2;    // softmax scale * log2(e)
  int head_dim;        // 64 or 128
  int causal;          // 1: key j <= query s; 0: every key (bidirectional)
  int o_tiled = 0;     // o in the tiled layout over o_stride columns (rows padded to 16)
};
hipError_t launch_attention_mfma(const AttnParams& p, int op, hipStream_t s);

// ---- fp32 path -----------------------------------------------------------------------------
struct GemmF32Params {
  const float* A; int64_t lda;
  const float* B0; const float* B1; const float* B2; int nseg0, nseg1; int64_t ldb;
  float* C; int64_t ldc;
  const float* R; int64_t ldr;
  int M, N, K;
};
// dual = false: C = A B^T (+ R); dual = true: C[M, N] = silu(A B0^T) * (A B1^T), N = F.
hipError_t launch_gemm_f32(const GemmF32Params& p, bool dual, hipStream_t s);

struct AttnF32Params {
  const float* q; const float* k; const float* v; float* o;
  int64_t q_stride, k_stride, v_stride, o_stride;
  int S, nh, nkv;
  float scale;
  int causal;          // 1: key j <= query s; 0: every key
};
hipError_t launch_attention_f32(const AttnF32Params& p, int head_dim, hipStream_t s);

}  // namespace q3
