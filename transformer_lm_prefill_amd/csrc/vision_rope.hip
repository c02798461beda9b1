// Rotary position tables of a vision-tower patch grid and their application to q / k, for the
// bidirectional attention blocks of the vision encoders on the pages.
//
// Tables (cos and sin, fp32 [n, head_dim], patches in merge-block order: frames in order;
// within a frame merge x merge blocks row-major, each block's patches row-major):
//   layout 0 (inferencelayer 0.2.3, vision.rs, `rope_tables_2d`): half = hd/2, nf = half/2;
//     angle j < nf = row * theta^(-2j/half), angle nf + j = col * theta^(-2j/half);
//   layout 1 (cortiq-engine 0.8.51, onevision2.rs, `rope_tables`): the half angles split 4:6:6
//     (unit = half/16) between frame, row and column, axis k with n_k slots turning by
//     theta^(-i/n_k);
//   both: entry j and entry j + half hold the same angle. Angles are formed in fp64.
// Application, in place on x [n, heads, hd] (row stride in elements), fp32 arithmetic:
//   pairing 0 (vision.rs, the block's `attention`): split halves, rotate_half,
//     y_i = x_i c_i - x_{i+half} s_i,  y_{i+half} = x_{i+half} c_{i+half} + x_i s_{i+half};
//   pairing 1 (onevision2.rs, `split_rope`): adjacent lanes,
//     y_{2i} = x_{2i} c_{2i} - x_{2i+1} s_{2i},  y_{2i+1} = x_{2i+1} c_{2i+1} + x_{2i} s_{2i+1}
//     (the two lanes of a pair take their own table entries, so their angles differ).
#include "common.h"
#include "kernels.h"

namespace q3 {

// One thread per (patch, angle slot j < half).
__global__ __launch_bounds__(256) void vision_rope_tables_kernel(int layout, int t, int h, int w, int merge,
                                                                 int hd, double log2_theta, float* cosv,
                                                                 float* sinv) {
  const int half = hd / 2;
  const int64_t n = static_cast<int64_t>(t) * h * w;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= n * half) return;
  const int64_t tok = idx / half;
  const int j = static_cast<int>(idx % half);
  // patch position from its index in merge-block order
  const int hw = h * w;
  const int frame = static_cast<int>(tok / hw);
  const int within_frame = static_cast<int>(tok % hw);
  const int per_block = merge * merge;
  const int block = within_frame / per_block, within = within_frame % per_block;
  const int blocks_w = w / merge;
  const int row = (block / blocks_w) * merge + within / merge;
  const int col = (block % blocks_w) * merge + within % merge;
  double ang;
  if (layout == 0) {
    const int nf = half / 2;
    const int i = j < nf ? j : j - nf;
    const double inv = exp2(-log2_theta * (2.0 * i) / half);
    ang = (j < nf ? row : col) * inv;
  } else {
    const int unit = half / 16, nt = 4 * unit, nh = 6 * unit;
    int axis_pos, i, cnt;
    if (j < nt) {
      axis_pos = frame; i = j; cnt = nt;
    } else if (j < nt + nh) {
      axis_pos = row; i = j - nt; cnt = nh;
    } else {
      axis_pos = col; i = j - nt - nh; cnt = 6 * unit;
    }
    ang = axis_pos * exp2(-log2_theta * static_cast<double>(i) / cnt);
  }
  double sd, cd;
  sincos(ang, &sd, &cd);
  const int64_t o = tok * hd + j;
  cosv[o] = static_cast<float>(cd);
  cosv[o + half] = static_cast<float>(cd);
  sinv[o] = static_cast<float>(sd);
  sinv[o + half] = static_cast<float>(sd);
}

template <int DT>
__device__ __forceinline__ float ld(const void* x, int64_t i) {
  if (DT == DT_F32) return static_cast<const float*>(x)[i];
  const uint16_t u = static_cast<const uint16_t*>(x)[i];
  return DT == DT_BF16 ? bf2f(u) : h2f(u);
}
template <int DT>
__device__ __forceinline__ void st(void* x, int64_t i, float v) {
  if (DT == DT_F32) static_cast<float*>(x)[i] = v;
  else static_cast<uint16_t*>(x)[i] = DT == DT_BF16 ? f2bf(v) : f2h(v);
}

// One thread per (patch, head, pair): the general form, for strides or alignments the vector
// form does not take.
template <int DT, int PAIRING>
__global__ __launch_bounds__(256) void apply_rope_tables_kernel(void* x, int n, int heads, int hd,
                                                                int64_t row_stride, const float* cosv,
                                                                const float* sinv) {
  const int half = hd / 2;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t per_tok = static_cast<int64_t>(heads) * half;
  if (idx >= per_tok * n) return;
  const int64_t tok = idx / per_tok;
  const int hh = static_cast<int>((idx % per_tok) / half);
  const int i = static_cast<int>(idx % half);
  const int a = PAIRING == 0 ? i : 2 * i;          // the pair's two lanes
  const int b = PAIRING == 0 ? i + half : 2 * i + 1;
  const int64_t base = tok * row_stride + static_cast<int64_t>(hh) * hd;
  const float xa = ld<DT>(x, base + a), xb = ld<DT>(x, base + b);
  const float* c = cosv + tok * hd;
  const float* s = sinv + tok * hd;
  st<DT>(x, base + a, xa * c[a] - xb * s[a]);
  st<DT>(x, base + b, xb * c[b] + xa * s[b]);
}

// Vector form: one thread per run of 8 elements of a head row (pairing 0: pairs i .. i+7, runs
// at i and i + half; pairing 1: 4 adjacent pairs), 16-byte accesses of x (two for fp32) and of
// the tables. Needs hd % 16 == 0, a row stride that is a multiple of 8 elements and 16-byte
// aligned x and tables.
__device__ __forceinline__ void tab8(const float* t, float (&v)[8]) {
  const f32x4 p = *reinterpret_cast<const f32x4*>(t), q = *reinterpret_cast<const f32x4*>(t + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = p[e];
    v[4 + e] = q[e];
  }
}

template <int DT, int PAIRING>
__global__ __launch_bounds__(256) void apply_rope_tables8_kernel(void* x, int n, int heads, int hd,
                                                                 int64_t row_stride, const float* cosv,
                                                                 const float* sinv) {
  const int half = hd / 2;
  const int runs = PAIRING == 0 ? half / 8 : hd / 8;  // threads per head row
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t per_tok = static_cast<int64_t>(heads) * runs;
  if (idx >= per_tok * n) return;
  const int64_t tok = idx / per_tok;
  const int hh = static_cast<int>((idx % per_tok) / runs);
  const int a = 8 * static_cast<int>(idx % runs);
  const int64_t base = tok * row_stride + static_cast<int64_t>(hh) * hd;
  const float* c = cosv + tok * hd;
  const float* sn = sinv + tok * hd;
  if (PAIRING == 0) {
    const int b = a + half;
    float xa[8], xb[8], ca[8], cb[8], sa[8], sb[8], ya[8], yb[8];
    load8<DT>(x, base + a, xa);
    load8<DT>(x, base + b, xb);
    tab8(c + a, ca); tab8(c + b, cb); tab8(sn + a, sa); tab8(sn + b, sb);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ya[e] = xa[e] * ca[e] - xb[e] * sa[e];
      yb[e] = xb[e] * cb[e] + xa[e] * sb[e];
    }
    store8<DT>(x, base + a, ya);
    store8<DT>(x, base + b, yb);
  } else {
    float v[8], cc[8], ss[8], y[8];
    load8<DT>(x, base + a, v);
    tab8(c + a, cc); tab8(sn + a, ss);
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      y[e] = v[e] * cc[e] - v[e + 1] * ss[e];
      y[e + 1] = v[e + 1] * cc[e + 1] + v[e] * ss[e + 1];
    }
    store8<DT>(x, base + a, y);
  }
}

hipError_t launch_vision_rope_tables(int layout, int t, int h, int w, int merge, int hd, double log2_theta,
                                     float* cosv, float* sinv, hipStream_t s) {
  const int64_t work = static_cast<int64_t>(t) * h * w * (hd / 2);
  if (work <= 0) return hipSuccess;
  const int64_t blocks = (work + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  vision_rope_tables_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(layout, t, h, w, merge, hd, log2_theta,
                                                                          cosv, sinv);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_apply_dt(void* x, int n, int heads, int hd, int64_t rs, const float* c, const float* sn,
                                  int pairing, unsigned blocks, hipStream_t s) {
  const bool vec = hd % 16 == 0 && rs % 8 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(c) % 16 == 0 && reinterpret_cast<uintptr_t>(sn) % 16 == 0;
  if (vec) {
    const int64_t work = static_cast<int64_t>(n) * heads * (pairing == 0 ? hd / 16 : hd / 8);
    const unsigned b8 = static_cast<unsigned>((work + 255) / 256);
    if (pairing == 0) apply_rope_tables8_kernel<DT, 0><<<b8, 256, 0, s>>>(x, n, heads, hd, rs, c, sn);
    else apply_rope_tables8_kernel<DT, 1><<<b8, 256, 0, s>>>(x, n, heads, hd, rs, c, sn);
  } else if (pairing == 0) {
    apply_rope_tables_kernel<DT, 0><<<blocks, 256, 0, s>>>(x, n, heads, hd, rs, c, sn);
  } else {
    apply_rope_tables_kernel<DT, 1><<<blocks, 256, 0, s>>>(x, n, heads, hd, rs, c, sn);
  }
  return hipGetLastError();
}

hipError_t launch_apply_rope_tables(void* x, int dt, int n, int heads, int hd, int64_t row_stride,
                                    const float* cosv, const float* sinv, int pairing, hipStream_t s) {
  const int64_t work = static_cast<int64_t>(n) * heads * (hd / 2);
  if (work <= 0) return hipSuccess;
  const int64_t blocks = (work + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const unsigned nb = static_cast<unsigned>(blocks);
  if (dt == DT_F32) return launch_apply_dt<DT_F32>(x, n, heads, hd, row_stride, cosv, sinv, pairing, nb, s);
  if (dt == DT_BF16) return launch_apply_dt<DT_BF16>(x, n, heads, hd, row_stride, cosv, sinv, pairing, nb, s);
  if (dt == DT_F16) return launch_apply_dt<DT_F16>(x, n, heads, hd, row_stride, cosv, sinv, pairing, nb, s);
  return hipErrorInvalidValue;
}

}  // namespace q3
